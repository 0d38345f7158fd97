"""The C ABI without a GPU: the library loads, exports every declared entry
point, and rejects bad arguments with the documented codes before any HIP call."""

import ctypes
import os
import re

import pytest

import dit_circular_local_amd as ca

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include",
                      "clear_attn.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(clear_\w+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = ca.lib()
    names = _declared()
    assert names == sorted(ca.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_version():
    assert ca.version() == 10500  # 1.5.0: allocation-free forward (clear_attn_fwd_noalloc)


# fake, aligned, non-overlapping device addresses: validation must fail before use
Q, K, V, O = 0x10000000, 0x20000000, 0x30000000, 0x40000000
ok = dict(B=1, H=2, d=128, n_text=8, gh=4, gw=4, radius=2)


def _fwd(q=Q, k=K, v=V, o=O, **kw):
    a = dict(ok)
    a.update(kw)
    return ca.lib().clear_attn_fwd(q, k, v, o, a["B"], a["H"], a["d"], a["n_text"], a["gh"],
                                   a["gw"], a["radius"], None)


def _fwd_ex(dtype=0, r2=4, lse=None, splits=0, q=Q, k=K, v=V, o=O, **kw):
    a = dict(ok)
    a.update(kw)
    opts = ca._Opts(dtype, r2, lse, splits)
    return ca.lib().clear_attn_fwd_ex(q, k, v, o, a["B"], a["H"], a["d"], a["n_text"], a["gh"],
                                      a["gw"], ctypes.byref(opts), None)


@pytest.mark.parametrize("kw,frag", [
    (dict(d=96), "d must be"), (dict(d=0), "d must be"), (dict(radius=-1), "radius"),
    (dict(B=0), "B and H"), (dict(H=-3), "B and H"), (dict(n_text=-1), "n_text"),
    (dict(gh=0), "grid sides"), (dict(gw=8193), "grid sides"),
    (dict(q=0), "NULL"), (dict(o=0), "NULL"), (dict(q=Q + 8), "aligned"),
    (dict(o=Q + 4096), "overlap"), (dict(o=V - 16), "overlap"),
    (dict(n_text=2 ** 31 - 4096 - 16), "sequence too long"),
])
def test_fwd_rejects_bad_arguments(kw, frag):
    assert _fwd(**kw) == ca.CLEAR_EINVAL
    assert frag in ca.last_error()


@pytest.mark.parametrize("kw,frag", [
    (dict(dtype=2), "dtype"), (dict(r2=-2), "r2_max"), (dict(splits=65), "text_splits"),
    (dict(splits=-1), "text_splits"), (dict(n_text=0, r2=-1), "empty"), (dict(lse=6), "lse_out"),
])
def test_fwd_ex_rejects_bad_arguments(kw, frag):
    assert _fwd_ex(**kw) == ca.CLEAR_EINVAL
    assert frag in ca.last_error()


def test_tile_map_validation_and_size_query():
    L = ca.lib()
    n = ctypes.c_size_t()
    bad = [(0, 4, 1, 16, 8, 4, 8, 4, 8), (8, 8, -2, 16, 8, 4, 8, 4, 8), (8, 8, 4, 16, 8, 3, 8, 4, 8),
           (8, 8, 4, 16, 8, 2, 4, 4, 8), (8, 8, 4, 16, 8, 4, 8, 0, 8), (8, 8, 4, 16, 8, 4, 8, 4, 2000)]
    for args in bad:
        assert L.clear_tile_map_size(*args, ctypes.byref(n)) == ca.CLEAR_EINVAL, args
    assert L.clear_tile_map_size(8, 8, 4, 16, 8, 2, 4, 4, 8, ctypes.byref(n)) == ca.CLEAR_EINVAL
    assert "at most 8" in ca.last_error()
    # capacity 0 reports the size with ENOMEM and writes nothing
    assert L.clear_tile_map_build(64, 64, 64, 16, 8, 4, 8, 4, 8, None, None, None, 0,
                                  ctypes.byref(n)) == ca.CLEAR_ENOMEM
    assert n.value == ca.tile_map_size(64, 64, 64) > 0
    # the device builder checks the capacity on the host before launching anything
    assert L.clear_tile_map_build_device(64, 64, 64, 16, 8, 4, 8, 4, 8, None, None, None, 0,
                                         ctypes.byref(n), None) == ca.CLEAR_ENOMEM


def test_python_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 1, 8 + 16, 64)
    with pytest.raises(ValueError):
        ca.fwd(q, q, q, 8, 4, 4, radius=2)
    with pytest.raises(ValueError):
        ca.fwd(q, q, q, 8, 4, 4)


DO, LSE, DQ, DK, DV = 0x50000000, 0x60000000, 0x70000000, 0x80000000, 0x90000000


def _bwd(dtype=0, r2=4, lse_out=None, splits=0, window=0, q=Q, k=K, v=V, o=O, do=DO, lse=LSE, dq=DQ,
         dk=DK, dv=DV, **kw):
    a = dict(ok)
    a.update(kw)
    opts = ca._Opts(dtype, r2, lse_out, splits, window)
    return ca.lib().clear_attn_bwd(q, k, v, o, do, lse, dq, dk, dv, a["B"], a["H"], a["d"], a["n_text"],
                                   a["gh"], a["gw"], ctypes.byref(opts), None)


@pytest.mark.parametrize("kw,frag", [
    (dict(d=96), "d must be"), (dict(B=0), "B and H"), (dict(gw=0), "grid sides"),
    (dict(lse=0), "NULL"), (dict(dv=0), "NULL"), (dict(do=0), "NULL"),
    (dict(dq=Q), "overlap"), (dict(dk=DQ + 4096), "overlap"), (dict(dv=LSE), "overlap"),
    (dict(dq=DO - 16), "overlap"), (dict(lse=LSE + 2), "lse must be"), (dict(dk=DK + 8), "aligned"),
    (dict(lse_out=0x1000), "lse_out"), (dict(splits=65), "text_splits"), (dict(window=3), "window"),
    (dict(dtype=7), "dtype"), (dict(r2=-3), "r2_max"), (dict(n_text=0, r2=-1), "empty"),
    (dict(n_text=2 ** 31 - 4096 - 16), "sequence too long"),
])
def test_bwd_rejects_bad_arguments(kw, frag):
    assert _bwd(**kw) == ca.CLEAR_EINVAL
    assert frag in ca.last_error()


# ---------------------------------------------------------------- binding checks
# The binding must refuse buffers the C ABI cannot check (a host tensor, a
# tensor on another device, a too-small element type) before any launch.  These
# run without a GPU: a stand-in tensor reports CUDA placement and raises if the
# binding ever asks for its address.

class _FakeGpuTensor:
    def __init__(self, shape, dtype, device="cuda:0", is_cuda=True, contiguous=True):
        import torch
        self.shape = tuple(shape)
        self.dtype = dtype
        self.device = torch.device(device)
        self.is_cuda = is_cuda
        self._contig = contiguous

    def dim(self):
        return len(self.shape)

    def is_contiguous(self):
        return self._contig

    def data_ptr(self):
        raise AssertionError("the binding reached a launch with a bad buffer")

    def element_size(self):
        return 2


def _qkv(dtype=None, shape=(1, 2, 8 + 16, 64)):
    import torch
    dtype = dtype or torch.bfloat16
    return tuple(_FakeGpuTensor(shape, dtype) for _ in range(3))


def test_binding_fwd_rejects_bad_out_before_launch():
    import torch
    q, k, v = _qkv()
    bad = [
        _FakeGpuTensor(q.shape, torch.bfloat16, device="cpu", is_cuda=False),   # host tensor
        _FakeGpuTensor(q.shape, torch.bfloat16, device="cuda:1"),               # other device
        _FakeGpuTensor(q.shape, torch.float16),                                 # wrong dtype
        _FakeGpuTensor((1, 2, 8 + 16, 32), torch.bfloat16),                     # wrong shape
        _FakeGpuTensor(q.shape, torch.bfloat16, contiguous=False),
    ]
    for out in bad:
        with pytest.raises((ValueError, TypeError)):
            ca.fwd(q, k, v, 8, 4, 4, radius=2, out=out)
    k2 = _FakeGpuTensor(q.shape, torch.bfloat16, device="cuda:1")
    with pytest.raises(ValueError):
        ca.fwd(q, k2, v, 8, 4, 4, radius=2, out=_FakeGpuTensor(q.shape, torch.bfloat16))


def test_binding_bwd_rejects_bad_buffers_before_launch():
    import torch
    q, k, v = _qkv()
    B, H, N, d = q.shape
    good = dict(out=_FakeGpuTensor(q.shape, torch.bfloat16), dout=_FakeGpuTensor(q.shape, torch.bfloat16),
                lse=_FakeGpuTensor((B, H, N), torch.float32))
    grads = tuple(_FakeGpuTensor(q.shape, torch.bfloat16) for _ in range(3))
    cases = [
        dict(good, lse=_FakeGpuTensor((B, H, N), torch.bfloat16)),
        dict(good, lse=_FakeGpuTensor((B, H, N), torch.float32, device="cpu", is_cuda=False)),
        dict(good, dout=_FakeGpuTensor(q.shape, torch.float32)),
        dict(good, out=_FakeGpuTensor(q.shape, torch.bfloat16, device="cuda:3")),
    ]
    for c in cases:
        with pytest.raises((ValueError, TypeError)):
            ca.bwd(q, k, v, c["out"], c["dout"], c["lse"], 8, 4, 4, radius=2, grads=grads)
    for i in range(3):
        g = list(grads)
        g[i] = _FakeGpuTensor(q.shape, torch.bfloat16, device="cpu", is_cuda=False)
        with pytest.raises(ValueError):
            ca.bwd(q, k, v, good["out"], good["dout"], good["lse"], 8, 4, 4, radius=2, grads=tuple(g))


def test_binding_strip_and_merge_reject_bad_partials_before_launch():
    import torch
    q, k, v = _qkv()
    B, H, N, d = q.shape
    out = _FakeGpuTensor(q.shape, torch.bfloat16)
    po = _FakeGpuTensor((B * H, 8, d), torch.float32)
    pml = _FakeGpuTensor((B * H, 8, 2), torch.float32)
    for bad_o, bad_ml in [(_FakeGpuTensor((B * H, 8, d), torch.bfloat16), pml),
                          (po, _FakeGpuTensor((B * H, 8, 2), torch.float16)),
                          (_FakeGpuTensor((B * H, 8, d), torch.float32, device="cpu", is_cuda=False), pml)]:
        with pytest.raises((ValueError, TypeError)):
            ca.fwd_strip(q, k, v, 8, 4, 4, 0, 2, out, bad_o, bad_ml, radius=2)
    with pytest.raises((ValueError, TypeError)):
        ca.fwd_strip(q, k, v, 8, 4, 4, 0, 2, _FakeGpuTensor(q.shape, torch.float32), po, pml, radius=2)
    P = 3
    po3 = _FakeGpuTensor((P, B * H, 8, d), torch.float32)
    pml3 = _FakeGpuTensor((P, B * H, 8, 2), torch.float32)
    merge_cases = [
        (_FakeGpuTensor(q.shape, torch.float16), po3, pml3),          # fp16 out: 4-byte writes would overrun
        (out, _FakeGpuTensor((P, B * H, 8, d), torch.bfloat16), pml3),
        (out, po3, _FakeGpuTensor((P, B * H, 8, 2), torch.float32, device="cuda:2")),
        (out, _FakeGpuTensor((P, B * H, 8, d), torch.float32, device="cpu", is_cuda=False), pml3),
        (_FakeGpuTensor(q.shape, torch.bfloat16, device="cpu", is_cuda=False), po3, pml3),
    ]
    for o, a, b in merge_cases:
        with pytest.raises((ValueError, TypeError)):
            ca.text_merge(a, b, o, 8, 4, 4)


def test_descriptor_builder_checks_before_launch():
    L = ca.lib()
    n = ctypes.c_size_t()
    # capacity too small: size reported, nothing launched
    assert L.clear_tile_map_descriptors(0, 64, 64, 64, None, None, None, None, 0, ctypes.byref(n),
                                        None) == ca.CLEAR_ENOMEM
    assert n.value == ca.tile_map_size(64, 64, 64)
    assert L.clear_tile_map_descriptors(2, 64, 64, 64, None, None, None, None, 0, ctypes.byref(n),
                                        None) == ca.CLEAR_EINVAL
    assert L.clear_tile_map_descriptors(0, 0, 64, 64, None, None, None, None, 0, ctypes.byref(n),
                                        None) == ca.CLEAR_EINVAL
    assert L.clear_tile_map_descriptors(0, 64, 64, 64, 0x1000, 0x2000, 0x3000, None, n.value,
                                        ctypes.byref(n), None) == ca.CLEAR_EINVAL
    assert "NULL" in ca.last_error()


def _noalloc(splits=0, q=Q, k=K, v=V, o=O, **kw):
    a = dict(ok)
    a.update(kw)
    opts = ca._Opts(0, a.pop("r2", 4), None, splits, 0)
    return ca.lib().clear_attn_fwd_noalloc(q, k, v, o, a["B"], a["H"], a["d"], a["n_text"], a["gh"], a["gw"],
                                           ctypes.byref(opts), None)


def test_noalloc_forward_checks_before_any_hip_call():
    """The allocation-free forward shares the forward's argument checks, and
    refuses, before touching the device, a tile map that does not fit its fixed
    scratch (a 4096 x 4096 grid at r = 32 needs some 440 MB) and explicit text
    splits whose partials do not fit beside the map."""
    for kw, frag in [(dict(d=96), "d must be"), (dict(q=0), "NULL"), (dict(o=Q + 16), "overlap"),
                     (dict(gh=0), "grid sides")]:
        assert _noalloc(**kw) == ca.CLEAR_EINVAL
        assert frag in ca.last_error()
    big = 0x4000000000  # far apart: 4096^2 tokens of d 128 bf16 are 4.3 GB per tensor
    rc = _noalloc(q=big, k=2 * big, v=3 * big, o=4 * big, B=1, H=1, n_text=512, gh=4096, gw=4096, r2=1024)
    assert rc == ca.CLEAR_ENOMEM and "no-alloc scratch" in ca.last_error()
    rc = _noalloc(splits=64, B=1, H=24, n_text=512, gh=64, gw=64, r2=256)
    assert rc == ca.CLEAR_ENOMEM and "text splits" in ca.last_error()


def test_plain_c_caller(tmp_path):
    """The header compiles as C99 with warnings as errors, and a C program
    linked against the library gets the documented results from calls that
    need no GPU."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no C compiler")
    here = os.path.dirname(os.path.abspath(__file__))
    libdir = os.path.dirname(ca.LIB_PATH)
    exe = str(tmp_path / "abi_check")
    subprocess.run([cc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-pedantic",
                    "-I", os.path.dirname(HEADER), os.path.join(here, "c_abi", "abi_check.c"),
                    "-L", libdir, "-lclear_attn", f"-Wl,-rpath,{libdir}", "-o", exe], check=True)
    r = subprocess.run([exe], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "tile map entries 2" in r.stdout and r.stdout.rstrip().endswith("ok")
