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
    assert ca.version() == 10300  # 1.3.0: gradients (clear_attn_bwd)


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
