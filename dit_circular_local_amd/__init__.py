"""CLEAR circular-window attention for AMD Instinct MI355X (gfx950).

Thin ctypes binding of ``libclear_attn.so`` (C ABI in ``include/clear_attn.h``).
This module only marshals arguments: every step of the attention runs in the
library's HIP kernels.  PyTorch supplies device memory and the stream.  If the
library has not been built, every call raises (there is no fallback).

    from dit_circular_local_amd import fwd
    out = fwd(q, k, v, n_text=512, grid_h=64, grid_w=64, radius=16)
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

import numpy as np

__all__ = [
    "ClearError", "fwd", "fwd_noalloc", "bwd", "fwd_strip", "text_merge", "strip_rows", "tile_map_size", "tile_map_build", "tile_map_build_device",
    "tile_map_descriptors", "release_cache", "last_error", "version", "lib", "EXPORTS",
    "CLEAR_OK", "CLEAR_EINVAL", "CLEAR_ENOMEM", "CLEAR_EHIP", "CLEAR_ENOTSUP",
    "CLEAR_BF16", "CLEAR_FP32", "NOALLOC_SCRATCH_BYTES", "CLEAR_MERGE_EXACT", "CLEAR_MERGE_PATCH_AVERAGE", "CLEAR_WINDOW_CIRCLE", "CLEAR_WINDOW_SQUARE", "WINDOWS", "TILE_H", "TILE_W", "SUB_H", "SUB_W", "KEY_H", "KEY_W", "CHUNK",
    "MAX_GRID",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libclear_attn.so")

CLEAR_OK, CLEAR_EINVAL, CLEAR_ENOMEM, CLEAR_EHIP, CLEAR_ENOTSUP = 0, -22, -12, -5, -95
CLEAR_BF16, CLEAR_FP32 = 0, 1
CLEAR_WINDOW_CIRCLE, CLEAR_WINDOW_SQUARE = 0, 1
CLEAR_MERGE_EXACT, CLEAR_MERGE_PATCH_AVERAGE = 0, 1
WINDOWS = {"circle": CLEAR_WINDOW_CIRCLE, "square": CLEAR_WINDOW_SQUARE}
TILE_H, TILE_W, SUB_H, SUB_W, KEY_H, KEY_W, CHUNK = 16, 8, 4, 8, 4, 8, 32
MAX_GRID = 8192
NOALLOC_SCRATCH_BYTES = 64 << 20

# every entry point declared in include/clear_attn.h
EXPORTS = (
    "clear_attn_fwd", "clear_attn_fwd_ex", "clear_tile_map_size", "clear_tile_map_build",
    "clear_tile_map_build_device", "clear_tile_map_size_ex", "clear_tile_map_build_ex",
    "clear_tile_map_build_device_ex", "clear_attn_fwd_strip", "clear_text_merge", "clear_attn_bwd",
    "clear_tile_map_descriptors", "clear_attn_fwd_noalloc", "clear_last_error",
    "clear_release_cache", "clear_version",
)


class ClearError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class _Opts(ctypes.Structure):
    _fields_ = [("dtype", ctypes.c_int), ("r2_max", ctypes.c_int),
                ("lse_out", ctypes.c_void_p), ("text_splits", ctypes.c_int), ("window", ctypes.c_int)]


_lib = None


def lib():
    """The loaded library (raises if it was not built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                           "(or python dit_circular_local_amd/build.py)")
    L = ctypes.CDLL(LIB_PATH)
    i, p, sz, szp = ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)
    L.clear_attn_fwd.argtypes = [p, p, p, p, i, i, i, i, i, i, i, p]
    L.clear_attn_fwd.restype = i
    L.clear_attn_fwd_ex.argtypes = [p, p, p, p, i, i, i, i, i, i, ctypes.POINTER(_Opts), p]
    L.clear_attn_fwd_ex.restype = i
    L.clear_tile_map_size.argtypes = [i, i, i, i, i, i, i, i, i, szp]
    L.clear_tile_map_size.restype = i
    L.clear_tile_map_build.argtypes = [i, i, i, i, i, i, i, i, i, p, p, p, sz, szp]
    L.clear_tile_map_build.restype = i
    L.clear_tile_map_build_device.argtypes = [i, i, i, i, i, i, i, i, i, p, p, p, sz, szp, p]
    L.clear_tile_map_build_device.restype = i
    L.clear_tile_map_size_ex.argtypes = [i] + L.clear_tile_map_size.argtypes
    L.clear_tile_map_size_ex.restype = i
    L.clear_tile_map_build_ex.argtypes = [i] + L.clear_tile_map_build.argtypes
    L.clear_tile_map_build_ex.restype = i
    L.clear_tile_map_build_device_ex.argtypes = [i] + L.clear_tile_map_build_device.argtypes
    L.clear_tile_map_build_device_ex.restype = i
    L.clear_attn_fwd_noalloc.argtypes = [p, p, p, p, i, i, i, i, i, i, ctypes.POINTER(_Opts), p]
    L.clear_attn_fwd_noalloc.restype = i
    L.clear_tile_map_descriptors.argtypes = [i, i, i, i, p, p, p, p, sz, szp, p]
    L.clear_tile_map_descriptors.restype = i
    L.clear_attn_fwd_strip.argtypes = [p, p, p, p, i, i, i, i, i, i, ctypes.POINTER(_Opts), i, i, i, p, p, p]
    L.clear_attn_fwd_strip.restype = i
    L.clear_text_merge.argtypes = [p, p, i, i, p, p, i, i, i, i, i, i, i, p]
    L.clear_text_merge.restype = i
    L.clear_attn_bwd.argtypes = [p, p, p, p, p, p, p, p, p, i, i, i, i, i, i, ctypes.POINTER(_Opts), p]
    L.clear_attn_bwd.restype = i
    L.clear_last_error.argtypes = []
    L.clear_last_error.restype = ctypes.c_char_p
    L.clear_release_cache.argtypes = []
    L.clear_release_cache.restype = None
    L.clear_version.argtypes = []
    L.clear_version.restype = i
    _lib = L
    return L


def last_error() -> str:
    return lib().clear_last_error().decode()


def _check(rc: int):
    if rc != CLEAR_OK:
        raise ClearError(rc, last_error())


def version() -> int:
    return lib().clear_version()


def release_cache() -> None:
    lib().clear_release_cache()


def _stream_of(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _window_code(window: str) -> int:
    if window not in WINDOWS:
        raise ValueError(f"window must be one of {sorted(WINDOWS)} (got {window!r})")
    return WINDOWS[window]


def _expect(t, name: str, device, dtype, shape) -> None:
    """Raise unless ``t`` is a contiguous GPU tensor on ``device`` with the given
    dtype and shape.  Every buffer the library writes or reads goes through this
    before any launch: the C ABI sees only addresses and cannot tell a host
    pointer, a tensor on another device or a too-small element type from a good
    one."""
    if not getattr(t, "is_cuda", False) or t.device != device:
        raise ValueError(f"{name} must be a GPU tensor on {device} (got {getattr(t, 'device', type(t))})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)} (got {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def fwd(q, k, v, n_text: int, grid_h: int, grid_w: int, radius: Optional[int] = None,
        r2: Optional[int] = None, out=None, return_lse: bool = False, text_splits: int = 0,
        use_ex: Optional[bool] = None, window: str = "circle"):
    """CLEAR attention forward on torch tensors [B, H, N, d] (bf16 or fp32, on the GPU).

    Give either ``radius`` (r2 = radius^2, the "<=" reading) or ``r2`` directly
    (e.g. radius^2 - 1 for the strict "<" reading, -1 for no image keys).
    ``window="square"`` selects the square-window variant (max(dy^2, dx^2) <= r2).
    Returns ``out`` or ``(out, lse)``.
    """
    import torch

    dtype = _check_qkv(q, k, v)
    B, H, N, d = q.shape
    if N != n_text + grid_h * grid_w:
        raise ValueError(f"N = {N} != n_text + grid_h * grid_w = {n_text + grid_h * grid_w}")
    if (radius is None) == (r2 is None):
        raise ValueError("give exactly one of radius and r2")
    if out is None:
        out = torch.empty_like(q)
    else:
        _expect(out, "out", q.device, q.dtype, q.shape)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device) if return_lse else None
    stream = _stream_of(q)
    L = lib()
    wcode = _window_code(window)
    if use_ex is None:
        use_ex = not (dtype == CLEAR_BF16 and r2 is None and not return_lse and text_splits == 0
                      and wcode == CLEAR_WINDOW_CIRCLE)
    if not use_ex and wcode != CLEAR_WINDOW_CIRCLE:
        raise ValueError("the square window needs the _ex entry point")
    if not use_ex:
        rc = L.clear_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              B, H, d, n_text, grid_h, grid_w, int(radius), stream)
    else:
        if r2 is None:
            if radius < 0:
                raise ValueError("radius must be >= 0")
            r2 = min(int(radius) * int(radius), 2 ** 31 - 1)
        opts = _Opts(dtype, int(r2), lse.data_ptr() if lse is not None else None, int(text_splits), wcode)
        rc = L.clear_attn_fwd_ex(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 B, H, d, n_text, grid_h, grid_w, ctypes.byref(opts), stream)
    _check(rc)
    return (out, lse) if return_lse else out


def fwd_noalloc(q, k, v, n_text: int, grid_h: int, grid_w: int, radius: Optional[int] = None,
                r2: Optional[int] = None, out=None, lse=None, text_splits: int = 0, window: str = "circle"):
    """The forward through clear_attn_fwd_noalloc: the library allocates nothing
    (its tile map and text-row partials live in a fixed per-GPU scratch; see
    include/clear_attn.h).  ``out`` (and ``lse`` [B, H, N] float32, if wanted)
    are the caller's; when ``out`` is None it is allocated here by torch,
    before the call.  Returns ``out``."""
    import torch

    dtype = _check_qkv(q, k, v)
    B, H, N, d = q.shape
    if N != n_text + grid_h * grid_w:
        raise ValueError(f"N = {N} != n_text + grid_h * grid_w = {n_text + grid_h * grid_w}")
    if (radius is None) == (r2 is None):
        raise ValueError("give exactly one of radius and r2")
    if r2 is None:
        if radius < 0:
            raise ValueError("radius must be >= 0")
        r2 = min(int(radius) * int(radius), 2 ** 31 - 1)
    if out is None:
        out = torch.empty_like(q)
    else:
        _expect(out, "out", q.device, q.dtype, q.shape)
    if lse is not None:
        _expect(lse, "lse", q.device, torch.float32, (B, H, N))
    opts = _Opts(dtype, int(r2), lse.data_ptr() if lse is not None else None, int(text_splits),
                 _window_code(window))
    _check(lib().clear_attn_fwd_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, d,
                                        n_text, grid_h, grid_w, ctypes.byref(opts), _stream_of(q)))
    return out


def _check_qkv(q, k, v):
    import torch

    if q.dtype != k.dtype or q.dtype != v.dtype:
        raise TypeError("q, k, v must share a dtype")
    if q.dtype == torch.bfloat16:
        dtype = CLEAR_BF16
    elif q.dtype == torch.float32:
        dtype = CLEAR_FP32
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    if q.dim() != 4 or k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must all be [B, H, N, d]")
    if not (q.is_cuda and k.is_cuda and v.is_cuda):
        raise ValueError("q, k, v must be GPU tensors")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k, v must be on one device")
    if not (q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous")
    return dtype


def bwd(q, k, v, out, dout, lse, n_text: int, grid_h: int, grid_w: int, radius: Optional[int] = None,
        r2: Optional[int] = None, text_splits: int = 0, window: str = "circle", grads=None):
    """Gradients (dq, dk, dv) of the CLEAR attention layer for upstream gradient
    ``dout``, given the forward's inputs, its output ``out`` and its ``lse``
    (``fwd(..., return_lse=True)``).  Same options as ``fwd``; ``grads`` may
    pass preallocated (dq, dk, dv).  See clear_attn_bwd in include/clear_attn.h."""
    import torch

    dtype = _check_qkv(q, k, v)
    B, H, N, d = q.shape
    if N != n_text + grid_h * grid_w:
        raise ValueError(f"N = {N} != n_text + grid_h * grid_w = {n_text + grid_h * grid_w}")
    _expect(out, "out", q.device, q.dtype, q.shape)
    _expect(dout, "dout", q.device, q.dtype, q.shape)
    _expect(lse, "lse", q.device, torch.float32, (B, H, N))
    if (radius is None) == (r2 is None):
        raise ValueError("give exactly one of radius and r2")
    if r2 is None:
        if radius < 0:
            raise ValueError("radius must be >= 0")
        r2 = min(int(radius) * int(radius), 2 ** 31 - 1)
    if grads is None:
        grads = tuple(torch.empty_like(q) for _ in range(3))
    if len(grads) != 3:
        raise ValueError("grads must be (dq, dk, dv)")
    for name, t in zip(("dq", "dk", "dv"), grads):
        _expect(t, name, q.device, q.dtype, q.shape)
    dq, dk, dv = grads
    opts = _Opts(dtype, int(r2), None, int(text_splits), _window_code(window))
    _check(lib().clear_attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                                lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, d, n_text,
                                grid_h, grid_w, ctypes.byref(opts), _stream_of(q)))
    return dq, dk, dv


def strip_rows(grid_h: int, strips: int):
    """Row ranges of `strips` horizontal strips of equal height (differing by at
    most one row): strip p covers rows p*grid_h//strips .. (p+1)*grid_h//strips - 1."""
    if strips < 1 or strips > grid_h:
        raise ValueError("need 1 <= strips <= grid_h")
    return [(p * grid_h // strips, (p + 1) * grid_h // strips) for p in range(strips)]


def fwd_strip(q, k, v, n_text: int, grid_h: int, grid_w: int, row_begin: int, row_end: int,
              out, part_o, part_ml, radius: Optional[int] = None, r2: Optional[int] = None,
              with_text_keys: bool = False, window: str = "circle"):
    """One strip (image rows [row_begin, row_end)) of a patch-parallel layer:
    writes those rows of ``out`` and the text-row partial into ``part_o``
    [B*H, n_text, d] / ``part_ml`` [B*H, n_text, 2] (float32 GPU tensors or
    views).  See clear_attn_fwd_strip in include/clear_attn.h."""
    dtype = _check_qkv(q, k, v)
    B, H, N, d = q.shape
    if N != n_text + grid_h * grid_w:
        raise ValueError("N != n_text + grid_h * grid_w")
    if (radius is None) == (r2 is None):
        raise ValueError("give exactly one of radius and r2")
    if r2 is None:
        r2 = min(int(radius) * int(radius), 2 ** 31 - 1)
    import torch

    _expect(out, "out", q.device, q.dtype, q.shape)
    if n_text:
        _expect(part_o, "part_o", q.device, torch.float32, (B * H, n_text, d))
        _expect(part_ml, "part_ml", q.device, torch.float32, (B * H, n_text, 2))
    opts = _Opts(dtype, int(r2), None, 0, _window_code(window))
    _check(lib().clear_attn_fwd_strip(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, d,
                                      n_text, grid_h, grid_w, ctypes.byref(opts), row_begin, row_end,
                                      int(bool(with_text_keys)), part_o.data_ptr() if n_text else None,
                                      part_ml.data_ptr() if n_text else None, _stream_of(q)))
    return out


def text_merge(part_o, part_ml, out, n_text: int, grid_h: int, grid_w: int, mode: str = "exact",
               return_lse: bool = False):
    """Text rows of ``out`` [B, H, N, d] from stacked partials part_o
    [P, B*H, n_text, d] / part_ml [P, B*H, n_text, 2]; mode "exact" (log-sum-exp)
    or "patch_average" (the Eq. 7 text rows)."""
    import torch

    modes = {"exact": CLEAR_MERGE_EXACT, "patch_average": CLEAR_MERGE_PATCH_AVERAGE}
    if mode not in modes:
        raise ValueError(f"mode must be one of {sorted(modes)}")
    if out.dim() != 4:
        raise ValueError("out must be [B, H, N, d]")
    B, H, N, d = out.shape
    if N != n_text + grid_h * grid_w:
        raise ValueError(f"N = {N} != n_text + grid_h * grid_w = {n_text + grid_h * grid_w}")
    if out.dtype == torch.bfloat16:
        dtype = CLEAR_BF16
    elif out.dtype == torch.float32:
        dtype = CLEAR_FP32
    else:
        raise TypeError(f"out must be bfloat16 or float32 (got {out.dtype})")
    _expect(out, "out", out.device, out.dtype, out.shape)
    if part_o.dim() != 4:
        raise ValueError("part_o must be [P, B*H, n_text, d]")
    P = part_o.shape[0]
    _expect(part_o, "part_o", out.device, torch.float32, (P, B * H, n_text, d))
    _expect(part_ml, "part_ml", out.device, torch.float32, (P, B * H, n_text, 2))
    lse = torch.empty((B, H, N), dtype=torch.float32, device=out.device) if return_lse else None
    _check(lib().clear_text_merge(part_o.data_ptr(), part_ml.data_ptr(), P, modes[mode], out.data_ptr(),
                                  lse.data_ptr() if lse is not None else None, B, H, d, n_text, grid_h,
                                  grid_w, dtype, _stream_of(out)))
    return (out, lse) if return_lse else out


def tile_map_size(grid_h, grid_w, r2, tile_h=TILE_H, tile_w=TILE_W, sub_h=SUB_H, sub_w=SUB_W,
                  key_h=KEY_H, key_w=KEY_W, window: str = "circle"):
    n = ctypes.c_size_t()
    _check(lib().clear_tile_map_size_ex(_window_code(window), grid_h, grid_w, r2, tile_h, tile_w, sub_h,
                                        sub_w, key_h, key_w, ctypes.byref(n)))
    return n.value


def _ntiles(grid_h, grid_w, tile_h, tile_w):
    return (-(-grid_h // tile_h)) * (-(-grid_w // tile_w))


def tile_map_build(grid_h, grid_w, r2, tile_h=TILE_H, tile_w=TILE_W, sub_h=SUB_H, sub_w=SUB_W,
                   key_h=KEY_H, key_w=KEY_W, window: str = "circle"):
    """Host-built tile map as numpy arrays (layout in include/clear_attn.h)."""
    L = lib()
    n = tile_map_size(grid_h, grid_w, r2, tile_h, tile_w, sub_h, sub_w, key_h, key_w, window)
    nt = _ntiles(grid_h, grid_w, tile_h, tile_w)
    off = np.zeros(nt + 1, np.uint32)
    kt = np.zeros(max(n, 1), np.uint32)
    fl = np.zeros(max(n, 1), np.uint16)
    got = ctypes.c_size_t()
    _check(L.clear_tile_map_build_ex(_window_code(window), grid_h, grid_w, r2, tile_h, tile_w, sub_h,
                                     sub_w, key_h, key_w, off.ctypes.data, kt.ctypes.data,
                                     fl.ctypes.data, n, ctypes.byref(got)))
    return {"offsets": off, "key_tiles": kt[:n], "flags": fl[:n]}


def tile_map_build_device(grid_h, grid_w, r2, tile_h=TILE_H, tile_w=TILE_W, sub_h=SUB_H,
                          sub_w=SUB_W, key_h=KEY_H, key_w=KEY_W, device="cuda", window: str = "circle"):
    """Device-built tile map; returns numpy copies of the device arrays."""
    import torch

    L = lib()
    n = tile_map_size(grid_h, grid_w, r2, tile_h, tile_w, sub_h, sub_w, key_h, key_w, window)
    nt = _ntiles(grid_h, grid_w, tile_h, tile_w)
    off = torch.zeros(nt + 1, dtype=torch.int32, device=device)
    kt = torch.zeros(max(n, 1), dtype=torch.int32, device=device)
    fl = torch.zeros(max(n, 1), dtype=torch.int16, device=device)
    got = ctypes.c_size_t()
    _check(L.clear_tile_map_build_device_ex(_window_code(window), grid_h, grid_w, r2, tile_h, tile_w,
                                            sub_h, sub_w, key_h, key_w, off.data_ptr(), kt.data_ptr(),
                                            fl.data_ptr(), n, ctypes.byref(got), _stream_of(off)))
    torch.cuda.current_stream(off.device).synchronize()
    return {
        "offsets": off.cpu().numpy().view(np.uint32),
        "key_tiles": kt.cpu().numpy().view(np.uint32)[:n],
        "flags": fl.cpu().numpy().view(np.uint16)[:n],
    }


def tile_map_descriptors(grid_h, grid_w, r2, device="cuda", window: str = "circle"):
    """The kernels' tile map built on the device with each entry's descriptor
    (clear_tile_map_descriptors); returns numpy copies, ``desc`` as [n, 4] uint32."""
    import torch

    L = lib()
    n = tile_map_size(grid_h, grid_w, r2, window=window)
    nt = _ntiles(grid_h, grid_w, TILE_H, TILE_W)
    off = torch.zeros(nt + 1, dtype=torch.int32, device=device)
    kt = torch.zeros(max(n, 1), dtype=torch.int32, device=device)
    fl = torch.zeros(max(n, 1), dtype=torch.int16, device=device)
    desc = torch.zeros((max(n, 1), 4), dtype=torch.int32, device=device)
    got = ctypes.c_size_t()
    _check(L.clear_tile_map_descriptors(_window_code(window), grid_h, grid_w, r2, off.data_ptr(),
                                        kt.data_ptr(), fl.data_ptr(), desc.data_ptr(), n, ctypes.byref(got),
                                        _stream_of(off)))
    torch.cuda.current_stream(off.device).synchronize()
    return {
        "offsets": off.cpu().numpy().view(np.uint32),
        "key_tiles": kt.cpu().numpy().view(np.uint32)[:n],
        "flags": fl.cpu().numpy().view(np.uint16)[:n],
        "desc": desc.cpu().numpy().view(np.uint32)[:n],
    }
