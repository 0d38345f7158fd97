"""Seeded synthetic Q/K/V for CLEAR attention.

This module only draws inputs.  It holds none of the attention arithmetic, so
both the GPU path's tests and the CPU oracle can take their inputs from it.

Workloads (the shapes the pages' experiments run FLUX-1.dev at: 24 heads,
head_dim 128, 512 text tokens, and 1024^2 ... 8192^2 images, i.e. token grids
of 64^2 ... 512^2 after the 16x patchify; atlas.scime.ai summary of CLEAR,
"Key results"; pith.science review, "Assumptions & free parameters" for
r in {8, 16, 32}):

* ``tiny``    B1 H1 d64, 16x16 grid + 8 text tokens, r = 4, float32,
              Q/K/V ~ N(0, 1) / sqrt(64), no normalisation;
* ``flux1k``  B1 H24 d128, 64x64 grid + 512 text, r in {8, 16, 32};
* ``flux2k``  128x128 grid, ``flux4k`` 256x256, ``flux8k`` 512x512 (r in {8, 32}).

FLUX configs draw N(0, 1) in float32, RMS-normalise Q and K per token and head
(x / sqrt(mean_c x_c^2 + 1e-6), no learned weight: a stand-in for the model's
QK-norm, which sits upstream of attention), then round Q, K, V to bfloat16
with round-to-nearest-even.

Every (tensor, batch, head) slab has its own seed derived from the base seed,
so any head can be regenerated alone (the oracle checks sampled heads of the
512x512 workload without drawing all 24).

The backward's upstream gradient dO is drawn the same way (N(0, 1) times the
workload's scale, rounded to its dtype, no normalisation), from seeds of its
own.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Tuple

import torch

__all__ = ["Workload", "WORKLOADS", "make_qkv", "make_head", "make_dout", "slab_seed"]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    n_text: int
    grid_h: int
    grid_w: int
    radii: Tuple[int, ...]
    dtype: str          # "bf16" or "fp32"
    rms_norm: bool
    scale: float        # multiplies the N(0,1) draw (before normalisation)

    @property
    def n(self) -> int:
        return self.n_text + self.grid_h * self.grid_w


WORKLOADS = {
    "tiny": Workload("tiny", 1, 1, 64, 8, 16, 16, (4,), "fp32", False, 1.0 / 8.0),
    "flux1k": Workload("flux1k", 1, 24, 128, 512, 64, 64, (8, 16, 32), "bf16", True, 1.0),
    "flux2k": Workload("flux2k", 1, 24, 128, 512, 128, 128, (8, 16, 32), "bf16", True, 1.0),
    "flux4k": Workload("flux4k", 1, 24, 128, 512, 256, 256, (8, 16, 32), "bf16", True, 1.0),
    "flux8k": Workload("flux8k", 1, 24, 128, 512, 512, 512, (8, 32), "bf16", True, 1.0),
}

_TENSOR_ID = {"q": 0, "k": 1, "v": 2}


_DOUT_BASE = 1 << 48


def slab_seed(seed: int, tensor: str, b: int, h: int) -> int:
    """Seed of one [N, d] slab: a fixed injective map of (seed, tensor, b, h);
    tensor "dout" maps above every Q/K/V seed."""
    if tensor == "dout":
        return _DOUT_BASE + slab_seed(seed, "q", b, h)
    return ((seed * 3 + _TENSOR_ID[tensor]) * 4096 + b) * 4096 + h


def _torch_dtype(dtype: str):
    return {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]


def make_head(n: int, d: int, tensor: str, b: int, h: int, seed: int = 0,
              dtype: str = "bf16", rms_norm: bool = True, scale: float = 1.0,
              q_mult: float = 1.0) -> torch.Tensor:
    """One [n, d] CPU slab of Q, K or V."""
    g = torch.Generator(device="cpu")
    g.manual_seed(slab_seed(seed, tensor, b, h))
    x = torch.randn(n, d, generator=g, dtype=torch.float32) * scale
    if rms_norm and tensor in ("q", "k"):
        x = x / torch.sqrt(x.pow(2).mean(dim=-1, keepdim=True) + 1e-6)
    if tensor == "q" and q_mult != 1.0:
        x = x * q_mult
    return x.to(_torch_dtype(dtype))


def make_qkv(B: int, H: int, n_text: int, grid_h: int, grid_w: int, d: int,
             dtype: str = "bf16", seed: int = 0, rms_norm: bool = True,
             scale: float = 1.0, q_mult: float = 1.0,
             device: Optional[str] = None):
    """Q, K, V of shape [B, H, n_text + grid_h*grid_w, d], contiguous.

    Slabs are drawn on the CPU; with ``device`` set they are moved there one
    slab at a time (so a 512x512 workload never holds float32 copies of all
    heads at once).
    """
    n = n_text + grid_h * grid_w
    tdt = _torch_dtype(dtype)
    out = []
    for name in ("q", "k", "v"):
        t = torch.empty((B, H, n, d), dtype=tdt, device=device or "cpu")
        for b in range(B):
            for h in range(H):
                t[b, h].copy_(make_head(n, d, name, b, h, seed, dtype, rms_norm, scale, q_mult))
        out.append(t)
    return tuple(out)


def make_dout(B: int, H: int, n: int, d: int, dtype: str = "bf16", seed: int = 0,
              scale: float = 1.0, device: Optional[str] = None) -> torch.Tensor:
    """Upstream gradient dO [B, H, n, d]: N(0, 1) * scale per slab, rounded to dtype."""
    t = torch.empty((B, H, n, d), dtype=_torch_dtype(dtype), device=device or "cpu")
    for b in range(B):
        for h in range(H):
            g = torch.Generator(device="cpu")
            g.manual_seed(slab_seed(seed, "dout", b, h))
            t[b, h].copy_((torch.randn(n, d, generator=g, dtype=torch.float32) * scale).to(t.dtype))
    return t


def workload_qkv(w: Workload, seed: int = 0, device: Optional[str] = None,
                 q_mult: float = 1.0):
    """Q, K, V of a named workload."""
    return make_qkv(w.B, w.H, w.n_text, w.grid_h, w.grid_w, w.d, w.dtype, seed,
                    w.rms_norm, w.scale, q_mult, device)
