"""GPU parity of the square-window variant (max(dy^2, dx^2) <= r2) against the
fp64 oracle, through the C ABI.  Same bars as the circular window: fp32 max-abs
1e-5 (which also pins the masks: one key too many or too few moves an output by
far more), bf16 max-abs 2e-2, tile maps bit for bit."""

import math

import numpy as np
import pytest
import torch

import dit_circular_local_amd as ca
from dit_circular_local_amd.inputs import WORKLOADS, make_qkv, workload_qkv
from oracle import attention, attention_rows, tile_map_bruteforce
from window_box import box_reference

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 2e-2}


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _check(dtype, B, H, n_text, gh, gw, d, r2, seed=0, q_mult=1.0):
    q, k, v = make_qkv(B, H, n_text, gh, gw, d, dtype, seed, rms_norm=(dtype == "bf16"),
                       scale=1.0 if dtype == "bf16" else 1.0 / math.sqrt(d), q_mult=q_mult,
                       device="cuda")
    out = ca.fwd(q, k, v, n_text, gh, gw, r2=r2, window="square")
    torch.cuda.synchronize()
    ref, _ = attention(_np(q), _np(k), _np(v), n_text, gh, gw, r2, workers=8, window="square")
    err = np.abs(_np(out) - ref).max()
    assert err <= TOL[dtype], f"square {dtype} {gh}x{gw}+{n_text} d{d} r2={r2}: max-abs {err:.3e}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_text,gh,gw", [(8, 16, 16), (0, 19, 13), (130, 24, 40)])
@pytest.mark.parametrize("r2", [-1, 0, 1, 4, 9, 24, 64, 10 ** 6])
def test_square_fp32_masks_exact(d, n_text, gh, gw, r2):
    if n_text == 0 and r2 < 0:
        pytest.skip("empty rows")
    _check("fp32", 1, 2, n_text, gh, gw, d, r2)


@pytest.mark.parametrize("n_text,gh,gw,r2", [(8, 16, 16, 4), (33, 37, 19, 16), (512, 20, 24, 64)])
def test_square_bf16_small_grids(n_text, gh, gw, r2):
    _check("bf16", 1, 2, n_text, gh, gw, 128, r2)


@pytest.mark.parametrize("r", [8, 16])
def test_square_flux_1024(r):
    _check("bf16", 1, 4, 512, 64, 64, 128, r * r, seed=3)
    _check("fp32", 1, 2, 512, 64, 64, 128, r * r, seed=4, q_mult=2.0)


@pytest.mark.parametrize("gh,gw,r2", [(64, 64, 64), (37, 19, 5), (512, 512, 1024)])
def test_square_device_tile_map_matches_host(gh, gw, r2):
    dev = ca.tile_map_build_device(gh, gw, r2, window="square")
    host = ca.tile_map_build(gh, gw, r2, window="square")
    for key in host:
        np.testing.assert_array_equal(dev[key], host[key], err_msg=key)
    if gh * gw <= 4096:
        ref = tile_map_bruteforce(gh, gw, r2, box=True, window="square")
        for key in ref:
            np.testing.assert_array_equal(dev[key], ref[key], err_msg=key)


def test_square_and_circle_differ_and_share_nothing_cached():
    """Both windows on the same (grid, r2) in one process: each matches its own oracle
    (the tile-map cache is keyed by the window)."""
    q, k, v = make_qkv(1, 1, 16, 24, 24, 128, "fp32", 9, rms_norm=False, scale=1 / 8, device="cuda")
    oc = ca.fwd(q, k, v, 16, 24, 24, r2=25, use_ex=True)
    osq = ca.fwd(q, k, v, 16, 24, 24, r2=25, window="square")
    torch.cuda.synchronize()
    rc, _ = attention(_np(q), _np(k), _np(v), 16, 24, 24, 25)
    rs, _ = attention(_np(q), _np(k), _np(v), 16, 24, 24, 25, window="square")
    assert np.abs(_np(oc) - rc).max() <= 1e-5 and np.abs(_np(osq) - rs).max() <= 1e-5
    assert np.abs(rc - rs).max() > 1e-3


def test_square_flux_8192_sampled_rows():
    """512x512 grid + 512 text, 24 heads, bf16, r = 32: sampled rows of two heads."""
    w = WORKLOADS["flux8k"]
    q, k, v = workload_qkv(w, seed=0, device="cuda")
    out = ca.fwd(q, k, v, w.n_text, w.grid_h, w.grid_w, r2=32 * 32, window="square")
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    g = w.grid_h
    cells = [(0, 0), (g - 1, g - 1), (0, g - 1), (g // 2, g // 2), (31, 33), (200, 7)]
    cells += [tuple(c) for c in rng.integers(0, g, (20, 2))]
    rows = sorted(set([w.n_text + y * g + x for y, x in cells] + [0, w.n_text - 1]))
    for h in (0, 23):
        ref, _ = attention_rows(_np(q[0, h]), _np(k[0, h]), _np(v[0, h]), w.n_text, g, g, 32 * 32,
                                rows, window="square")
        err = np.abs(_np(out[0, h, rows]) - ref).max()
        assert err <= 2e-2, f"head {h}: max-abs {err:.3e}"
    del q, k, v, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("r", [8, 32])
def test_square_flux_8192_fp32_boundary_rows(r):
    """512x512 grid + 512 text, 24 heads in one launch, fp32 inputs with the
    FLUX recipe, square window: rows of heads 0 and 23 on the tilings'
    boundaries, the grid's edges and corners, and random rows, against the
    window-box reference at 1e-5, where one key too many or too few shows."""
    w = WORKLOADS["flux8k"]
    q, k, v = make_qkv(w.B, w.H, w.n_text, w.grid_h, w.grid_w, w.d, "fp32", seed=120 + r, rms_norm=True,
                       scale=1.0, device="cuda")
    out = ca.fwd(q, k, v, w.n_text, w.grid_h, w.grid_w, radius=r, window="square")
    torch.cuda.synchronize()
    g = w.grid_h
    rng = np.random.default_rng(r)
    ys = sorted({0, 1, 3, 4, 15, 16, 31, 32, g // 2, g - 17, g - 16, g - 5, g - 4, g - 1})
    xs = sorted({0, 1, 7, 8, 15, 16, g // 2, g - 9, g - 8, g - 1})
    cells = sorted(set([(y, x) for y in ys for x in xs] + [tuple(int(c) for c in rc)
                                                         for rc in rng.integers(0, g, (30, 2))]))
    for h in (0, 23):
        rows, ref = box_reference(q[0, h], k[0, h], v[0, h], w.n_text, g, g, r * r, cells, window="square")
        err = np.abs(_np(out[0, h, rows]) - ref)
        i = int(err.max(axis=1).argmax())
        assert err.max() <= 1e-5, f"r={r} head {h}: max-abs {err.max():.3e} at cell {cells[i]}"
    del q, k, v, out
    torch.cuda.empty_cache()
