"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bars: fp32 max-abs <= 1e-5, bf16 max-abs <= 2e-2 (inputs widened exactly, the
GPU output widened, oracle in fp64).  One key wrongly admitted or dropped moves
an output by ~1/(window size), far above 1e-5, so the fp32 cases (which run the
same chunk lists, flags and masks as bf16, at d = 64 and 128) pin the masks;
the bf16 cases at r <= 2 pin them for bf16 as well.
"""

import math

import numpy as np
import pytest
import torch

import dit_circular_local_amd as ca
from dit_circular_local_amd.inputs import WORKLOADS, make_qkv, workload_qkv
from oracle import attention, attention_rows, tile_map_bruteforce

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 2e-2}
# Log-sum-exp: the bf16 path sums the probabilities after rounding them to bf16
# (the values its P.V product uses), each off by at most 2^-9 relative, so the
# log of the sum is off by at most ~2^-9; 2^-8 leaves a factor of two.  The fp32
# path sums fp32 probabilities.
LSE_TOL = {"fp32": 1e-5, "bf16": 2.0 ** -8}


def _np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def _run(q, k, v, n_text, gh, gw, r2, **kw):
    out = ca.fwd(q, k, v, n_text, gh, gw, r2=r2, **kw)
    torch.cuda.synchronize()
    return out


def _check_full(dtype, B, H, n_text, gh, gw, d, r2, seed=0, q_mult=1.0, splits=0, lse=True):
    q, k, v = make_qkv(B, H, n_text, gh, gw, d, dtype, seed, rms_norm=(dtype == "bf16"),
                       scale=1.0 if dtype == "bf16" else 1.0 / math.sqrt(d), q_mult=q_mult,
                       device="cuda")
    out, l = _run(q, k, v, n_text, gh, gw, r2, return_lse=lse, text_splits=splits) if lse else \
        (_run(q, k, v, n_text, gh, gw, r2, text_splits=splits), None)
    ref, ref_lse = attention(_np(q), _np(k), _np(v), n_text, gh, gw, r2, workers=8)
    err = np.abs(_np(out) - ref).max()
    assert err <= TOL[dtype], f"{dtype} B{B} H{H} T{n_text} {gh}x{gw} d{d} r2={r2}: max-abs {err:.3e}"
    if lse:
        lerr = np.abs(_np(l) - ref_lse).max()
        assert lerr <= LSE_TOL[dtype], f"lse max-abs {lerr:.3e}"
    return err


def test_tiny_config_fp32():
    """16x16 grid + 8 text tokens, d 64, r 4, fp32: every output element."""
    w = WORKLOADS["tiny"]
    q, k, v = workload_qkv(w, seed=0, device="cuda")
    out = _run(q, k, v, w.n_text, w.grid_h, w.grid_w, 16)
    ref, _ = attention(_np(q), _np(k), _np(v), w.n_text, w.grid_h, w.grid_w, 16)
    assert np.abs(_np(out) - ref).max() <= 1e-5


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_text,gh,gw", [(8, 16, 16), (0, 19, 13), (1, 37, 19), (130, 24, 40)])
@pytest.mark.parametrize("r2", [-1, 0, 1, 2, 4, 8, 24, 63, 64, 10 ** 6])
def test_fp32_masks_exact(d, n_text, gh, gw, r2):
    if n_text == 0 and r2 < 0:
        pytest.skip("empty rows")
    _check_full("fp32", 1, 2, n_text, gh, gw, d, r2)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_text,gh,gw", [(8, 16, 16), (0, 21, 11), (33, 37, 19), (512, 20, 24)])
@pytest.mark.parametrize("r2", [-1, 0, 1, 2, 5, 16, 63, 64, 10 ** 6])
def test_bf16_small_grids(d, n_text, gh, gw, r2):
    if n_text == 0 and r2 < 0:
        pytest.skip("empty rows")
    _check_full("bf16", 1, 2, n_text, gh, gw, d, r2)


def test_radius_zero_without_text_is_exact_copy_of_v():
    """r2 = 0, no text: each row admits only itself, so O = V exactly (bf16)."""
    q, k, v = make_qkv(1, 3, 0, 23, 17, 128, "bf16", 5, device="cuda")
    out = _run(q, k, v, 0, 23, 17, 0)
    assert torch.equal(out, v)


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 64])
def test_text_splits_agree(splits):
    _check_full("fp32", 1, 2, 150, 30, 30, 128, 49, splits=splits)


def test_batch_and_heads_and_large_logits():
    _check_full("bf16", 2, 3, 40, 33, 18, 128, 36)
    # Q x 8: peaked softmax, exercises the running-max updates
    _check_full("bf16", 1, 2, 64, 32, 32, 128, 64, q_mult=8.0)
    _check_full("fp32", 1, 2, 64, 32, 32, 128, 64, q_mult=8.0)


def test_strict_and_inclusive_conventions_differ_only_on_the_circle():
    q, k, v = make_qkv(1, 1, 16, 40, 40, 128, "fp32", 3, rms_norm=False, scale=1 / 8, device="cuda")
    for r in (4, 8):
        for r2 in (r * r, r * r - 1):
            out = _run(q, k, v, 16, 40, 40, r2)
            ref, _ = attention(_np(q), _np(k), _np(v), 16, 40, 40, r2)
            assert np.abs(_np(out) - ref).max() <= 1e-5


@pytest.mark.parametrize("r", [8, 16, 32])
def test_flux_1024_bf16_and_fp32(r):
    """64x64 grid + 512 text, d 128: bf16 on 4 heads, fp32 (mask exactness) on 2 heads."""
    _check_full("bf16", 1, 4, 512, 64, 64, 128, r * r, seed=1)
    _check_full("fp32", 1, 2, 512, 64, 64, 128, r * r, seed=2)


def test_default_entry_point_matches_ex():
    q, k, v = make_qkv(1, 2, 512, 32, 32, 128, "bf16", 7, device="cuda")
    a = ca.fwd(q, k, v, 512, 32, 32, radius=8, use_ex=False)
    b = ca.fwd(q, k, v, 512, 32, 32, radius=8, use_ex=True)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_deterministic_repeats():
    q, k, v = make_qkv(1, 4, 512, 64, 64, 128, "bf16", 11, device="cuda")
    a = ca.fwd(q, k, v, 512, 64, 64, radius=16)
    # poison a second output buffer first
    b = torch.full_like(a, float("nan"))
    ca.fwd(q, k, v, 512, 64, 64, radius=16, out=b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@pytest.mark.parametrize("gh,gw,r2", [(64, 64, 64), (64, 64, 1023), (37, 19, 5), (512, 512, 1024),
                                      (9, 40, -1), (128, 128, 10 ** 6)])
def test_device_tile_map_matches_host(gh, gw, r2):
    dev = ca.tile_map_build_device(gh, gw, r2)
    host = ca.tile_map_build(gh, gw, r2)
    for key in host:
        np.testing.assert_array_equal(dev[key], host[key], err_msg=key)
    if gh * gw <= 4096:
        ref = tile_map_bruteforce(gh, gw, r2, box=True)
        for key in ref:
            np.testing.assert_array_equal(dev[key], ref[key], err_msg=key)


def _sample_rows(n_text, g, rng, n_img=48, n_txt=6):
    cells = [(0, 0), (0, g - 1), (g - 1, 0), (g - 1, g - 1), (15, 7), (16, 8), (g // 2, g // 2),
             (31, 0), (0, 31), (g - 17, g - 9)]
    cells += [tuple(x) for x in rng.integers(0, g, (n_img - len(cells), 2))]
    rows = [n_text + y * g + x for y, x in cells]
    rows += [0, n_text - 1] + rng.integers(0, n_text, n_txt - 2).tolist()
    return sorted(set(rows))


@pytest.mark.parametrize("r", [8, 16, 32])
def test_flux_2048_whole_heads(r):
    """128x128 grid + 512 text tokens, 24 heads in one launch (the 2048^2 FLUX
    shape): three heads compared element by element with the oracle, every
    output finite."""
    w = WORKLOADS["flux2k"]
    q, k, v = workload_qkv(w, seed=r, device="cuda")
    out = ca.fwd(q, k, v, w.n_text, w.grid_h, w.grid_w, radius=r)
    torch.cuda.synchronize()
    heads = [0, 11, 23]
    ref, _ = attention(_np(q[:, heads]), _np(k[:, heads]), _np(v[:, heads]), w.n_text, w.grid_h, w.grid_w,
                       r * r, workers=8)
    err = np.abs(_np(out[:, heads]) - ref).max()
    assert err <= 2e-2, f"r={r}: max-abs {err:.3e}"
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("r", [8, 16, 32])
def test_flux_4096_sampled_rows(r):
    """256x256 grid + 512 text tokens, 24 heads in one launch (the 4096^2
    FLUX shape): sampled rows of two heads against the oracle row by row."""
    w = WORKLOADS["flux4k"]
    q, k, v = workload_qkv(w, seed=r, device="cuda")
    out = ca.fwd(q, k, v, w.n_text, w.grid_h, w.grid_w, radius=r)
    torch.cuda.synchronize()
    rng = np.random.default_rng(100 + r)
    for h in (0, 23):
        rows = _sample_rows(w.n_text, w.grid_h, rng)
        ref, _ = attention_rows(_np(q[0, h]), _np(k[0, h]), _np(v[0, h]), w.n_text, w.grid_h,
                                w.grid_w, r * r, rows)
        err = np.abs(_np(out[0, h, rows]) - ref).max()
        assert err <= 2e-2, f"r={r} head {h}: max-abs {err:.3e}"
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("r", [8, 32])
def test_flux_8192_sampled_rows(r):
    """512x512 grid + 512 text tokens, 24 heads, bf16, the benchmark's launch
    configuration: sampled rows of two heads against the oracle row by row."""
    w = WORKLOADS["flux8k"]
    q, k, v = workload_qkv(w, seed=0, device="cuda")
    out = ca.fwd(q, k, v, w.n_text, w.grid_h, w.grid_w, radius=r)
    torch.cuda.synchronize()
    rng = np.random.default_rng(r)
    for h in (0, 23):
        rows = _sample_rows(w.n_text, w.grid_h, rng)
        ref, _ = attention_rows(_np(q[0, h]), _np(k[0, h]), _np(v[0, h]), w.n_text, w.grid_h,
                                w.grid_w, r * r, rows)
        got = _np(out[0, h, rows])
        err = np.abs(got - ref).max()
        assert err <= 2e-2, f"head {h}: max-abs {err:.3e}"
    assert torch.isfinite(out).all()
    del q, k, v, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("window", ["circle", "square"])
def test_radius_beyond_the_mask_table(window):
    """Radius 257 on a 262 x 21 grid + 8 text tokens, fp32, d 64: no lane-mask
    table is built above radius 256 (the grid's diagonal still exceeds it, so r2
    is not clamped), and partly admitted key tiles wholly on the grid take their
    masks from the per-element computation (rows more than 257 apart are cut).
    Sampled 8 x 8 blocks (top, bottom, ragged corners, middle) and text rows
    against the oracle row by row at 1e-5."""
    n_text, gh, gw, d, r2 = 8, 262, 21, 64, 257 * 257
    q, k, v = make_qkv(1, 1, n_text, gh, gw, d, "fp32", 7, scale=1.0 / math.sqrt(d), device="cuda")
    out = ca.fwd(q, k, v, n_text, gh, gw, r2=r2, window=window)
    torch.cuda.synchronize()
    blocks = [(0, 0), (0, 13), (254, 0), (256, 16), (128, 8), (4, 8), (259, 5)]
    rows = [0, n_text - 1] + [n_text + (y0 + y) * gw + x0 + x for y0, x0 in blocks
                              for y in range(8) for x in range(8) if y0 + y < gh and x0 + x < gw]
    ref, _ = attention_rows(_np(q[0, 0]), _np(k[0, 0]), _np(v[0, 0]), n_text, gh, gw, r2, rows, window=window)
    err = np.abs(_np(out[0, 0, rows]) - ref).max()
    assert err <= TOL["fp32"], f"{window} r2={r2}: max-abs {err:.3e}"


def test_host_threads_share_the_tile_map_cache():
    """Eight host threads call the forward at once on one stream (ctypes drops
    the GIL for the call), building six tile maps concurrently in a cold cache;
    every output equals a single-threaded run bit for bit (the cache is guarded
    by the library's mutex; calls on one stream are ordered)."""
    import threading

    configs = [(16, 16, 16), (19, 13, 9), (24, 40, 25), (16, 16, 4), (33, 7, 2), (9, 30, 64)]
    n_text, d = 8, 64
    inputs = [make_qkv(1, 2, n_text, gh, gw, d, "fp32", 40 + i, scale=1.0 / math.sqrt(d), device="cuda")
              for i, (gh, gw, _) in enumerate(configs)]
    ca.release_cache()
    ref = [ca.fwd(q, k, v, n_text, gh, gw, r2=r2) for (q, k, v), (gh, gw, r2) in zip(inputs, configs)]
    torch.cuda.synchronize()
    ca.release_cache()
    jobs = [i % len(configs) for i in range(2 * len(configs))]
    outs = [torch.empty_like(inputs[i][0]) for i in jobs]
    errors = []
    stream = torch.cuda.current_stream()

    def worker(t):
        try:
            with torch.cuda.stream(stream):
                for n in range(t, len(jobs), 8):
                    i = jobs[n]
                    (q, k, v), (gh, gw, r2) = inputs[i], configs[i]
                    ca.fwd(q, k, v, n_text, gh, gw, r2=r2, out=outs[n])
        except Exception as e:  # noqa: BLE001 - reported below
            errors.append(repr(e))

    threads = [threading.Thread(target=worker, args=(t,)) for t in range(8)]
    for t in threads:
        t.start()
    for t in threads:
        t.join()
    torch.cuda.synchronize()
    assert not errors, errors
    for n, i in enumerate(jobs):
        assert torch.equal(outs[n], ref[i]), f"job {n} (config {configs[i]})"


@pytest.mark.parametrize("gh,gw", [(ca.MAX_GRID, 3), (5, ca.MAX_GRID)])
@pytest.mark.parametrize("r2", [9, 10 ** 6])
def test_maximum_grid_side(gh, gw, r2):
    """Grid sides at the largest accepted value (CLEAR_MAX_GRID), fp32, d 64,
    4 text tokens; r2 = 10^6 exceeds the mask table's radius (no table).
    Sampled rows (both ends of the long side, the middle, text rows) against
    the oracle at 1e-5."""
    n_text, d = 4, 64
    q, k, v = make_qkv(1, 1, n_text, gh, gw, d, "fp32", 50, scale=1.0 / math.sqrt(d), device="cuda")
    out = ca.fwd(q, k, v, n_text, gh, gw, r2=r2)
    torch.cuda.synchronize()
    cells = [(0, 0), (gh - 1, gw - 1), (gh // 2, gw // 2), (gh - 1, 0), (0, gw - 1), (gh // 3, gw // 3)]
    rows = [0, n_text - 1] + [n_text + y * gw + x for y, x in cells]
    ref, _ = attention_rows(_np(q[0, 0]), _np(k[0, 0]), _np(v[0, 0]), n_text, gh, gw, r2, rows)
    err = np.abs(_np(out[0, 0, rows]) - ref).max()
    assert err <= TOL["fp32"], f"{gh}x{gw} r2={r2}: max-abs {err:.3e}"
    assert torch.isfinite(out).all()


@pytest.mark.parametrize("n_text,gh,gw", [(3, 1, 1), (0, 1, 1), (5, 1, 7), (0, 9, 1), (2, 1, 40)])
@pytest.mark.parametrize("r2", [0, 1, 50])
def test_degenerate_grids(n_text, gh, gw, r2):
    """One image token, one row, one column (with and without text), fp32,
    every output element and the LSE against the oracle."""
    _check_full("fp32", 1, 2, n_text, gh, gw, 64, r2)


def test_full_grid_heads_beyond_4_gb():
    """The largest grid, 8192 x 8192 with 2 text tokens (N = 67,108,866), bf16,
    d 128: one head of K is 17.2 GB, so key offsets within a head pass 2^31,
    2^32 and 2^33 bytes.
    * r = 197 would list more key tiles than the kernels index (2^31 - 1): the
      call fails with CLEAR_ENOTSUP before launching anything.
    * r = 2: image rows at the corners, the middle and on both sides of the
      2^31 / 2^32 / 2^33-byte token offsets against the oracle on the window box
      around each cell (an exact sub-problem, see tests/window_box.py).
    * Text rows: their queries are zero, so every key weighs the same; with V
      the indicator of 128 consecutive key ranges times 128, output column c is
      128 x (range c's share of the keys), about 1.  A key range lost or counted
      twice by the split text rows moves its column by its share."""
    from window_box import box_reference

    G, n_text, d = ca.MAX_GRID, 2, 128
    N = n_text + G * G
    gen = torch.Generator(device="cuda").manual_seed(71)
    q, k, v = (torch.randn(1, 1, N, d, device="cuda", dtype=torch.bfloat16, generator=gen) for _ in range(3))
    q[0, 0, :n_text] = 0
    with pytest.raises(ca.ClearError) as err:
        ca.fwd(q, k, v, n_text, G, G, radius=197)
    assert err.value.code == ca.CLEAR_ENOTSUP

    out = _run(q, k, v, n_text, G, G, 4)
    row_bytes = d * 2
    toks = [N - 1] + [b // row_bytes + s for b in (2 ** 31, 2 ** 32, 2 ** 33) for s in (-1, 0, 1)]
    cells = [(0, 0), (0, G - 1), (G - 1, 0), (G // 2, G // 2)] + [divmod(t - n_text, G) for t in toks]
    rows, ref = box_reference(q[0, 0], k[0, 0], v[0, 0], n_text, G, G, 4, cells)
    err_img = np.abs(_np(out[0, 0, rows]) - ref).max()
    assert err_img <= TOL["bf16"], f"image rows: max-abs {err_img:.3e}"

    del out
    blk = torch.arange(N, device="cuda") * 128 // N
    v.zero_()
    v[0, 0, torch.arange(N, device="cuda"), blk] = 128.0
    out = _run(q, k, v, n_text, G, G, 4)
    want = 128.0 * torch.bincount(blk, minlength=128).double().cpu().numpy() / N
    err_txt = np.abs(_np(out[0, 0, :n_text]) - want[None, :]).max()
    assert err_txt <= TOL["bf16"], f"text rows: max-abs {err_txt:.3e}"
    del q, k, v, out, blk
    torch.cuda.empty_cache()
