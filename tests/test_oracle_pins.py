"""Pins of the CPU oracle's attention and counts against facts outside the oracle.

Each test fixes something the pages or plain mathematics determine, chosen so
that a plausible slip in the oracle (dropped 1/sqrt(d), a transposed operand,
"<" for "<=", grid_h for grid_w, text coupling dropped, a candidate box one
cell short) fails at least one of them.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import (attention, attention_head, attention_rows, clear_mask,
                    lattice_count, pair_count, pair_count_bruteforce)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def _sdpa(q, k, v):
    """Dense softmax attention by torch's library routine, CPU float64."""
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a))[None, None] for a in (q, k, v))
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, 0].numpy()


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("n_text,gh,gw,d", [(3, 5, 7, 16), (0, 4, 4, 8), (8, 6, 3, 32)])
def test_radius_beyond_diagonal_is_dense_attention(n_text, gh, gw, d):
    """r^2 >= (gh-1)^2 + (gw-1)^2 admits every pair: CLEAR == full attention."""
    n = n_text + gh * gw
    q, k, v = (_rand((n, d), s) for s in (1, 2, 3))
    for r2 in ((gh - 1) ** 2 + (gw - 1) ** 2, 10 ** 6):
        out, _ = attention_head(q, k, v, n_text, gh, gw, r2, block=4)
        np.testing.assert_allclose(out, _sdpa(q, k, v), rtol=0, atol=1e-12)


def test_radius_zero_without_text_returns_v_exactly():
    """r2 = 0, no text: each image row admits only itself, so O_i = v_i exactly."""
    gh, gw, d = 6, 5, 16
    q, k, v = (_rand((gh * gw, d), s) for s in (4, 5, 6))
    out, _ = attention_head(q, k, v, 0, gh, gw, 0, block=4)
    assert np.array_equal(out, v)
    # the strict reading of r = 1 ("< 1") is the same lattice set as r2 = 0
    out1, _ = attention_head(q, k, v, 0, gh, gw, 1 * 1 - 1, block=4)
    assert np.array_equal(out1, v)


def test_radius_zero_with_text_is_attention_over_text_plus_self():
    n_text, gh, gw, d = 4, 5, 6, 16
    n = n_text + gh * gw
    q, k, v = (_rand((n, d), s) for s in (7, 8, 9))
    out, _ = attention_head(q, k, v, n_text, gh, gw, 0, block=4)
    for i in range(n):
        keys = list(range(n)) if i < n_text else list(range(n_text)) + [i]
        ref = _sdpa(q[i:i + 1], k[keys], v[keys])
        np.testing.assert_allclose(out[i:i + 1], ref, rtol=0, atol=1e-12)


def test_negative_r2_is_text_only_for_image_rows():
    n_text, gh, gw, d = 5, 4, 7, 8
    n = n_text + gh * gw
    q, k, v = (_rand((n, d), s) for s in (10, 11, 12))
    out, _ = attention_head(q, k, v, n_text, gh, gw, -1, block=3)
    ref_img = _sdpa(q[n_text:], k[:n_text], v[:n_text])
    np.testing.assert_allclose(out[n_text:], ref_img, rtol=0, atol=1e-12)
    np.testing.assert_allclose(out[:n_text], _sdpa(q[:n_text], k, v), rtol=0, atol=1e-12)


def test_empty_rows_are_rejected():
    q = _rand((9, 4), 0)
    with pytest.raises(ValueError):
        attention_head(q, q, q, 0, 3, 3, -1)
    with pytest.raises(ValueError):
        attention_rows(q, q, q, 0, 3, 3, -1, rows=[0])


def test_rows_sum_to_one_and_masked_probs_are_zero():
    n_text, gh, gw, d, r2 = 3, 7, 9, 8, 5
    n = n_text + gh * gw
    q, k, v = (_rand((n, d), s, 2.0) for s in (13, 14, 15))
    rows = list(range(n))
    _, _, p = attention_rows(q, k, v, n_text, gh, gw, r2, rows, return_probs=True)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=0, atol=1e-13)
    m = clear_mask(rows, range(n), n_text, gw, r2)
    assert np.all(p[~m] == 0.0)
    assert np.all(p[m] > 0.0)


def test_constant_v_gives_constant_output():
    n_text, gh, gw, d = 2, 6, 6, 8
    n = n_text + gh * gw
    q, k = _rand((n, d), 16), _rand((n, d), 17)
    v = np.full((n, d), 0.375)
    out, _ = attention_head(q, k, v, n_text, gh, gw, 4, block=4)
    np.testing.assert_allclose(out, 0.375, rtol=0, atol=1e-14)


def _window_interval_mean(v, n_text, gh, gw, r2, y, x):
    """Mean of v over text keys plus the disk around (y, x), enumerated per key
    row as the column interval |dx| <= isqrt(r2 - dy^2): a construction that
    does not evaluate the mask."""
    keys = list(range(n_text))
    if r2 >= 0:
        w = math.isqrt(r2)
        for dy in range(-w, w + 1):
            ky = y + dy
            if not 0 <= ky < gh:
                continue
            half = math.isqrt(r2 - dy * dy)
            for kx in range(max(0, x - half), min(gw - 1, x + half) + 1):
                keys.append(n_text + ky * gw + kx)
    return v[keys].mean(axis=0), len(keys)


@pytest.mark.parametrize("r2", [0, 1, 2, 4, 5, 10, 16, 24])
def test_zero_queries_average_v_over_the_window(r2):
    """Q = 0 makes every admitted logit 0, so O_i is the plain mean of v_j over
    the admitted keys.  The admitted set is rebuilt independently of the mask."""
    n_text, gh, gw, d = 3, 9, 11, 4
    n = n_text + gh * gw
    q = np.zeros((n, d))
    k, v = _rand((n, d), 18), _rand((n, d), 19)
    out, _ = attention_head(q, k, v, n_text, gh, gw, r2, block=4)
    for y in range(gh):
        for x in range(gw):
            ref, _ = _window_interval_mean(v, n_text, gh, gw, r2, y, x)
            np.testing.assert_allclose(out[n_text + y * gw + x], ref, rtol=0, atol=1e-13)
    np.testing.assert_allclose(out[:n_text], np.broadcast_to(v.mean(axis=0), (n_text, d)),
                               rtol=0, atol=1e-13)


def test_text_permutation():
    """Permuting text tokens leaves image outputs unchanged and permutes text outputs."""
    n_text, gh, gw, d, r2 = 6, 5, 5, 8, 2
    n = n_text + gh * gw
    q, k, v = (_rand((n, d), s) for s in (20, 21, 22))
    perm = np.random.default_rng(0).permutation(n_text)
    full = np.concatenate([perm, np.arange(n_text, n)])
    out, _ = attention_head(q, k, v, n_text, gh, gw, r2, block=4)
    out_p, _ = attention_head(q[full], k[full], v[full], n_text, gh, gw, r2, block=4)
    np.testing.assert_allclose(out_p[n_text:], out[n_text:], rtol=0, atol=1e-13)
    np.testing.assert_allclose(out_p[:n_text], out[perm], rtol=0, atol=1e-13)


def test_grid_transpose_on_a_non_square_grid():
    """Relabelling image cell (y, x) as (x, y) on the transposed grid permutes the
    outputs the same way; a grid_h / grid_w mix-up breaks this."""
    n_text, gh, gw, d, r2 = 2, 5, 9, 8, 5
    n = n_text + gh * gw
    q, k, v = (_rand((n, d), s) for s in (23, 24, 25))
    # new index of old image cell (y, x) is n_text + x*gh + y on the gw x gh grid
    new_of_old = np.arange(n)
    for y in range(gh):
        for x in range(gw):
            new_of_old[n_text + y * gw + x] = n_text + x * gh + y
    old_of_new = np.argsort(new_of_old)
    out, _ = attention_head(q, k, v, n_text, gh, gw, r2, block=4)
    out_t, _ = attention_head(q[old_of_new], k[old_of_new], v[old_of_new], n_text, gw, gh, r2, block=4)
    np.testing.assert_allclose(out_t[new_of_old], out, rtol=0, atol=1e-13)


def test_horizontal_flip_symmetry():
    n_text, gh, gw, d, r2 = 1, 6, 7, 8, 8
    n = n_text + gh * gw
    q, k, v = (_rand((n, d), s) for s in (26, 27, 28))
    flip = np.arange(n)
    for y in range(gh):
        for x in range(gw):
            flip[n_text + y * gw + x] = n_text + y * gw + (gw - 1 - x)
    out, _ = attention_head(q, k, v, n_text, gh, gw, r2, block=4)
    out_f, _ = attention_head(q[flip], k[flip], v[flip], n_text, gh, gw, r2, block=4)
    np.testing.assert_allclose(out_f[flip], out, rtol=0, atol=1e-13)


def test_locality_keys_outside_the_window_do_not_matter():
    n_text, gh, gw, d, r2 = 2, 10, 10, 8, 4
    n = n_text + gh * gw
    q, k, v = (_rand((n, d), s) for s in (29, 30, 31))
    i = n_text + 5 * gw + 5
    far = [j for j in range(n_text, n) if not clear_mask([i], [j], n_text, gw, r2)[0, 0]]
    v2, k2 = v.copy(), k.copy()
    v2[far] += 100.0
    k2[far] *= -3.0
    o1, _ = attention_rows(q, k, v, n_text, gh, gw, r2, [i])
    o2, _ = attention_rows(q, k2, v2, n_text, gh, gw, r2, [i])
    assert np.array_equal(o1, o2)
    # and the near ones do matter
    near = [j for j in range(n_text, n) if clear_mask([i], [j], n_text, gw, r2)[0, 0]]
    v3 = v.copy()
    v3[near[0]] += 1.0
    o3, _ = attention_rows(q, k, v3, n_text, gh, gw, r2, [i])
    assert not np.array_equal(o1, o3)


@pytest.mark.parametrize("n_text,gh,gw,r2,block", [
    (3, 9, 13, 10, 4), (0, 7, 5, 2, 3), (5, 12, 12, 17, 8), (2, 17, 3, 9, 8), (4, 6, 6, -1, 4)])
def test_blocked_oracle_matches_full_row_definition(n_text, gh, gw, r2, block):
    """The blocked oracle (candidate box per block) against the per-row
    definition over all N keys, including ragged blocks at the grid edge."""
    n = n_text + gh * gw
    d = 8
    q, k, v = (_rand((n, d), s, 1.5) for s in (32, 33, 34))
    out, lse = attention_head(q, k, v, n_text, gh, gw, r2, block=block)
    ref, ref_lse = attention_rows(q, k, v, n_text, gh, gw, r2, range(n))
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)


def test_lse_is_log_partition():
    n_text, gh, gw, d, r2 = 2, 4, 4, 8, 2
    n = n_text + gh * gw
    q, k, v = (_rand((n, d), s) for s in (35, 36, 37))
    _, lse = attention_rows(q, k, v, n_text, gh, gw, r2, range(n))
    s = q @ k.T / math.sqrt(d)
    m = clear_mask(range(n), range(n), n_text, gw, r2)
    ref = np.log(np.where(m, np.exp(s), 0.0).sum(axis=1))
    np.testing.assert_allclose(lse, ref, rtol=0, atol=1e-12)


def test_batched_driver_matches_per_head():
    B, H, n_text, gh, gw, d, r2 = 2, 2, 3, 5, 6, 8, 4
    n = n_text + gh * gw
    q, k, v = (_rand((B, H, n, d), s) for s in (38, 39, 40))
    out, lse = attention(q, k, v, n_text, gh, gw, r2, block=4, workers=2)
    for b in range(B):
        for h in range(H):
            o, l_ = attention_head(q[b, h], k[b, h], v[b, h], n_text, gh, gw, r2, block=4)
            np.testing.assert_array_equal(out[b, h], o)
            np.testing.assert_array_equal(lse[b, h], l_)


# ---------------------------------------------------------------- counts

def _gauss(r: int) -> int:
    """Gauss circle count 1 + 4r + 4 * sum_{i=1..r} floor(sqrt(r^2 - i^2))."""
    return 1 + 4 * r + 4 * sum(math.isqrt(r * r - i * i) for i in range(1, r + 1))


def test_lattice_counts_match_the_gauss_circle_closed_form():
    for r in range(0, 41):
        assert lattice_count(r * r) == _gauss(r)
    assert [lattice_count(r * r) for r in (4, 8, 16, 32)] == [49, 197, 797, 3209]
    # strict "<" reading: four fewer points on the axes at these radii
    assert [lattice_count(r * r - 1) for r in (4, 8, 16, 32)] == [45, 193, 793, 3205]


@pytest.mark.parametrize("r", [4, 8, 16, 32])
def test_interior_query_admits_the_lattice_disk(r):
    """The oracle's own mask, counted over one interior row, equals the disk count."""
    n_text, g = 7, 2 * r + 3
    y = x = r + 1
    i = n_text + y * g + x
    row = clear_mask([i], range(n_text + g * g), n_text, g, r * r)[0]
    assert int(row[n_text:].sum()) == _gauss(r)
    assert int(row[:n_text].sum()) == n_text


def test_circle_costs_about_pi_over_4_of_its_square():
    """The review's 'about pi/4 of a square window' claim, exactly."""
    ratios = {r: lattice_count(r * r) / (2 * r + 1) ** 2 for r in (8, 16, 32, 400)}
    assert round(ratios[8], 2) == 0.68
    assert round(ratios[16], 2) == 0.73
    assert round(ratios[32], 2) == 0.76
    assert abs(ratios[400] - math.pi / 4) < 0.01


@pytest.mark.parametrize("n_text,gh,gw,r2", [
    (0, 5, 5, 0), (3, 4, 9, 1), (2, 7, 3, 2), (5, 6, 6, 5), (1, 8, 5, 13), (4, 5, 7, -1), (2, 4, 4, 1000)])
def test_pair_count_matches_mask_sum(n_text, gh, gw, r2):
    assert pair_count(n_text, gh, gw, r2)["total"] == pair_count_bruteforce(n_text, gh, gw, r2)


def test_pages_reduction_and_speedup_figures():
    """99.5 % fewer attention pairs at 8192^2 and the 6.3x figure (see golden file)."""
    with open(os.path.join(GOLDEN, "pages_numbers.json")) as f:
        g = json.load(f)
    grid = g["readings"]["token_grid_8k"]["value"]
    n_text = g["readings"]["n_text"]["value"]
    r = g["readings"]["radius_for_99_5"]["value"]
    c = pair_count(n_text, grid, grid, r * r)
    reduction = 100.0 * (1.0 - c["total"] / c["dense"])
    assert round(reduction, g["attention_compute_reduction_percent_8k"]["printed_precision"]) == \
        g["attention_compute_reduction_percent_8k"]["value"]
    # the counts behind it, also listed in the design notes
    assert c["img_img"] == 50_968_484
    assert c["total"] == 319_666_084
    t = g["seconds_per_50_steps_8k"]
    assert round(t["flux_1_dev"] / t["clear_r8"], 1) == g["speedup_8k"]["value"]
    # if text queries saw only text (not the review's reading), 8K r=8 would read 99.7
    alt = c["img_img"] + c["img_text"] + n_text * n_text
    assert round(100.0 * (1.0 - alt / c["dense"]), 1) == 99.7


# ---------------------------------------------------------------- in_window_pairs
# The oracle's pair counter converts a timed sample of oracle rows into
# in-window FLOPs.  Pinned against the separable closed form (pair_count, itself
# pinned to the mask sum above), against direct mask sums of the sampled rows,
# and by additivity over disjoint row subsets.

@pytest.mark.parametrize("window", ["circle", "square"])
@pytest.mark.parametrize("n_text,gh,gw,r2,block", [
    (3, 9, 13, 5, 4), (0, 8, 8, 0, 8), (5, 17, 6, 20, 8), (2, 10, 10, -1, 4), (4, 7, 11, 1000, 3)])
def test_in_window_pairs_whole_layer_equals_closed_form(window, n_text, gh, gw, r2, block):
    from oracle import in_window_pairs

    assert in_window_pairs(n_text, gh, gw, r2, block=block, window=window) == \
        pair_count(n_text, gh, gw, r2, window)["total"]


@pytest.mark.parametrize("window", ["circle", "square"])
def test_in_window_pairs_subset_equals_mask_sum_of_its_rows(window):
    """A chosen set of text rows and image blocks: the count equals the mask
    summed over exactly those query rows and every key."""
    from oracle import in_window_pairs

    n_text, gh, gw, r2, block = 6, 19, 14, 18, 4
    n = n_text + gh * gw
    text_rows = [0, 2, 5]
    blocks = [(0, 0), (2, 3), (4, 1), (4, 3)]  # includes the clipped bottom-right block
    rows = list(text_rows)
    for by, bx in blocks:
        for y in range(by * block, min(gh, by * block + block)):
            for x in range(bx * block, min(gw, bx * block + block)):
                rows.append(n_text + y * gw + x)
    want = int(clear_mask(rows, range(n), n_text, gw, r2, window).sum())
    assert in_window_pairs(n_text, gh, gw, r2, text_rows=text_rows, blocks=blocks, block=block,
                           window=window) == want


def test_in_window_pairs_is_additive_over_disjoint_subsets():
    from oracle import in_window_pairs

    n_text, gh, gw, r2, block = 7, 16, 24, 50, 8
    nby, nbx = -(-gh // block), -(-gw // block)
    all_blocks = [(by, bx) for by in range(nby) for bx in range(nbx)]
    a = in_window_pairs(n_text, gh, gw, r2, text_rows=[0, 1, 2], blocks=all_blocks[::2], block=block)
    b = in_window_pairs(n_text, gh, gw, r2, text_rows=[3, 4, 5, 6], blocks=all_blocks[1::2], block=block)
    assert a + b == pair_count(n_text, gh, gw, r2)["total"]
    # an empty subset counts nothing; text rows alone count N each
    assert in_window_pairs(n_text, gh, gw, r2, text_rows=[], blocks=[], block=block) == 0
    assert in_window_pairs(n_text, gh, gw, r2, text_rows=[1, 4], blocks=[], block=block) == \
        2 * (n_text + gh * gw)
