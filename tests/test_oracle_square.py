"""Pins of the oracle's square-window variant (max(dy^2, dx^2) <= r2).

The square window is the one the circle is inscribed in; the pith.science
review of CLEAR ("What carries the argument") prices the circular window at
about pi/4 of it.  Each pin below comes from outside the oracle: a closed form,
a library routine, set inclusion, or an independent summation method.
"""

import math

import numpy as np
import pytest
import torch

from oracle import (attention_head, attention_rows, clear_mask, lattice_count, pair_count,
                    pair_count_bruteforce, tile_map_bruteforce)


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a))[None, None] for a in (q, k, v))
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, 0].numpy()


def test_square_lattice_count_is_a_square():
    """(2 * isqrt(r2) + 1)^2 offsets for every r2 >= 0, none for r2 < 0."""
    assert lattice_count(-1, "square") == 0
    for r2 in range(0, 1200):
        assert lattice_count(r2, "square") == (2 * math.isqrt(r2) + 1) ** 2
    assert [lattice_count(r * r, "square") for r in (4, 8, 16, 32)] == [81, 289, 1089, 4225]


def test_circle_over_square_is_the_pages_pi_over_4():
    """The ratio the review quotes, taken from the two windows' own counts."""
    ratio = {r: lattice_count(r * r) / lattice_count(r * r, "square") for r in (8, 16, 32, 400)}
    assert round(ratio[8], 2) == 0.68 and round(ratio[16], 2) == 0.73 and round(ratio[32], 2) == 0.76
    assert abs(ratio[400] - math.pi / 4) < 0.01


def _axis_sum(g, w):
    """sum over |d| <= w of the query positions whose key at offset d is on an axis of length g."""
    return sum(max(0, g - abs(d)) for d in range(-w, w + 1))


@pytest.mark.parametrize("n_text,gh,gw,r2", [(0, 5, 5, 0), (3, 4, 9, 1), (2, 7, 3, 4), (5, 6, 6, 5),
                                             (1, 8, 5, 13), (4, 5, 7, -1), (2, 4, 4, 1000)])
def test_square_pair_count_is_a_separable_product(n_text, gh, gw, r2):
    """Image-image pairs factor into one sum per axis; totals equal the mask's own sum."""
    pc = pair_count(n_text, gh, gw, r2, "square")
    w = math.isqrt(r2) if r2 >= 0 else -1
    expect = _axis_sum(gh, w) * _axis_sum(gw, w) if w >= 0 else 0
    assert pc["img_img"] == expect
    assert pc["total"] == pair_count_bruteforce(n_text, gh, gw, r2, "square")


def test_square_mask_sits_between_two_circles():
    """circle(r2) is inside square(r2), which is inside circle(2 r2)."""
    n_text, gh, gw = 3, 9, 11
    idx = np.arange(n_text + gh * gw)
    for r2 in (0, 1, 2, 4, 9, 10, 30):
        c = clear_mask(idx, idx, n_text, gw, r2)
        s = clear_mask(idx, idx, n_text, gw, r2, "square")
        c2 = clear_mask(idx, idx, n_text, gw, 2 * r2)
        assert not (c & ~s).any() and not (s & ~c2).any()
        w = math.isqrt(r2)
        assert (s & ~c).any() == (2 * w * w > r2)  # the square's corners lie outside the circle


@pytest.mark.parametrize("n_text,gh,gw,d", [(3, 5, 7, 16), (0, 4, 4, 8)])
def test_square_beyond_the_grid_is_dense_attention(n_text, gh, gw, d):
    n = n_text + gh * gw
    q, k, v = (_rand((n, d), s) for s in (1, 2, 3))
    for r2 in (max(gh - 1, gw - 1) ** 2, 10 ** 6):
        out, _ = attention_head(q, k, v, n_text, gh, gw, r2, block=4, window="square")
        np.testing.assert_allclose(out, _sdpa(q, k, v), rtol=0, atol=1e-12)


def test_square_radius_zero_returns_v_exactly():
    gh, gw, d = 6, 5, 16
    q, k, v = (_rand((gh * gw, d), s) for s in (4, 5, 6))
    out, _ = attention_head(q, k, v, 0, gh, gw, 0, block=4, window="square")
    assert np.array_equal(out, v)


@pytest.mark.parametrize("r2", [1, 4, 9, 16])
def test_zero_queries_average_v_over_the_clipped_square(r2):
    """Q = 0 gives equal logits, so each image row is the mean of V over text keys
    plus the clipped square; the square's sum comes from 2-D prefix sums."""
    n_text, gh, gw, d = 2, 7, 9, 4
    n = n_text + gh * gw
    q = np.zeros((n, d))
    k, v = _rand((n, d), 7), _rand((n, d), 8)
    out, _ = attention_head(q, k, v, n_text, gh, gw, r2, block=4, window="square")
    w = math.isqrt(r2)
    img = v[n_text:].reshape(gh, gw, d)
    pre = np.zeros((gh + 1, gw + 1, d))
    pre[1:, 1:] = img.cumsum(0).cumsum(1)
    tsum = v[:n_text].sum(0)
    for y in range(gh):
        for x in range(gw):
            y0, y1, x0, x1 = max(0, y - w), min(gh, y + w + 1), max(0, x - w), min(gw, x + w + 1)
            box = pre[y1, x1] - pre[y0, x1] - pre[y1, x0] + pre[y0, x0]
            cnt = (y1 - y0) * (x1 - x0) + n_text
            np.testing.assert_allclose(out[n_text + y * gw + x], (box + tsum) / cnt, rtol=0, atol=1e-12)


def test_square_transpose_and_flip_symmetry():
    n_text, gh, gw, d, r2 = 3, 5, 8, 8, 5
    n = n_text + gh * gw
    q, k, v = (_rand((n, d), s) for s in (9, 10, 11))

    def perm(order):  # image tokens reordered, text first unchanged
        return np.concatenate([np.arange(n_text), n_text + order.ravel()])

    grid = np.arange(gh * gw).reshape(gh, gw)
    ref, _ = attention_head(q, k, v, n_text, gh, gw, r2, block=4, window="square")
    p = perm(grid.T)  # transposed grid: gw x gh
    out_t, _ = attention_head(q[p], k[p], v[p], n_text, gw, gh, r2, block=4, window="square")
    np.testing.assert_allclose(out_t, ref[p], rtol=0, atol=1e-12)
    p = perm(grid[:, ::-1])
    out_f, _ = attention_head(q[p], k[p], v[p], n_text, gh, gw, r2, block=4, window="square")
    np.testing.assert_allclose(out_f, ref[p], rtol=0, atol=1e-12)


def test_square_rows_match_blocked_driver():
    n_text, gh, gw, d, r2 = 4, 9, 10, 8, 8
    n = n_text + gh * gw
    q, k, v = (_rand((n, d), s) for s in (12, 13, 14))
    out, lse = attention_head(q, k, v, n_text, gh, gw, r2, block=4, window="square")
    rows = list(range(n))
    o2, l2 = attention_rows(q, k, v, n_text, gh, gw, r2, rows, window="square")
    np.testing.assert_allclose(out, o2, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, l2, rtol=0, atol=1e-12)


def test_square_tile_flags_follow_the_interval_rule():
    """The brute-force tile map agrees with the per-axis interval rule written out
    here: touched iff both axes have an offset within isqrt(r2); full iff every
    offset on both axes is."""
    gh, gw, th, tw, sh, sw, kh, kw = 13, 17, 4, 4, 2, 4, 2, 4
    for r2 in (0, 1, 4, 9, 26):
        tm = tile_map_bruteforce(gh, gw, r2, th, tw, sh, sw, kh, kw, window="square")
        w = math.isqrt(r2)
        ntx, nkx = -(-gw // tw), -(-gw // kw)
        for t in range(len(tm["offsets"]) - 1):
            ty, tx = divmod(t, ntx)
            listed = dict(zip(tm["key_tiles"][tm["offsets"][t]:tm["offsets"][t + 1]].tolist(),
                              tm["flags"][tm["offsets"][t]:tm["offsets"][t + 1]].tolist()))
            for kt in range(-(-gh // kh) * nkx):
                ky, kx = divmod(kt, nkx)
                kys = range(ky * kh, min(gh, ky * kh + kh))
                kxs = range(kx * kw, min(gw, kx * kw + kw))
                f = 0
                for s in range((th // sh) * (tw // sw)):
                    sy, sx = divmod(s, tw // sw)
                    qys = range(ty * th + sy * sh, min(gh, ty * th + sy * sh + sh))
                    qxs = range(tx * tw + sx * sw, min(gw, tx * tw + sx * sw + sw))
                    if not len(qys) or not len(qxs):
                        continue
                    dy = [abs(a - b) for a in qys for b in kys]
                    dx = [abs(a - b) for a in qxs for b in kxs]
                    if min(dy) <= w and min(dx) <= w:
                        f |= 1 << s
                        if len(kys) == kh and len(kxs) == kw and max(dy) <= w and max(dx) <= w:
                            f |= 1 << (8 + s)
                assert listed.get(kt, 0) == f, (r2, t, kt)
