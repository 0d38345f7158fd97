"""Pins of the oracle's patch-parallel pieces: the strip split and the Eq. 7
patch-averaged text rows (pith.science review of CLEAR, "What carries the
argument").  Each pin is fixed by arithmetic outside the oracle."""

import math

import numpy as np
import pytest
import torch

from oracle import attention_rows, strip_rows, text_rows_patch_average


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _sdpa(q, k, v):
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(a))[None, None] for a in (q, k, v))
    return torch.nn.functional.scaled_dot_product_attention(tq, tk, tv)[0, 0].numpy()


@pytest.mark.parametrize("gh,p", [(512, 8), (10, 3), (7, 7), (5, 1)])
def test_strips_partition_the_rows(gh, p):
    s = strip_rows(gh, p)
    assert s[0][0] == 0 and s[-1][1] == gh and len(s) == p
    assert all(a1 == b0 for (_, a1), (b0, _) in zip(s, s[1:]))
    h = [b - a for a, b in s]
    assert max(h) - min(h) <= 1 and min(h) >= 1


def test_one_patch_is_exact_text_attention():
    """N = 1: the single patch holds every key, so Eq. 7 is plain softmax attention."""
    n_text, gh, gw, d = 5, 4, 6, 16
    n = n_text + gh * gw
    q, k, v = (_rand((n, d), s) for s in (1, 2, 3))
    got = text_rows_patch_average(q, k, v, n_text, gh, gw, 1)
    np.testing.assert_allclose(got, _sdpa(q[:n_text], k, v), rtol=0, atol=1e-12)
    ref, _ = attention_rows(q, k, v, n_text, gh, gw, 0, range(n_text))
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_zero_queries_average_the_patch_means():
    """Q = 0: each patch's softmax is the plain mean of V over its keys (text keys plus
    the patch rows), and Eq. 7 averages those means with weight 1/N."""
    n_text, gh, gw, d, P = 3, 7, 5, 4, 3
    n = n_text + gh * gw
    q = np.zeros((n, d))
    k, v = _rand((n, d), 4), _rand((n, d), 5)
    got = text_rows_patch_average(q, k, v, n_text, gh, gw, P)
    bounds = [(p * gh // P, (p + 1) * gh // P) for p in range(P)]   # equal heights, written out
    means = [(v[:n_text].sum(0) + v[n_text + y0 * gw:n_text + y1 * gw].sum(0)) / (n_text + (y1 - y0) * gw)
             for y0, y1 in bounds]
    np.testing.assert_allclose(got, np.tile(np.mean(means, axis=0), (n_text, 1)), rtol=0, atol=1e-12)


def test_patch_average_differs_from_exact_and_weights_patches_equally():
    """With more than one patch the average is not the exact softmax: the exact one
    weights each patch by its partition function, Eq. 7 by 1/N.  Rebuilding both
    from per-patch log-sum-exp terms (computed here directly) recovers each."""
    n_text, gh, gw, d, P = 4, 6, 6, 8, 3
    n = n_text + gh * gw
    q, k, v = (_rand((n, d), s) for s in (6, 7, 8))
    got = text_rows_patch_average(q, k, v, n_text, gh, gw, P)
    s = q[:n_text] @ k.T / math.sqrt(d)
    outs, lses = [], []
    for p in range(P):
        y0, y1 = p * gh // P, (p + 1) * gh // P
        keys = np.r_[0:n_text, n_text + y0 * gw:n_text + y1 * gw]
        e = np.exp(s[:, keys])
        outs.append(e @ v[keys] / e.sum(1, keepdims=True))
        lses.append(np.log(e.sum(1)))
    np.testing.assert_allclose(got, np.mean(outs, axis=0), rtol=0, atol=1e-12)
    exact = _sdpa(q[:n_text], k, v)
    assert np.abs(got - exact).max() > 1e-3


def test_patch_average_rejects_image_rows():
    n_text, gh, gw, d = 2, 3, 3, 4
    q = k = v = np.zeros((n_text + gh * gw, d))
    with pytest.raises(ValueError):
        text_rows_patch_average(q, k, v, n_text, gh, gw, 2, rows=[n_text])
