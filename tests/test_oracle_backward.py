"""Pins of the oracle's backward (dQ, dK, dV of CLEAR attention).

Each pin comes from outside the backward's own formulas: finite differences of
the (separately pinned) forward oracle, torch autograd through a dense masked
softmax whose mask is written out here by loops, closed forms of special cases,
and invariants of softmax attention.
"""

import math

import numpy as np
import pytest
import torch

from oracle import attention_backward, attention_backward_head, attention_head, key_grads


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _case(n_text, gh, gw, d, seed):
    n = n_text + gh * gw
    return [_rand((n, d), seed + i) for i in range(4)]


def _loop_mask(n_text, gh, gw, r2, window):
    n = n_text + gh * gw
    m = np.zeros((n, n), dtype=bool)
    for i in range(n):
        for j in range(n):
            if i < n_text or j < n_text:
                m[i, j] = True
                continue
            yi, xi = divmod(i - n_text, gw)
            yj, xj = divmod(j - n_text, gw)
            dy2, dx2 = (yi - yj) ** 2, (xi - xj) ** 2
            m[i, j] = (dy2 + dx2 <= r2) if window == "circle" else (max(dy2, dx2) <= r2)
    return m


def _autograd(q, k, v, do, mask):
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    s = (tq @ tk.T) / math.sqrt(q.shape[1])
    if mask is not None:
        s = s.masked_fill(~torch.from_numpy(mask), float("-inf"))
    o = torch.softmax(s, dim=1) @ tv
    o.backward(torch.tensor(do))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("n_text,gh,gw,r2,window", [
    (3, 5, 7, 4, "circle"), (0, 6, 4, 2, "circle"), (5, 4, 4, 0, "circle"),
    (2, 5, 6, 5, "square"), (4, 3, 9, -1, "circle"),
])
def test_directional_finite_differences_of_the_forward(n_text, gh, gw, r2, window):
    """d/dt L(x + t u) at t = 0, with L = sum(dO * O) from the forward oracle,
    equals <grad, u> for random directions u (central differences, h = 1e-5)."""
    d = 8
    q, k, v, do = _case(n_text, gh, gw, d, 10)
    dq, dk, dv = attention_backward_head(q, k, v, do, n_text, gh, gw, r2, block=4, window=window)

    def loss(a, b, c):
        return float((attention_head(a, b, c, n_text, gh, gw, r2, block=4, window=window)[0] * do).sum())

    rng = np.random.default_rng(3)
    h = 1e-5
    for _ in range(3):
        uq, uk, uv = (rng.standard_normal(q.shape) for _ in range(3))
        fd = (loss(q + h * uq, k + h * uk, v + h * uv) - loss(q - h * uq, k - h * uk, v - h * uv)) / (2 * h)
        an = float((dq * uq).sum() + (dk * uk).sum() + (dv * uv).sum())
        assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (fd, an)


def test_elementwise_finite_differences_tiny():
    """Every gradient element of a 2 + 3x3 case against a central difference."""
    n_text, gh, gw, d, r2 = 2, 3, 3, 4, 1
    q, k, v, do = _case(n_text, gh, gw, d, 20)
    grads = attention_backward_head(q, k, v, do, n_text, gh, gw, r2, block=2)

    def loss(x):
        return float((attention_head(*x, n_text, gh, gw, r2, block=2)[0] * do).sum())

    h = 1e-6
    for t in range(3):
        for idx in np.ndindex(q.shape):
            plus = [q.copy(), k.copy(), v.copy()]
            minus = [q.copy(), k.copy(), v.copy()]
            plus[t][idx] += h
            minus[t][idx] -= h
            fd = (loss(plus) - loss(minus)) / (2 * h)
            assert abs(fd - grads[t][idx]) <= 1e-7, (t, idx, fd, grads[t][idx])


@pytest.mark.parametrize("n_text,gh,gw,r2,window", [
    (4, 6, 8, 5, "circle"), (0, 7, 5, 9, "circle"), (6, 5, 5, 2, "square"), (3, 8, 3, 16, "circle"),
])
def test_matches_autograd_of_dense_masked_softmax(n_text, gh, gw, r2, window):
    q, k, v, do = _case(n_text, gh, gw, 16, 30)
    got = attention_backward_head(q, k, v, do, n_text, gh, gw, r2, block=4, window=window)
    ref = _autograd(q, k, v, do, _loop_mask(n_text, gh, gw, r2, window))
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=0, atol=1e-12)


def test_beyond_the_diagonal_is_dense_attention_gradient():
    n_text, gh, gw = 3, 4, 6
    q, k, v, do = _case(n_text, gh, gw, 8, 40)
    ref = _autograd(q, k, v, do, None)
    for r2 in ((gh - 1) ** 2 + (gw - 1) ** 2, 10 ** 6):
        got = attention_backward_head(q, k, v, do, n_text, gh, gw, r2, block=4)
        for g, r in zip(got, ref):
            np.testing.assert_allclose(g, r, rtol=0, atol=1e-12)


def test_radius_zero_without_text_passes_dout_to_v_exactly():
    """Each row admits only itself: O = V, so dV = dO and dQ = dK = 0, exactly."""
    gh, gw, d = 5, 4, 8
    q, k, v, do = _case(0, gh, gw, d, 50)
    dq, dk, dv = attention_backward_head(q, k, v, do, 0, gh, gw, 0, block=4)
    assert np.array_equal(dv, do)
    assert not dq.any() and not dk.any()


@pytest.mark.parametrize("window", ["circle", "square"])
def test_softmax_invariants(window):
    """Shifting every key by one vector changes each row's logits by a constant,
    so sum_j dK_j = 0; rows of P sum to one, so sum_j dV_j = sum_i dO_i; a
    constant V makes O constant, so dQ = dK = 0."""
    n_text, gh, gw, d, r2 = 3, 6, 7, 8, 4
    q, k, v, do = _case(n_text, gh, gw, d, 60)
    dq, dk, dv = attention_backward_head(q, k, v, do, n_text, gh, gw, r2, block=4, window=window)
    np.testing.assert_allclose(dk.sum(0), 0.0, atol=1e-12)
    np.testing.assert_allclose(dv.sum(0), do.sum(0), rtol=0, atol=1e-12)
    vc = np.tile(_rand((1, d), 61), (len(v), 1))
    dq, dk, _ = attention_backward_head(q, k, vc, do, n_text, gh, gw, r2, block=4, window=window)
    assert np.abs(dq).max() <= 1e-12 and np.abs(dk).max() <= 1e-12


def test_text_permutation_equivariance():
    """Permuting the text tokens permutes their gradient rows and leaves the image rows."""
    n_text, gh, gw, d, r2 = 5, 4, 5, 8, 2
    q, k, v, do = _case(n_text, gh, gw, d, 70)
    ref = attention_backward_head(q, k, v, do, n_text, gh, gw, r2, block=4)
    perm = np.r_[np.random.default_rng(1).permutation(n_text), n_text:len(q)]
    got = attention_backward_head(q[perm], k[perm], v[perm], do[perm], n_text, gh, gw, r2, block=4)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r[perm], rtol=0, atol=1e-12)


def test_subsets_reproduce_the_full_backward():
    """dq rows of chosen groups and dk / dv of chosen keys equal the full result."""
    n_text, gh, gw, d, r2 = 4, 12, 10, 8, 9
    q, k, v, do = _case(n_text, gh, gw, d, 80)
    dq, dk, dv = attention_backward_head(q, k, v, do, n_text, gh, gw, r2, block=4)
    dq_s, _, _ = attention_backward_head(q, k, v, do, n_text, gh, gw, r2, block=4,
                                         text_rows=[1, 3], blocks=[(1, 2)])
    rows = [1, 3] + [n_text + y * gw + x for y in range(4, 8) for x in range(8, 10)]
    np.testing.assert_allclose(dq_s[rows], dq[rows], rtol=0, atol=1e-12)
    keys = [0, n_text + 0, n_text + 5 * gw + 3, n_text + gh * gw - 1]
    dk_s, dv_s = key_grads(q, k, v, do, n_text, gh, gw, r2, keys, block=4)
    np.testing.assert_allclose(dk_s, dk[keys], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv_s, dv[keys], rtol=0, atol=1e-12)
    dk_i, dv_i = key_grads(q, k, v, do, n_text, gh, gw, r2, keys[1:], block=4)
    np.testing.assert_allclose(dk_i, dk[keys[1:]], rtol=0, atol=1e-12)
    np.testing.assert_allclose(dv_i, dv[keys[1:]], rtol=0, atol=1e-12)


def test_batched_driver_matches_per_head():
    n_text, gh, gw, d, r2 = 2, 4, 4, 8, 2
    rng = np.random.default_rng(90)
    q, k, v, do = (rng.standard_normal((2, 2, n_text + gh * gw, d)) for _ in range(4))
    got = attention_backward(q, k, v, do, n_text, gh, gw, r2, block=4)
    for b in range(2):
        for h in range(2):
            ref = attention_backward_head(q[b, h], k[b, h], v[b, h], do[b, h], n_text, gh, gw, r2, block=4)
            for g, r in zip(got, ref):
                np.testing.assert_array_equal(g[b, h], r)
