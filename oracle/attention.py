"""CLEAR attention forward, by definition, in float64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): the library never calls
this code.

Token order and mask
--------------------
The pith.science review of CLEAR ("Core claim") writes the mask with 1-based
indices and the text tokens first:

    M_ij = 1  if  i <= n_text  or  j <= n_text  or  (dx_ij)^2 + (dy_ij)^2 < r^2

Here indices are 0-based (text tokens are 0 .. n_text-1), the image grid is
flattened row-major after them (image token n_text + y*grid_w + x sits at row y,
column x), and the radius test is carried as a parameter ``r2``: a pair of image
tokens is admitted when dy^2 + dx^2 <= r2.  ``r2 = r*r`` is the "<=" reading;
the strict "<" the review prints is ``r2 = r*r - 1`` on the integer lattice.
A negative ``r2`` admits no image key at all.  Keys outside the grid do not
exist (no padding, no wrap-around).

Square window (a variant, not CLEAR's own mask)
-----------------------------------------------
The same review ("What carries the argument") weighs the circular window
against the square window it is inscribed in (the circle costs about pi/4 of
it).  ``window="square"`` replaces the distance test by
max(dy^2, dx^2) <= r2, i.e. max(|dy|, |dx|) <= isqrt(r2): the square of half
side r for r2 = r*r.  Everything else is unchanged.

Attention
---------
s_ij = (q_i . k_j) / sqrt(d)            (Eq. 1 / Eq. 7 of the paper, as quoted
                                          in the same review)
O_i  = sum_j M_ij exp(s_ij - m_i) v_j / sum_j M_ij exp(s_ij - m_i),
m_i  = max over admitted j of s_ij,     lse_i = m_i + log(sum_j M_ij exp(s_ij - m_i))

A row with no admitted key (only possible when n_text == 0 and r2 < 0) is
undefined; the functions raise ValueError for it.
"""

from __future__ import annotations

import math
from typing import Iterable, Optional, Sequence

import numpy as np

__all__ = [
    "WINDOWS",
    "strip_rows",
    "text_rows_patch_average",
    "clear_mask",
    "attention_rows",
    "attention_head",
    "attention",
    "in_window_pairs",
]


def _coords(idx: np.ndarray, n_text: int, grid_w: int):
    """Grid (y, x) of token indices under text-first, row-major flattening.

    The values are meaningless for text tokens (idx < n_text); callers OR the
    text condition in front of every use.
    """
    p = idx.astype(np.int64) - n_text
    return p // grid_w, p % grid_w


WINDOWS = ("circle", "square")


def clear_mask(rows: Sequence[int], cols: Sequence[int], n_text: int,
               grid_w: int, r2: int, window: str = "circle") -> np.ndarray:
    """Boolean mask M[rows, cols], evaluated element by element from its definition."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.asarray(cols, dtype=np.int64)[None, :]
    yi, xi = _coords(i, n_text, grid_w)
    yj, xj = _coords(j, n_text, grid_w)
    if window == "circle":
        near = (yi - yj) ** 2 + (xi - xj) ** 2 <= r2
    elif window == "square":
        near = np.maximum((yi - yj) ** 2, (xi - xj) ** 2) <= r2
    else:
        raise ValueError(f"unknown window {window!r}")
    return (i < n_text) | (j < n_text) | near


def _masked_softmax_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                              mask: np.ndarray, scale: float):
    """Rows of softmax(q k^T * scale, restricted to mask) @ v, in float64.

    Returns (out [R, d], lse [R], probs [R, C]).
    """
    s = (q @ k.T) * scale
    if not mask.any(axis=1).all():
        raise ValueError("a query row admits no key (n_text == 0 and r2 < 0)")
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.where(mask, np.exp(s - m), 0.0)
    l = e.sum(axis=1, keepdims=True)
    p = e / l
    return p @ v, m[:, 0] + np.log(l[:, 0]), p


def _check(n_text: int, grid_h: int, grid_w: int, r2: int, n: int):
    if n != n_text + grid_h * grid_w:
        raise ValueError(f"sequence length {n} != n_text + grid_h*grid_w = "
                         f"{n_text + grid_h * grid_w}")
    if n_text == 0 and r2 < 0:
        raise ValueError("n_text == 0 and r2 < 0: every image row is empty")


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_text: int,
                   grid_h: int, grid_w: int, r2: int, rows: Iterable[int],
                   return_probs: bool = False, window: str = "circle"):
    """Exact output rows of one (batch, head) slice, each over all N keys.

    q, k, v: [N, d] arrays (any float dtype, widened to float64).
    The mask of every requested row is evaluated against every key from the
    definition, with no candidate restriction.  Used for sampled rows at large
    sizes and as the brute-force reference at small ones.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = k.shape
    _check(n_text, grid_h, grid_w, r2, n)
    rows = np.asarray(list(rows), dtype=np.int64)
    mask = clear_mask(rows, np.arange(n), n_text, grid_w, r2, window)
    out, lse, p = _masked_softmax_attention(q[rows], k, v, mask, 1.0 / math.sqrt(d))
    if return_probs:
        return out, lse, p
    return out, lse


def _image_block_candidates(y0: int, y1: int, x0: int, x1: int, n_text: int,
                            grid_h: int, grid_w: int, r2: int) -> np.ndarray:
    """Text keys plus the image keys of the clipped box [y0-w, y1+w] x [x0-w, x1+w].

    w = isqrt(r2): a key outside that box has |dy| > w or |dx| > w, so
    dy^2 + dx^2 > r2 and max(dy^2, dx^2) > r2: either window rejects it.  The
    box only saves work; the mask is still evaluated on every candidate.
    """
    text = np.arange(n_text, dtype=np.int64)
    if r2 < 0:
        return text
    w = math.isqrt(r2)
    ys = np.arange(max(0, y0 - w), min(grid_h - 1, y1 + w) + 1)
    xs = np.arange(max(0, x0 - w), min(grid_w - 1, x1 + w) + 1)
    img = n_text + (ys[:, None] * grid_w + xs[None, :]).ravel()
    return np.concatenate([text, img])


def attention_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_text: int,
                   grid_h: int, grid_w: int, r2: int, block: int = 8,
                   text_rows: Optional[Sequence[int]] = None,
                   blocks: Optional[Sequence[tuple]] = None, window: str = "circle"):
    """CLEAR attention for one (batch, head) slice.

    q, k, v: [N, d] arrays.  Returns (out [N, d] float64, lse [N] float64).

    * Text rows (i < n_text) attend to all N keys, 64 rows at a time.
    * Image rows are processed in block x block squares of the grid; each
      square gathers the text keys plus the clipped box around it and applies
      the mask element-wise.

    ``text_rows`` / ``blocks`` restrict the work to a subset (the other rows are
    left NaN): text_rows is a list of text-row indices, blocks a list of
    (block_row, block_col) pairs.  Default: everything.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    _check(n_text, grid_h, grid_w, r2, n)
    scale = 1.0 / math.sqrt(d)
    out = np.full((n, d), np.nan)
    lse = np.full((n,), np.nan)

    trows = np.arange(n_text) if text_rows is None else np.asarray(text_rows, dtype=np.int64)
    all_keys = np.arange(n, dtype=np.int64)
    for s in range(0, len(trows), 64):
        rows = trows[s:s + 64]
        mask = clear_mask(rows, all_keys, n_text, grid_w, r2, window)
        o, l_, _ = _masked_softmax_attention(q[rows], k, v, mask, scale)
        out[rows], lse[rows] = o, l_

    nby = -(-grid_h // block)
    nbx = -(-grid_w // block)
    if blocks is None:
        blocks = [(by, bx) for by in range(nby) for bx in range(nbx)]
    for by, bx in blocks:
        y0, x0 = by * block, bx * block
        y1, x1 = min(grid_h, y0 + block) - 1, min(grid_w, x0 + block) - 1
        ys = np.arange(y0, y1 + 1)
        xs = np.arange(x0, x1 + 1)
        rows = n_text + (ys[:, None] * grid_w + xs[None, :]).ravel()
        cols = _image_block_candidates(y0, y1, x0, x1, n_text, grid_h, grid_w, r2)
        mask = clear_mask(rows, cols, n_text, grid_w, r2, window)
        o, l_, _ = _masked_softmax_attention(q[rows], k[cols], v[cols], mask, scale)
        out[rows], lse[rows] = o, l_
    return out, lse


def _one_blas_thread():
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # threadpoolctl missing: keep the library default
        pass


def _head_job(args):
    qh, kh, vh, n_text, grid_h, grid_w, r2, block, window = args
    return attention_head(qh, kh, vh, n_text, grid_h, grid_w, r2, block, window=window)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_text: int,
              grid_h: int, grid_w: int, r2: int, block: int = 8,
              workers: int = 1, window: str = "circle"):
    """CLEAR attention for [B, H, N, d] inputs.  Returns (out, lse) in float64.

    Batches and heads are independent; with ``workers > 1`` they are spread
    over a process pool.
    """
    q = np.asarray(q)
    B, H, N, d = q.shape
    jobs = [(q[b, h], k[b, h], v[b, h], n_text, grid_h, grid_w, r2, block, window)
            for b in range(B) for h in range(H)]
    if workers > 1 and len(jobs) > 1:
        import multiprocessing as mp
        # fresh interpreters: the caller may hold a GPU context, which must not be
        # forked; one BLAS thread per worker, so the pool does not oversubscribe
        with mp.get_context("spawn").Pool(min(workers, len(jobs)), initializer=_one_blas_thread) as pool:
            res = pool.map(_head_job, jobs)
    else:
        res = [_head_job(j) for j in jobs]
    out = np.stack([o for o, _ in res]).reshape(B, H, N, d)
    lse = np.stack([l_ for _, l_ in res]).reshape(B, H, N)
    return out, lse


def in_window_pairs(n_text: int, grid_h: int, grid_w: int, r2: int,
                    text_rows: Optional[Sequence[int]] = None,
                    blocks: Optional[Sequence[tuple]] = None, block: int = 8,
                    window: str = "circle") -> int:
    """Number of admitted (query, key) pairs covered by a subset of rows.

    Counts mask entries element by element over the same row subsets that
    ``attention_head`` accepts, so a timed oracle run can be converted into
    in-window FLOPs (4*d per admitted pair).
    """
    n = n_text + grid_h * grid_w
    trows = np.arange(n_text) if text_rows is None else np.asarray(text_rows)
    total = len(trows) * n
    nby, nbx = -(-grid_h // block), -(-grid_w // block)
    if blocks is None:
        blocks = [(by, bx) for by in range(nby) for bx in range(nbx)]
    for by, bx in blocks:
        y0, x0 = by * block, bx * block
        y1, x1 = min(grid_h, y0 + block) - 1, min(grid_w, x0 + block) - 1
        ys, xs = np.arange(y0, y1 + 1), np.arange(x0, x1 + 1)
        rows = n_text + (ys[:, None] * grid_w + xs[None, :]).ravel()
        cols = _image_block_candidates(y0, y1, x0, x1, n_text, grid_h, grid_w, r2)
        total += int(clear_mask(rows, cols, n_text, grid_w, r2, window).sum())
    return total


# ---------------------------------------------------------------- patch-parallel text rows

def strip_rows(grid_h: int, strips: int):
    """Image-row ranges of `strips` horizontal patches of equal height (the last
    ones one row taller when grid_h is not a multiple): patch p covers rows
    floor(p * grid_h / strips) .. floor((p + 1) * grid_h / strips) - 1."""
    if strips < 1 or strips > grid_h:
        raise ValueError("need 1 <= strips <= grid_h")
    return [(p * grid_h // strips, (p + 1) * grid_h // strips) for p in range(strips)]


def text_rows_patch_average(q: np.ndarray, k: np.ndarray, v: np.ndarray, n_text: int,
                            grid_h: int, grid_w: int, strips: int,
                            rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Text-query rows under the patch-wise approximation (Eq. 7 as quoted in the
    pith.science review of CLEAR, "What carries the argument"):

        O_text = (1 / N) * sum_p softmax(Q_text K_p^T / sqrt(d)) V_p

    with N = `strips` horizontal image patches.  Reading: patch p's keys K_p, V_p
    are all text tokens plus the image tokens of its rows (each device of a
    patch-parallel run holds the text tokens and its own patch), and the softmax
    runs over exactly those keys.  One (batch, head) slice; float64.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n, d = q.shape
    if n != n_text + grid_h * grid_w:
        raise ValueError("sequence length does not match the grid")
    trows = np.arange(n_text) if rows is None else np.asarray(rows, dtype=np.int64)
    if len(trows) and (trows.min() < 0 or trows.max() >= n_text):
        raise ValueError("rows must be text rows")
    text = np.arange(n_text, dtype=np.int64)
    acc = np.zeros((len(trows), d))
    for y0, y1 in strip_rows(grid_h, strips):
        keys = np.concatenate([text, n_text + np.arange(y0 * grid_w, y1 * grid_w, dtype=np.int64)])
        mask = np.ones((len(trows), len(keys)), dtype=bool)
        o, _, _ = _masked_softmax_attention(q[trows], k[keys], v[keys], mask, 1.0 / math.sqrt(d))
        acc += o
    return acc / strips
