"""Gradients of CLEAR attention, by the chain rule through its definition, in
float64 on the CPU.

TEST INFRASTRUCTURE ONLY (see the package docstring): the library never calls
this code.

The forward is the masked softmax attention of ``oracle.attention`` (the mask of
the pith.science review of CLEAR, "Core claim"; logits scaled by 1/sqrt(d)).
The backward is the step that follows it in the paper's attention-only
distillation fine-tuning (the same review, "What carries the argument": only
the attention layers are trained).  For a loss L with dO = dL/dO:

    P_ij  = M_ij exp(s_ij - lse_i)           (row softmax over admitted keys)
    dV_j  = sum_i P_ij dO_i                  (O_i = sum_j P_ij v_j)
    dP_ij = dO_i . v_j
    dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik)  (Jacobian of a row softmax)
    dQ_i  = sum_j dS_ij k_j / sqrt(d)        (s_ij = q_i . k_j / sqrt(d))
    dK_j  = sum_i dS_ij q_i / sqrt(d)

Pairs outside the mask have P_ij = 0 and contribute nothing.  The rows are
visited in the same groups as the forward oracle (text rows against every key;
image rows in square blocks against the text keys plus the clipped box around
the block, with the mask evaluated element by element); dK and dV receive each
group's contribution by addition.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

from .attention import _check, _image_block_candidates, clear_mask

__all__ = ["attention_backward_head", "attention_backward", "key_grads"]


def _group_grads(q, k, v, dout, rows, cols, mask, scale):
    """(dS, P) of one group of query rows against candidate keys `cols`."""
    s = (q[rows] @ k[cols].T) * scale
    if not mask.any(axis=1).all():
        raise ValueError("a query row admits no key (n_text == 0 and r2 < 0)")
    s = np.where(mask, s, -np.inf)
    m = s.max(axis=1, keepdims=True)
    e = np.where(mask, np.exp(s - m), 0.0)
    p = e / e.sum(axis=1, keepdims=True)
    dp = dout[rows] @ v[cols].T
    ds = p * (dp - (p * dp).sum(axis=1, keepdims=True))
    return ds, p


def _groups(n_text, grid_h, grid_w, r2, block, text_rows, blocks, window):
    """(rows, cols, mask) for the chosen query groups, as the forward oracle forms them."""
    n = n_text + grid_h * grid_w
    trows = np.arange(n_text) if text_rows is None else np.asarray(text_rows, dtype=np.int64)
    all_keys = np.arange(n, dtype=np.int64)
    for s in range(0, len(trows), 64):
        rows = trows[s:s + 64]
        yield rows, all_keys, clear_mask(rows, all_keys, n_text, grid_w, r2, window)
    nby, nbx = -(-grid_h // block), -(-grid_w // block)
    if blocks is None:
        blocks = [(by, bx) for by in range(nby) for bx in range(nbx)]
    for by, bx in blocks:
        y0, x0 = by * block, bx * block
        y1, x1 = min(grid_h, y0 + block) - 1, min(grid_w, x0 + block) - 1
        ys, xs = np.arange(y0, y1 + 1), np.arange(x0, x1 + 1)
        rows = n_text + (ys[:, None] * grid_w + xs[None, :]).ravel()
        cols = _image_block_candidates(y0, y1, x0, x1, n_text, grid_h, grid_w, r2)
        yield rows, cols, clear_mask(rows, cols, n_text, grid_w, r2, window)


def attention_backward_head(q, k, v, dout, n_text: int, grid_h: int, grid_w: int, r2: int,
                            block: int = 8, text_rows: Optional[Sequence[int]] = None,
                            blocks: Optional[Sequence[tuple]] = None, window: str = "circle"):
    """(dq, dk, dv) of one (batch, head) slice for upstream gradient `dout`.

    q, k, v, dout: [N, d].  With ``text_rows`` / ``blocks`` (as in
    ``attention_head``) only those query rows are visited: their dq rows are
    exact, the other dq rows are NaN, and dk / dv hold only the contributions of
    the visited rows.
    """
    q, k, v, dout = (np.asarray(a, dtype=np.float64) for a in (q, k, v, dout))
    n, d = q.shape
    _check(n_text, grid_h, grid_w, r2, n)
    scale = 1.0 / math.sqrt(d)
    full = text_rows is None and blocks is None
    dq = np.zeros((n, d)) if full else np.full((n, d), np.nan)
    dk = np.zeros((n, d))
    dv = np.zeros((n, d))
    for rows, cols, mask in _groups(n_text, grid_h, grid_w, r2, block, text_rows, blocks, window):
        ds, p = _group_grads(q, k, v, dout, rows, cols, mask, scale)
        dq[rows] = (ds @ k[cols]) * scale
        dk[cols] += (ds.T @ q[rows]) * scale   # cols are distinct within a group
        dv[cols] += p.T @ dout[rows]
    return dq, dk, dv


def key_grads(q, k, v, dout, n_text: int, grid_h: int, grid_w: int, r2: int,
              keys: Sequence[int], block: int = 8, window: str = "circle"):
    """Exact (dk, dv) rows for the chosen key tokens only, for sampled checks at
    sizes where the whole backward is too slow.

    Visits every text row and every image block that holds a query admitting
    one of the keys (a text key is admitted by every query, so then all rows;
    an image key at (y, x) only by queries in the box y +- w, x +- w with
    w = isqrt(r2), besides the text rows).  Returns arrays [len(keys), d].
    """
    keys = np.asarray(keys, dtype=np.int64)
    if (keys < n_text).any():
        blocks = None
    else:
        w = math.isqrt(r2) if r2 >= 0 else -1
        need = set()
        for j in keys:
            y, x = divmod(int(j) - n_text, grid_w)
            if w < 0:
                continue
            for by in range(max(0, y - w) // block, min(grid_h - 1, y + w) // block + 1):
                for bx in range(max(0, x - w) // block, min(grid_w - 1, x + w) // block + 1):
                    need.add((by, bx))
        blocks = sorted(need)
    _, dk, dv = attention_backward_head(q, k, v, dout, n_text, grid_h, grid_w, r2, block,
                                        text_rows=np.arange(n_text), blocks=blocks, window=window)
    return dk[keys], dv[keys]


def _head_job(args):
    qh, kh, vh, dh, n_text, grid_h, grid_w, r2, block, window = args
    return attention_backward_head(qh, kh, vh, dh, n_text, grid_h, grid_w, r2, block, window=window)


def attention_backward(q, k, v, dout, n_text: int, grid_h: int, grid_w: int, r2: int,
                       block: int = 8, workers: int = 1, window: str = "circle"):
    """(dq, dk, dv) for [B, H, N, d] inputs, float64; heads spread over a
    process pool when ``workers > 1``."""
    q = np.asarray(q)
    B, H, N, d = q.shape
    jobs = [(q[b, h], k[b, h], v[b, h], dout[b, h], n_text, grid_h, grid_w, r2, block, window)
            for b in range(B) for h in range(H)]
    if workers > 1 and len(jobs) > 1:
        import multiprocessing as mp
        with mp.get_context("spawn").Pool(min(workers, len(jobs))) as pool:
            res = pool.map(_head_job, jobs)
    else:
        res = [_head_job(j) for j in jobs]
    return tuple(np.stack([r[i] for r in res]).reshape(B, H, N, d) for i in range(3))
