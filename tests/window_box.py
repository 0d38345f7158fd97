"""Exact reference rows of image queries, from the window box around each cell.

Every key an image query at (y, x) admits lies in the box [y - w, y + w] x
[x - w, x + w] clipped to the grid, w = isqrt(r2): a key outside it has
|dy| > w or |dx| > w, so dy^2 + dx^2 > r2 and max(dy^2, dx^2) > r2.  The box,
with the text tokens in front, is therefore a CLEAR problem of its own in which
the query admits exactly the keys it admits in the full grid, and the oracle
evaluated on it gives that row of the full problem.  Grids too large to copy to
the host are checked this way, row by row.
"""

import math

import numpy as np
import torch

from oracle import attention_rows


def box_reference(q, k, v, n_text, gh, gw, r2, cells, window="circle"):
    """q, k, v: [N, d] tensors of one (batch, head), on any device; cells:
    image cells (y, x).  Returns the cells' token indices and the oracle's rows
    (float64, one per cell)."""
    w = math.isqrt(r2)
    rows, refs = [], []
    for y, x in cells:
        y0, y1 = max(0, y - w), min(gh - 1, y + w)
        x0, x1 = max(0, x - w), min(gw - 1, x + w)
        bh, bw = y1 - y0 + 1, x1 - x0 + 1
        cells_tok = n_text + torch.arange(y0, y1 + 1).view(-1, 1) * gw + torch.arange(x0, x1 + 1).view(1, -1)
        idx = torch.cat([torch.arange(n_text), cells_tok.reshape(-1)]).to(k.device)
        ks = k[idx].double().cpu().numpy()
        vs = v[idx].double().cpu().numpy()
        row = n_text + y * gw + x
        local = n_text + (y - y0) * bw + (x - x0)
        qs = np.zeros_like(ks)
        qs[local] = q[row].double().cpu().numpy()
        ref, _ = attention_rows(qs, ks, vs, n_text, bh, bw, r2, [local], window=window)
        rows.append(row)
        refs.append(ref[0])
    return rows, np.stack(refs)
