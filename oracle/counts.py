"""Lattice-point and admitted-pair counts by enumeration.

TEST INFRASTRUCTURE ONLY (see the package docstring).

* ``lattice_count(r2)`` -- integer offsets (dy, dx) with dy^2 + dx^2 <= r2:
  the number of image keys an interior query admits.  The pith.science review
  of CLEAR ("What carries the argument") says a circular window costs about
  pi/4 of the square window it is inscribed in; these counts make that exact.
* ``pair_count`` -- admitted (query, key) pairs of a whole layer, the quantity
  behind the 99.5 % attention-compute reduction that the atlas.scime.ai summary
  of CLEAR ("Key results") and the paper's abstract quote at 8192 x 8192.
* ``pair_count_bruteforce`` -- the same, summed from the mask itself (small
  grids only); pins ``pair_count``.

Each takes ``window="square"`` for the square-window variant
(max(dy^2, dx^2) <= r2), where the counts are plain products.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["lattice_count", "pair_count", "pair_count_bruteforce"]


def _inside(dy, dx, r2, window):
    if window == "circle":
        return dy * dy + dx * dx <= r2
    if window == "square":
        return np.maximum(dy * dy, dx * dx) <= r2
    raise ValueError(f"unknown window {window!r}")


def lattice_count(r2: int, window: str = "circle") -> int:
    """#{(dy, dx) in Z^2 inside the window}, by enumerating the bounding square."""
    if r2 < 0:
        return 0
    w = math.isqrt(r2)
    d = np.arange(-w, w + 1, dtype=np.int64)
    return int(_inside(d[:, None], d[None, :], r2, window).sum())


def pair_count(n_text: int, grid_h: int, grid_w: int, r2: int, window: str = "circle") -> dict:
    """Admitted pairs of one attention layer (one batch, one head).

    The image-image part enumerates the offsets (dy, dx) of the disk and counts,
    for each, the query positions whose key at that offset lies on the grid:
    (grid_h - |dy|) * (grid_w - |dx|) when both factors are positive.
    Image queries also admit all n_text text keys; text queries admit all N keys.
    """
    img = 0
    if r2 >= 0:
        w = math.isqrt(r2)
        for dy in range(-w, w + 1):
            for dx in range(-w, w + 1):
                if _inside(dy, dx, r2, window):
                    img += max(0, grid_h - abs(dy)) * max(0, grid_w - abs(dx))
    n_img = grid_h * grid_w
    n = n_text + n_img
    img_text = n_img * n_text
    text_rows = n_text * n
    return {
        "img_img": img,
        "img_text": img_text,
        "text_rows": text_rows,
        "total": img + img_text + text_rows,
        "dense": n * n,
    }


def pair_count_bruteforce(n_text: int, grid_h: int, grid_w: int, r2: int,
                          window: str = "circle") -> int:
    """Total admitted pairs, summing the mask of every (query, key) pair."""
    from .attention import clear_mask

    n = n_text + grid_h * grid_w
    idx = np.arange(n)
    return int(clear_mask(idx, idx, n_text, grid_w, r2, window).sum())
