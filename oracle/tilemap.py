"""Tile lists of CLEAR's circular window (and of the square variant), by brute force.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The GPU path groups image queries into query tiles of tile_h x tile_w grid
cells, each split into sub-tiles of sub_h x sub_w cells (one per wavefront),
and image keys into key tiles of key_h x key_w cells.  For each query tile it
needs the key tiles that at least one of its sub-tiles touches under the mask of
the pith.science review of CLEAR ("Core claim"), and for every listed key tile
and sub-tile whether the sub-tile admits some / every pair.  This module
computes that from the mask, pair by pair, with no geometric shortcut.

Format (shared with the library's builders, which must match it bit for bit)
-----------------------------------------------------------------------------
* query tiles are numbered row-major: t = ty * ceil(grid_w / tile_w) + tx; tile
  t covers rows [ty*tile_h, ty*tile_h + tile_h) and columns
  [tx*tile_w, tx*tile_w + tile_w), clipped to the grid; sub-tiles are numbered
  row-major within their tile;
* key tiles are numbered row-major the same way with key_h x key_w cells:
  id = kty * ceil(grid_w / key_w) + ktx;
* ``offsets[t] .. offsets[t+1]`` index the entries of query tile t; entry e is
  ``key_tiles[e]`` (ascending ids within a tile) with ``flags[e]`` (uint16):
  bit s set when sub-tile s admits at least one pair (query cell of the
  sub-tile on the grid, key cell of the key tile on the grid); bit 8+s set when
  in addition the key tile lies entirely on the grid, the sub-tile has a cell on
  the grid, and every such pair is admitted.  A key tile is listed when some bit
  0..7 is set.

``window="square"`` uses the square-window predicate max(dy^2, dx^2) <= r2 of
``oracle.attention.clear_mask`` instead.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["tile_map_bruteforce"]


def _near(qy, qx, ky, kx, r2, window="circle"):
    """Image-image part of the mask: [q, k] boolean matrix."""
    dy2 = (qy[:, None] - ky[None, :]) ** 2
    dx2 = (qx[:, None] - kx[None, :]) ** 2
    if window == "circle":
        return dy2 + dx2 <= r2
    if window == "square":
        return np.maximum(dy2, dx2) <= r2
    raise ValueError(f"unknown window {window!r}")


def _cells(y0, x0, h, w, grid_h, grid_w):
    ys = np.arange(y0, min(grid_h, y0 + h))
    xs = np.arange(x0, min(grid_w, x0 + w))
    yy, xx = np.meshgrid(ys, xs, indexing="ij")
    return yy.ravel(), xx.ravel()


def tile_map_bruteforce(grid_h: int, grid_w: int, r2: int, tile_h: int = 16,
                        tile_w: int = 8, sub_h: int = 4, sub_w: int = 8,
                        key_h: int = 4, key_w: int = 8, tiles=None,
                        box: bool = False, window: str = "circle") -> dict:
    """Build the tile map by evaluating the mask on every (query, key) pair.

    ``tiles`` restricts the output to a list of query-tile ids (offsets are then
    relative to that subset).  ``box=True`` only considers key tiles that
    intersect the query tile's bounding box widened by isqrt(r2) in each
    direction; a key tile outside that box holds no admitted key (every such key
    has |dy| > isqrt(r2) or |dx| > isqrt(r2), outside either window), so nothing
    changes but the time.
    """
    if tile_h % sub_h or tile_w % sub_w:
        raise ValueError("sub-tiles must divide the tile")
    nsy, nsx = tile_h // sub_h, tile_w // sub_w
    if nsy * nsx > 8:
        raise ValueError("at most 8 sub-tiles per tile")
    nty, ntx = -(-grid_h // tile_h), -(-grid_w // tile_w)
    nky, nkx = -(-grid_h // key_h), -(-grid_w // key_w)
    if tiles is None:
        tiles = range(nty * ntx)

    offsets, key_tiles, flags = [0], [], []
    for t in tiles:
        ty, tx = divmod(t, ntx)
        y0, x0 = ty * tile_h, tx * tile_w
        subs = []
        for s in range(nsy * nsx):
            sy, sx = divmod(s, nsx)
            qy, qx = _cells(y0 + sy * sub_h, x0 + sx * sub_w, sub_h, sub_w, grid_h, grid_w)
            subs.append((qy, qx))
        if box:
            w = math.isqrt(r2) if r2 >= 0 else -1
            if w < 0:
                cand = []
            else:
                y1, x1 = min(grid_h, y0 + tile_h) - 1, min(grid_w, x0 + tile_w) - 1
                kys = range(max(0, y0 - w) // key_h, min(grid_h - 1, y1 + w) // key_h + 1)
                kxs = range(max(0, x0 - w) // key_w, min(grid_w - 1, x1 + w) // key_w + 1)
                cand = [ky * nkx + kx for ky in kys for kx in kxs]
        else:
            cand = range(nky * nkx)
        for kt in cand:
            kty, ktx = divmod(kt, nkx)
            ky, kx = _cells(kty * key_h, ktx * key_w, key_h, key_w, grid_h, grid_w)
            on_grid = len(ky) == key_h * key_w
            f = 0
            for s, (qy, qx) in enumerate(subs):
                if len(qy) == 0:
                    continue
                m = _near(qy, qx, ky, kx, r2, window)
                if m.any():
                    f |= 1 << s
                    if on_grid and m.all():
                        f |= 1 << (8 + s)
            if f & 0xFF:
                key_tiles.append(kt)
                flags.append(f)
        offsets.append(len(key_tiles))

    return {
        "offsets": np.asarray(offsets, dtype=np.uint32),
        "key_tiles": np.asarray(key_tiles, dtype=np.uint32),
        "flags": np.asarray(flags, dtype=np.uint16),
    }
