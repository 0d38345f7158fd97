"""Tile lists of CLEAR's circular window, by brute force.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The GPU path groups image queries into query tiles of tile_h x tile_w grid
cells, each split into sub-tiles of sub_h x sub_w cells (one per wavefront).
For each query tile it needs the set of image keys that any of its queries
admits under the mask of the pith.science review of CLEAR ("Core claim"), as
key-row runs, cut into chunks of ``chunk`` keys, and for every chunk and
sub-tile whether the sub-tile admits any / every pair of the chunk.  This module
computes all of that from the mask, pair by pair, with no geometric shortcut.

Format (shared with the library's builders, which must match it bit for bit)
-----------------------------------------------------------------------------
* query tiles are numbered row-major: t = ty * ceil(grid_w / tile_w) + tx; tile
  t covers rows [ty*tile_h, ty*tile_h + tile_h) and columns
  [tx*tile_w, tx*tile_w + tile_w), clipped to the grid;
* ``run_offsets[t] .. run_offsets[t+1]`` index the runs of tile t; run r is
  ``runs[r] = (start, length)`` where start = ky*grid_w + kx0 is the image-token
  index (text tokens not counted) of the first key of a maximal run of admitted
  keys on key row ky.  Runs are listed by ascending ky, hence ascending start;
* concatenating a tile's runs gives its key list; it is cut into chunks of
  ``chunk`` keys (the last one may be short).  ``chunk_offsets[t] ..
  chunk_offsets[t+1]`` index the chunks of tile t;
* ``flags[c]`` (uint16) has bit s set when sub-tile s (row-major within the
  tile) admits at least one pair (query in the sub-tile and on the grid, key in
  chunk c), and bit 8+s set when the chunk holds ``chunk`` keys, the sub-tile
  has at least one query on the grid and every such pair is admitted.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = ["tile_map_bruteforce"]


def _near(qy, qx, ky, kx, r2):
    """Image-image part of the mask: [q, k] boolean matrix."""
    return (qy[:, None] - ky[None, :]) ** 2 + (qx[:, None] - kx[None, :]) ** 2 <= r2


def tile_map_bruteforce(grid_h: int, grid_w: int, r2: int, tile_h: int = 16,
                        tile_w: int = 8, sub_h: int = 4, sub_w: int = 8,
                        chunk: int = 32, tiles=None, box: bool = False) -> dict:
    """Build the tile map by evaluating the mask on every (query, key) pair.

    ``tiles`` restricts the output to a list of tile ids (offsets are then
    relative to that subset).  ``box=True`` only considers keys inside the
    tile's bounding box widened by isqrt(r2) in each direction, which cannot
    drop an admitted key (such a key has |dy| <= isqrt(r2) and |dx| <=
    isqrt(r2)); it makes large grids tractable.
    """
    if tile_h % sub_h or tile_w % sub_w:
        raise ValueError("sub-tiles must divide the tile")
    nsub_y, nsub_x = tile_h // sub_h, tile_w // sub_w
    if nsub_y * nsub_x > 8:
        raise ValueError("at most 8 sub-tiles per tile")
    nty, ntx = -(-grid_h // tile_h), -(-grid_w // tile_w)
    if tiles is None:
        tiles = range(nty * ntx)

    if not box:
        ky_all, kx_all = np.divmod(np.arange(grid_h * grid_w, dtype=np.int64), grid_w)

    run_offsets, chunk_offsets = [0], [0]
    runs, flags = [], []
    for t in tiles:
        ty, tx = divmod(t, ntx)
        y0, x0 = ty * tile_h, tx * tile_w
        y1, x1 = min(grid_h, y0 + tile_h), min(grid_w, x0 + tile_w)
        qy, qx = np.meshgrid(np.arange(y0, y1), np.arange(x0, x1), indexing="ij")
        qy, qx = qy.ravel(), qx.ravel()

        if box:
            w = math.isqrt(r2) if r2 >= 0 else -1
            if w < 0:
                ky, kx = np.zeros(0, np.int64), np.zeros(0, np.int64)
            else:
                ys = np.arange(max(0, y0 - w), min(grid_h, y1 + w))
                xs = np.arange(max(0, x0 - w), min(grid_w, x1 + w))
                ky, kx = np.meshgrid(ys, xs, indexing="ij")
                ky, kx = ky.ravel(), kx.ravel()
        else:
            ky, kx = ky_all, kx_all

        admitted = _near(qy, qx, ky, kx, r2).any(axis=0)
        keys = ky[admitted] * grid_w + kx[admitted]
        keys = np.sort(keys)

        # maximal runs of consecutive columns on one key row
        tile_runs = []
        for key in keys.tolist():
            if tile_runs:
                s, n = tile_runs[-1]
                if key == s + n and key // grid_w == s // grid_w:
                    tile_runs[-1] = (s, n + 1)
                    continue
            tile_runs.append((key, 1))
        runs.extend(tile_runs)
        run_offsets.append(len(runs))

        # chunks and their per-sub-tile flags
        kyl, kxl = np.divmod(keys, grid_w)
        nch = -(-len(keys) // chunk)
        for c in range(nch):
            cy, cx = kyl[c * chunk:(c + 1) * chunk], kxl[c * chunk:(c + 1) * chunk]
            f = 0
            for s in range(nsub_y * nsub_x):
                sy, sx = divmod(s, nsub_x)
                sel = ((qy >= y0 + sy * sub_h) & (qy < y0 + (sy + 1) * sub_h)
                       & (qx >= x0 + sx * sub_w) & (qx < x0 + (sx + 1) * sub_w))
                if not sel.any():
                    continue
                m = _near(qy[sel], qx[sel], cy, cx, r2)
                if m.any():
                    f |= 1 << s
                if len(cy) == chunk and m.all():
                    f |= 1 << (8 + s)
            flags.append(f)
        chunk_offsets.append(len(flags))

    return {
        "run_offsets": np.asarray(run_offsets, dtype=np.uint32),
        "runs": np.asarray(runs, dtype=np.uint32).reshape(-1, 2),
        "chunk_offsets": np.asarray(chunk_offsets, dtype=np.uint32),
        "flags": np.asarray(flags, dtype=np.uint16),
    }
