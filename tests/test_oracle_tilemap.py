"""Pins of the oracle's brute-force tile map."""

import math

import numpy as np
import pytest

from oracle import pair_count, tile_map_bruteforce


def _disk_keys(gh, gw, r2, y, x):
    """Image keys (y, x) of the window around a cell, built per key row from
    |dx| <= isqrt(r2 - dy^2) (no mask evaluation)."""
    out = set()
    if r2 < 0:
        return out
    w = math.isqrt(r2)
    for dy in range(-w, w + 1):
        ky = y + dy
        if 0 <= ky < gh:
            half = math.isqrt(r2 - dy * dy)
            for kx in range(max(0, x - half), min(gw - 1, x + half) + 1):
                out.add((ky, kx))
    return out


def _entries(tm, t):
    a, b = tm["offsets"][t], tm["offsets"][t + 1]
    return tm["key_tiles"][a:b].tolist(), tm["flags"][a:b].tolist()


def test_hand_derived_3x3_case():
    """grid 3x3, r2 = 1, query tiles 2x2 split into 1x2 sub-tiles, key tiles 2x2.

    Key tiles: 0 = rows 0-1 cols 0-1, 1 = rows 0-1 col 2, 2 = row 2 cols 0-1,
    3 = (2,2); only key tile 0 lies wholly on the grid.
    Query tile 0 = rows 0-1 cols 0-1 (sub-tile 0 = row 0, sub-tile 1 = row 1):
      kt0: (0,0)-(0,0) and (1,0)-(1,0) admitted, (0,0)-(1,1) and (1,0)-(0,1)
           have d2 = 2: touched by both, full for neither -> 0x3;
      kt1: (0,1)-(0,2) and (1,1)-(1,2) admitted -> 0x3;
      kt2: row 0 is 2 rows away (d2 >= 4); (1,0)-(2,0) admitted -> 0x2;
      kt3: nearest pairs (1,1)-(2,2) d2 = 2, (0,1)-(2,2) d2 = 5 -> not listed.
    Query tile 1 = (0,2), (1,2): kt0 -> 0x3 ((0,2)-(0,1), (1,2)-(1,1));
      kt1 -> 0x3 (every pair admitted, but kt1 is partly off the grid);
      kt2: nearest (1,2)-(2,1) d2 = 2 -> not listed; kt3: (1,2)-(2,2) -> 0x2.
    Query tile 2 = (2,0), (2,1) (sub-tile 1 is off the grid): kt0 via
      (2,0)-(1,0) -> 0x1; kt1: nearest (2,1)-(1,2) d2 = 2 -> not listed;
      kt2 -> 0x1; kt3 via (2,1)-(2,2) -> 0x1.
    Query tile 3 = (2,2): kt0 nearest (1,1) d2 = 2 -> not listed; kt1 via
      (1,2), kt2 via (2,1), kt3 via itself -> 0x1 each.
    """
    tm = tile_map_bruteforce(3, 3, 1, tile_h=2, tile_w=2, sub_h=1, sub_w=2, key_h=2, key_w=2)
    assert tm["offsets"].tolist() == [0, 3, 6, 9, 12]
    assert tm["key_tiles"].tolist() == [0, 1, 2, 0, 1, 3, 0, 2, 3, 1, 2, 3]
    assert tm["flags"].tolist() == [0x3, 0x3, 0x2, 0x3, 0x3, 0x2, 0x1, 0x1, 0x1, 0x1, 0x1, 0x1]


def test_hand_derived_full_flags():
    """grid 4x4, r2 = 8, query tile 2x2 with 1x2 sub-tiles, key tiles 2x2.
    Sub-tile 0 of query tile 0 = (0,0), (0,1); key tile 0 = rows 0-1 cols 0-1:
    the farthest pair (0,0)-(1,1) has d2 = 2 <= 8 -> full; key tile 3 = rows 2-3
    cols 2-3: (0,0)-(3,3) has d2 = 18 -> touched only ((0,1)-(2,2): 5)."""
    tm = tile_map_bruteforce(4, 4, 8, tile_h=2, tile_w=2, sub_h=1, sub_w=2, key_h=2, key_w=2)
    kts, fl = _entries(tm, 0)
    assert kts == [0, 1, 2, 3]
    assert fl[0] == 0x303
    # sub-tile 0 (row 0) to key tile 3 (rows 2-3, cols 2-3): not all admitted
    assert fl[3] & 0x1 and not fl[3] & 0x100


@pytest.mark.parametrize("gh,gw,r2,tiling", [
    (13, 11, 5, (4, 4, 2, 4, 2, 4)), (20, 9, 16, (16, 8, 4, 8, 4, 8)), (7, 30, 2, (16, 8, 4, 8, 4, 8)),
    (17, 17, 0, (8, 8, 4, 4, 4, 4)), (9, 9, 40, (4, 8, 2, 4, 2, 8)), (21, 19, 25, (16, 8, 4, 8, 4, 8))])
def test_listed_key_tiles_cover_exactly_the_touched_ones(gh, gw, r2, tiling):
    """Every admitted key of every query lies in a listed key tile of its query
    tile, and every listed key tile holds an admitted key of that query tile."""
    th, tw, sh, sw, kh, kw = tiling
    tm = tile_map_bruteforce(gh, gw, r2, th, tw, sh, sw, kh, kw)
    ntx, nkx = -(-gw // tw), -(-gw // kw)
    for t in range(len(tm["offsets"]) - 1):
        ty, tx = divmod(t, ntx)
        want = set()
        for y in range(ty * th, min(gh, ty * th + th)):
            for x in range(tx * tw, min(gw, tx * tw + tw)):
                want |= {(ky // kh) * nkx + kx // kw for ky, kx in _disk_keys(gh, gw, r2, y, x)}
        kts, fl = _entries(tm, t)
        assert kts == sorted(want)
        assert all(f & 0xFF for f in fl)


@pytest.mark.parametrize("gh,gw,r2", [(12, 12, 9), (10, 23, 20), (33, 8, 2), (24, 24, 64)])
def test_listed_tiles_cover_every_admitted_pair_once(gh, gw, r2):
    """Summing, over query tiles, the admitted pairs between the tile's queries
    and the cells of its listed key tiles gives the closed-form count."""
    th, tw, kh, kw = 16, 8, 4, 8
    tm = tile_map_bruteforce(gh, gw, r2)
    ntx, nkx = -(-gw // tw), -(-gw // kw)
    total = 0
    for t in range(len(tm["offsets"]) - 1):
        ty, tx = divmod(t, ntx)
        kts, _ = _entries(tm, t)
        cells = [(kt // nkx * kh + a, kt % nkx * kw + c) for kt in kts for a in range(kh) for c in range(kw)]
        cells = np.array([(y, x) for y, x in cells if y < gh and x < gw])
        for y in range(ty * th, min(gh, ty * th + th)):
            for x in range(tx * tw, min(gw, tx * tw + tw)):
                total += int(((cells[:, 0] - y) ** 2 + (cells[:, 1] - x) ** 2 <= r2).sum())
    assert total == pair_count(0, gh, gw, r2)["img_img"]


def test_every_pair_admitted():
    gh, gw = 20, 16
    tm = tile_map_bruteforce(gh, gw, 10 ** 6)
    nk = 5 * 2  # 5 key-tile rows x 2 key-tile columns
    for t in range(len(tm["offsets"]) - 1):
        kts, fl = _entries(tm, t)
        assert kts == list(range(nk))
        on = 0xF if t < 2 else 0x1   # tiles 2, 3: rows 16-19, only sub-tile 0 on the grid
        assert fl == [on | (on << 8)] * nk


def test_partly_off_grid_key_tiles_are_never_full():
    tm = tile_map_bruteforce(10, 13, 10 ** 6)   # key tiles 4x8 on a 10 x 13 grid
    nkx = 2
    for t in range(len(tm["offsets"]) - 1):
        for kt, f in zip(*_entries(tm, t)):
            kty, ktx = divmod(kt, nkx)
            whole = (kty + 1) * 4 <= 10 and (ktx + 1) * 8 <= 13
            assert ((f >> 8) != 0) == whole


def test_negative_r2_gives_empty_map():
    tm = tile_map_bruteforce(9, 9, -1)
    assert tm["key_tiles"].shape == (0,)
    assert np.all(tm["offsets"] == 0)


def test_radius_zero_unit_tiles_list_only_self():
    gh, gw = 5, 4
    tm = tile_map_bruteforce(gh, gw, 0, 1, 1, 1, 1, 1, 1)
    assert tm["key_tiles"].tolist() == list(range(gh * gw))
    assert tm["flags"].tolist() == [0x101] * (gh * gw)


@pytest.mark.parametrize("gh,gw,r2", [(24, 24, 64), (40, 19, 10)])
def test_full_implies_touched(gh, gw, r2):
    tm = tile_map_bruteforce(gh, gw, r2)
    f = tm["flags"].astype(int)
    assert np.all(((f >> 8) & ~f & 0xFF) == 0)


def test_box_restriction_changes_nothing():
    for gh, gw, r2 in [(30, 22, 25), (17, 40, 3), (9, 9, -1)]:
        full = tile_map_bruteforce(gh, gw, r2)
        boxed = tile_map_bruteforce(gh, gw, r2, box=True)
        for key in full:
            np.testing.assert_array_equal(full[key], boxed[key])
