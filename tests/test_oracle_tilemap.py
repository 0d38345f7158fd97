"""Pins of the oracle's brute-force tile map."""

import math

import numpy as np
import pytest

from oracle import pair_count, tile_map_bruteforce


def _disk_keys(gh, gw, r2, y, x):
    """Image keys of the window around (y, x), built per key row from
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
                out.add(ky * gw + kx)
    return out


def _tile_keys(tm, t):
    a, b = tm["run_offsets"][t], tm["run_offsets"][t + 1]
    keys = []
    for s, n in tm["runs"][a:b]:
        keys.extend(range(int(s), int(s) + int(n)))
    return keys


def test_hand_derived_3x3_case():
    """grid 3x3, r2 = 1, tile 2x2, sub-tiles 1x2, chunks of 4.

    Tile 0 holds (0,0) (0,1) (1,0) (1,1).  Keys within distance 1 of one of
    them: row 0 columns 0-2, row 1 columns 0-2, row 2 columns 0-1, i.e. runs
    (0,3) (3,3) (6,2) and key list 0..7, two chunks [0..3] and [4..7].
    Chunk 0 = (0,0) (0,1) (0,2) (1,0): sub-tile 0 = {(0,0), (0,1)} admits
    (0,0)-(0,0) but not (0,0)-(0,2); sub-tile 1 = {(1,0), (1,1)} admits
    (1,0)-(0,0) but not (1,0)-(0,2) -> touched by both, full for neither: 0x3.
    Chunk 1 = (1,1) (1,2) (2,0) (2,1): (0,1)-(1,1) admitted, (0,0)-(1,2) not;
    (1,1)-(1,1) admitted, (1,0)-(1,2) not -> 0x3.
    Tile 1 = column 2 of rows 0-1: (0,2) (1,2).  Keys: row 0 cols 1-2, row 1
    cols 1-2, row 2 col 2 -> runs (1,2) (4,2) (8,1), keys 1 2 4 5 8 -> chunks
    [1,2,4,5] and [8].  Chunk 0: sub-tile 0 = {(0,2)}: (0,2)-(1,1) has d2 = 2,
    so not full; sub-tile 1 = {(1,2)}: (1,2)-(0,1) d2 = 2 -> 0x3.  Chunk 1 =
    [(2,2)]: (0,2)-(2,2) d2 = 4 not admitted; (1,2)-(2,2) admitted; short
    chunk so never full -> 0x2.
    Tile 2 = row 2 cols 0-1 (sub-tile 1 is off the grid): keys row 1 cols 0-1,
    row 2 cols 0-2 -> runs (3,2) (6,3), keys 3 4 6 7 8 -> chunks [3,4,6,7],
    [8].  Chunk 0: (2,0)-(1,0) admitted, (2,0)-(1,1) d2 = 2 no -> 0x1.
    Chunk 1 = [(2,2)]: (2,1)-(2,2) admitted -> 0x1.
    Tile 3 = (2,2): keys (1,2) (2,1) (2,2) -> runs (5,1) (7,2) -> one short
    chunk, touched by sub-tile 0 -> 0x1.
    """
    tm = tile_map_bruteforce(3, 3, 1, tile_h=2, tile_w=2, sub_h=1, sub_w=2, chunk=4)
    assert tm["run_offsets"].tolist() == [0, 3, 6, 8, 10]
    assert tm["runs"].tolist() == [[0, 3], [3, 3], [6, 2], [1, 2], [4, 2], [8, 1],
                                   [3, 2], [6, 3], [5, 1], [7, 2]]
    assert tm["chunk_offsets"].tolist() == [0, 2, 4, 6, 7]
    assert tm["flags"].tolist() == [0x3, 0x3, 0x3, 0x2, 0x1, 0x1, 0x1]


@pytest.mark.parametrize("gh,gw,r2,tile", [
    (13, 11, 5, (4, 4, 2, 4, 8)), (20, 9, 16, (16, 8, 4, 8, 32)), (7, 30, 2, (16, 8, 4, 8, 32)),
    (17, 17, 0, (8, 8, 4, 4, 16)), (9, 9, 40, (4, 8, 2, 4, 16))])
def test_tile_key_lists_are_the_union_of_windows(gh, gw, r2, tile):
    th, tw, sh, sw, c = tile
    tm = tile_map_bruteforce(gh, gw, r2, th, tw, sh, sw, c)
    ntx = -(-gw // tw)
    nt = (-(-gh // th)) * ntx
    assert len(tm["run_offsets"]) == nt + 1
    for t in range(nt):
        ty, tx = divmod(t, ntx)
        want = set()
        for y in range(ty * th, min(gh, ty * th + th)):
            for x in range(tx * tw, min(gw, tx * tw + tw)):
                want |= _disk_keys(gh, gw, r2, y, x)
        got = _tile_keys(tm, t)
        assert got == sorted(want)
        nch = tm["chunk_offsets"][t + 1] - tm["chunk_offsets"][t]
        assert nch == -(-len(got) // c)
        # runs are maximal and lie on one key row each
        a, b = tm["run_offsets"][t], tm["run_offsets"][t + 1]
        rs = tm["runs"][a:b].astype(int)
        for s, n in rs:
            assert s // gw == (s + n - 1) // gw
        for (s0, n0), (s1, _) in zip(rs[:-1], rs[1:]):
            assert s0 // gw < s1 // gw


@pytest.mark.parametrize("gh,gw,r2", [(12, 12, 9), (10, 23, 20), (33, 8, 2)])
def test_chunks_cover_every_admitted_pair_once(gh, gw, r2):
    """Summing, over tiles, the admitted pairs between each tile's queries and
    its key list gives the closed-form image-image pair count."""
    th, tw = 16, 8
    tm = tile_map_bruteforce(gh, gw, r2, th, tw, 4, 8, 32)
    ntx = -(-gw // tw)
    total = 0
    for t in range(len(tm["run_offsets"]) - 1):
        ty, tx = divmod(t, ntx)
        keys = np.array(_tile_keys(tm, t))
        ky, kx = np.divmod(keys, gw)
        for y in range(ty * th, min(gh, ty * th + th)):
            for x in range(tx * tw, min(gw, tx * tw + tw)):
                total += int(((ky - y) ** 2 + (kx - x) ** 2 <= r2).sum())
    assert total == pair_count(0, gh, gw, r2)["img_img"]


def test_every_pair_admitted_gives_full_rows_and_full_flags():
    gh, gw = 20, 16
    tm = tile_map_bruteforce(gh, gw, 10 ** 6, 16, 8, 4, 8, 32)
    for t in range(len(tm["run_offsets"]) - 1):
        a, b = tm["run_offsets"][t], tm["run_offsets"][t + 1]
        assert tm["runs"][a:b].tolist() == [[y * gw, gw] for y in range(gh)]
    # tiles 0,1: all 4 sub-tiles on the grid; tiles 2,3: rows 16-19, only sub-tile 0
    f = tm["flags"].reshape(4, -1)
    assert np.all(f[:2] == 0xF0F)
    assert np.all(f[2:] == 0x101)


def test_negative_r2_gives_empty_map():
    tm = tile_map_bruteforce(9, 9, -1, 16, 8, 4, 8, 32)
    assert tm["runs"].shape == (0, 2)
    assert tm["flags"].shape == (0,)
    assert np.all(tm["run_offsets"] == 0) and np.all(tm["chunk_offsets"] == 0)


def test_radius_zero_unit_tiles_list_only_self():
    gh, gw = 5, 4
    tm = tile_map_bruteforce(gh, gw, 0, 1, 1, 1, 1, 1)
    assert tm["runs"].tolist() == [[i, 1] for i in range(gh * gw)]
    assert tm["flags"].tolist() == [0x101] * (gh * gw)


@pytest.mark.parametrize("gh,gw,r2", [(24, 24, 64), (40, 19, 10)])
def test_full_flags_imply_touched_and_whole_chunks(gh, gw, r2):
    tm = tile_map_bruteforce(gh, gw, r2, 16, 8, 4, 8, 32)
    f = tm["flags"].astype(int)
    assert np.all(((f >> 8) & ~f & 0xFF) == 0)
    for t in range(len(tm["run_offsets"]) - 1):
        a, b = tm["chunk_offsets"][t], tm["chunk_offsets"][t + 1]
        nkeys = len(_tile_keys(tm, t))
        if nkeys % 32:
            assert (f[b - 1] >> 8) == 0


def test_box_restriction_changes_nothing():
    for gh, gw, r2 in [(30, 22, 25), (17, 40, 3)]:
        full = tile_map_bruteforce(gh, gw, r2)
        boxed = tile_map_bruteforce(gh, gw, r2, box=True)
        for key in full:
            np.testing.assert_array_equal(full[key], boxed[key])
