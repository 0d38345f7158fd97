"""The library's host tile-map builder against the oracle's brute force, bit for bit."""

import ctypes

import numpy as np
import pytest

import dit_circular_local_amd as ca
from oracle import tile_map_bruteforce


def _same(lib_tm, ref):
    for key in ("offsets", "key_tiles", "flags"):
        np.testing.assert_array_equal(lib_tm[key], ref[key], err_msg=key)


def _radii(gh, gw):
    diag2 = (gh - 1) ** 2 + (gw - 1) ** 2
    out = []
    for r in (0, 1, 2, 3, 4, 8, 16, 32):
        out += [r * r, max(r * r - 1, -1)]
    return sorted(set(out + [-1, 2, 5, diag2, diag2 + 7]))


@pytest.mark.parametrize("gh,gw", [(1, 1), (1, 9), (7, 1), (5, 5), (16, 8), (17, 9), (13, 30), (33, 24)])
def test_small_grids_all_radii_both_conventions(gh, gw):
    for r2 in _radii(gh, gw):
        _same(ca.tile_map_build(gh, gw, r2), tile_map_bruteforce(gh, gw, r2))


@pytest.mark.parametrize("tiling", [(4, 4, 2, 4, 2, 4), (8, 8, 4, 4, 4, 4), (2, 2, 1, 2, 2, 2),
                                    (1, 1, 1, 1, 1, 1), (16, 16, 8, 8, 8, 8), (6, 9, 3, 3, 5, 2),
                                    (16, 8, 4, 8, 1, 32), (16, 8, 4, 8, 8, 4)])
def test_other_tilings(tiling):
    th, tw, sh, sw, kh, kw = tiling
    for gh, gw, r2 in [(11, 13, 5), (20, 7, 17), (9, 9, 0), (12, 12, 200)]:
        _same(ca.tile_map_build(gh, gw, r2, th, tw, sh, sw, kh, kw),
              tile_map_bruteforce(gh, gw, r2, th, tw, sh, sw, kh, kw))


@pytest.mark.parametrize("r", [8, 16, 32])
def test_flux_1024_grid_every_tile(r):
    """64 x 64 token grid (1024^2 image), the kernels' tiling, both conventions."""
    for r2 in (r * r, r * r - 1):
        _same(ca.tile_map_build(64, 64, r2), tile_map_bruteforce(64, 64, r2, box=True))


@pytest.mark.parametrize("g,r", [(512, 8), (512, 32), (256, 16), (128, 32)])
def test_large_grids_sampled_tiles(g, r):
    """8192^2 .. 2048^2 grids: sampled tiles (corners, edges, interior) bit for bit."""
    tm = ca.tile_map_build(g, g, r * r)
    ntx = g // 8
    nt = (g // 16) * ntx
    rng = np.random.default_rng(r)
    tiles = sorted(set([0, ntx - 1, nt - ntx, nt - 1, ntx + 1, nt // 2 + ntx // 2]
                       + rng.integers(0, nt, 6).tolist()))
    ref = tile_map_bruteforce(g, g, r * r, tiles=tiles, box=True)
    for i, t in enumerate(tiles):
        a, b = tm["offsets"][t], tm["offsets"][t + 1]
        ra, rb = ref["offsets"][i], ref["offsets"][i + 1]
        np.testing.assert_array_equal(tm["key_tiles"][a:b], ref["key_tiles"][ra:rb])
        np.testing.assert_array_equal(tm["flags"][a:b], ref["flags"][ra:rb])


@pytest.mark.parametrize("gh,gw", [(1, 9), (5, 5), (17, 9), (13, 30), (33, 24)])
def test_square_window_small_grids(gh, gw):
    """The square-window variant: host builder == brute force, bit for bit."""
    for r2 in _radii(gh, gw):
        _same(ca.tile_map_build(gh, gw, r2, window="square"),
              tile_map_bruteforce(gh, gw, r2, window="square"))


def test_square_window_other_tilings_and_flux_grid():
    for th, tw, sh, sw, kh, kw in [(8, 8, 4, 4, 4, 4), (6, 9, 3, 3, 5, 2), (16, 8, 4, 8, 8, 4)]:
        _same(ca.tile_map_build(20, 7, 17, th, tw, sh, sw, kh, kw, window="square"),
              tile_map_bruteforce(20, 7, 17, th, tw, sh, sw, kh, kw, window="square"))
    for r in (8, 16):
        _same(ca.tile_map_build(64, 64, r * r, window="square"),
              tile_map_bruteforce(64, 64, r * r, box=True, window="square"))


def test_unknown_window_is_rejected():
    with pytest.raises(ValueError):
        ca.tile_map_build(8, 8, 4, window="hexagon")
    rc = ca.lib().clear_tile_map_size_ex(7, 8, 8, 4, 16, 8, 4, 8, 4, 8, None)
    assert rc == ca.CLEAR_EINVAL


def test_entry_count_matches_the_listing_on_random_geometries():
    """The size query counts each key-tile row's run of listed columns in closed
    form; the builder lists key tiles one by one.  Both must equal the oracle's
    brute-force count over random grids, radii, tilings and both windows."""
    rng = np.random.default_rng(7)
    for _ in range(60):
        sh, sw = int(rng.integers(1, 5)), int(rng.integers(1, 5))
        nsy, nsx = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        th, tw = sh * nsy, sw * nsx
        kh, kw = int(rng.integers(1, 9)), int(rng.integers(1, 9))
        gh, gw = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        r2 = int(rng.integers(-1, (gh - 1) ** 2 + (gw - 1) ** 2 + 3))
        window = ("circle", "square")[int(rng.integers(0, 2))]
        args = (gh, gw, r2, th, tw, sh, sw, kh, kw)
        n = ca.tile_map_size(*args, window=window)
        ref = tile_map_bruteforce(*args, window=window)
        assert n == len(ref["key_tiles"]), (args, window)
        _same(ca.tile_map_build(*args, window=window), ref)


def test_maps_beyond_32_bit_offsets_are_rejected():
    """An 8192 x 8192 grid at r = 400 lists about 8.7e9 key tiles: the size
    query returns the count (in closed form, without listing them) and the
    builder, whose offsets are 32-bit, refuses it with nothing written."""
    g, r = ca.MAX_GRID, 400
    n = ca.tile_map_size(g, g, r * r)
    assert n > 2 ** 32 - 1
    got = ctypes.c_size_t()
    off = np.zeros(4, np.uint32)
    rc = ca.lib().clear_tile_map_build_ex(0, g, g, r * r, ca.TILE_H, ca.TILE_W, ca.SUB_H, ca.SUB_W, ca.KEY_H,
                                          ca.KEY_W, off.ctypes.data, None, None, 0, ctypes.byref(got))
    assert rc == ca.CLEAR_ENOTSUP and got.value == n
    assert not off.any()
    assert "32-bit" in ca.lib().clear_last_error().decode()


@pytest.mark.slow
@pytest.mark.parametrize("g", [128, 256, 512])
@pytest.mark.parametrize("r", [8, 16, 32])
def test_flux_grids_whole_map_against_bruteforce(g, r):
    """The 2048^2 / 4096^2 / 8192^2 token grids (128^2, 256^2, 512^2 cells) at the
    pages' radii: the kernels' whole tile map, every query tile and every flag,
    against the oracle's pair-by-pair brute force (candidate box only)."""
    _same(ca.tile_map_build(g, g, r * r), tile_map_bruteforce(g, g, r * r, box=True))
