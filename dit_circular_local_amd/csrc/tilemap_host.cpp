// tilemap_host.cpp -- host builder of the CLEAR tile map (closed form).
//
// For each query tile: the key tiles that at least one of its sub-tiles
// touches, in ascending key-tile id, each with per-sub-tile "touched" and
// "full" bits (see tile_geom.h for why the closed form is exact).  Layout
// documented in clear_attn.h.
#include "clear_internal.h"
#include "tile_geom.h"

namespace clear {

int tile_map_validate(int gh, int gw, int r2, int th, int tw, int sh, int sw, int kh, int kw) {
  if (gh < 1 || gw < 1 || gh > CLEAR_MAX_GRID || gw > CLEAR_MAX_GRID)
    return set_error(CLEAR_EINVAL, "grid sides must be in 1..%d (got %d x %d)",
                     CLEAR_MAX_GRID, gh, gw);
  if (r2 < -1) return set_error(CLEAR_EINVAL, "r2_max must be >= -1 (got %d)", r2);
  if (th < 1 || tw < 1 || sh < 1 || sw < 1 || th % sh || tw % sw)
    return set_error(CLEAR_EINVAL, "tile %dx%d / sub-tile %dx%d: sub-tiles must divide the tile",
                     th, tw, sh, sw);
  if ((th / sh) * (tw / sw) > 8)
    return set_error(CLEAR_EINVAL, "at most 8 sub-tiles per tile (got %d)", (th / sh) * (tw / sw));
  if (th > 1024 || tw > 1024)
    return set_error(CLEAR_EINVAL, "tile sides must be <= 1024");
  if (kh < 1 || kw < 1 || kh > 1024 || kw > 1024)
    return set_error(CLEAR_EINVAL, "key tile sides must be in 1..1024 (got %d x %d)", kh, kw);
  return CLEAR_OK;
}

size_t tile_map_count(const TileGeom& g) {
  size_t n = 0;
  const int nt = g.nty * g.ntx;
  for (int t = 0; t < nt; ++t) {
    int y0, y1, x0, x1;
    tile_rect(g, t, y0, y1, x0, x1);
    n += listed_key_tiles(g, y0, y1, x0, x1);
  }
  return n;
}

int tile_map_check_entries(size_t n_entries) {
  if (n_entries > 0xffffffffull)
    return set_error(CLEAR_ENOTSUP, "the tile map holds %zu entries; its 32-bit offsets reach at most %u",
                     n_entries, 0xffffffffu);
  return CLEAR_OK;
}

size_t tile_map_fill_host(const TileGeom& g, uint32_t* offsets, uint32_t* key_tiles, uint16_t* flags,
                          size_t cap) {
  const int nt = g.nty * g.ntx;
  size_t e = 0;
  for (int t = 0; t < nt; ++t) {
    offsets[t] = (uint32_t)e;
    int y0, y1, x0, x1, kylo, kyhi, kxlo, kxhi;
    tile_rect(g, t, y0, y1, x0, x1);
    candidate_key_tiles(g, y0, y1, x0, x1, kylo, kyhi, kxlo, kxhi);
    for (int ky = kylo; ky <= kyhi; ++ky)
      for (int kx = kxlo; kx <= kxhi; ++kx) {
        const unsigned f = key_tile_flags(g, y0, x0, ky, kx);
        if (f & 0xFFu) {
          if (e < cap) {
            key_tiles[e] = (uint32_t)(ky * g.nkx + kx);
            flags[e] = (uint16_t)f;
          }
          ++e;
        }
      }
  }
  offsets[nt] = (uint32_t)e;
  return e;
}

}  // namespace clear

using namespace clear;

static int window_validate(int window) {
  if (window != CLEAR_WINDOW_CIRCLE && window != CLEAR_WINDOW_SQUARE)
    return set_error(CLEAR_EINVAL, "window must be CLEAR_WINDOW_CIRCLE or CLEAR_WINDOW_SQUARE (got %d)",
                     window);
  return CLEAR_OK;
}

// Lane masks of partly admitted chunks, for the attention kernels' layout: a
// wavefront's 32 own cells are a 4 x 8 sub-tile (lane l: row (l % 32) / 8,
// column l % 8), and accumulator register i of lane group g = l / 32 holds
// the chunk tile's cell (i / 4, 4 g + i % 4).  Whether a pair is admitted
// depends only on the offset D = (chunk tile origin - sub-tile origin), a
// multiple of (4, 8); word i of the entry for D has bit l set iff lane l's
// register i is admitted.  The window is symmetric, so the same words serve a
// query sub-tile against key tiles and a key sub-tile against query tiles.
bool clear::mask_table_dims(const TileGeom& g, int& ky, int& kx) {
  static_assert(CLEAR_SUB_H == 4 && CLEAR_SUB_W == 8 && CLEAR_KEY_H == 4 && CLEAR_KEY_W == 8,
                "table layout follows the kernels' tiles");
  if (g.wmax < 0 || g.wmax > kMaskTableMaxRadius) return false;
  ky = (g.wmax + CLEAR_KEY_H - 1) / CLEAR_SUB_H;   // |D_y| <= wmax + 3
  kx = (g.wmax + CLEAR_KEY_W - 1) / CLEAR_SUB_W;   // |D_x| <= wmax + 7
  return true;
}

void clear::mask_table_fill(const TileGeom& g, int ky, int kx, uint64_t* out) {
  const int nx = 2 * kx + 1;
  for (int iy = -ky; iy <= ky; ++iy)
    for (int ix = -kx; ix <= kx; ++ix) {
      uint64_t* e = out + ((size_t)(iy + ky) * nx + (ix + kx)) * 16;
      for (int i = 0; i < 16; ++i) {
        uint64_t m = 0;
        for (int l = 0; l < 64; ++l) {
          const int qi = l & 31, grp = l >> 5;
          const long long dy = (qi >> 3) - (i >> 2) - CLEAR_SUB_H * iy;
          const long long dx = (qi & 7) - (4 * grp + (i & 3)) - CLEAR_SUB_W * ix;
          const bool in = g.window == kWindowSquare ? (dy * dy <= g.r2 && dx * dx <= g.r2)
                                                    : dy * dy + dx * dx <= g.r2;
          if (in) m |= 1ull << l;
        }
        e[i] = m;
      }
    }
}

extern "C" int clear_tile_map_size_ex(int window, int grid_h, int grid_w, int r2_max, int tile_h,
                                      int tile_w, int sub_h, int sub_w, int key_h, int key_w,
                                      size_t* n_entries) {
  clear_error_reset();
  int rc = window_validate(window);
  if (rc) return rc;
  rc = tile_map_validate(grid_h, grid_w, r2_max, tile_h, tile_w, sub_h, sub_w, key_h, key_w);
  if (rc) return rc;
  if (!n_entries) return set_error(CLEAR_EINVAL, "n_entries must not be NULL");
  TileGeom g = make_geom(grid_h, grid_w, r2_max, tile_h, tile_w, sub_h, sub_w, key_h, key_w, window);
  *n_entries = tile_map_count(g);
  return CLEAR_OK;
}

extern "C" int clear_tile_map_build_ex(int window, int grid_h, int grid_w, int r2_max, int tile_h,
                                       int tile_w, int sub_h, int sub_w, int key_h, int key_w,
                                       uint32_t* offsets, uint32_t* key_tiles, uint16_t* flags,
                                       size_t cap, size_t* n_entries) {
  clear_error_reset();
  int rc = window_validate(window);
  if (rc) return rc;
  rc = tile_map_validate(grid_h, grid_w, r2_max, tile_h, tile_w, sub_h, sub_w, key_h, key_w);
  if (rc) return rc;
  if (!n_entries) return set_error(CLEAR_EINVAL, "n_entries must not be NULL");
  TileGeom g = make_geom(grid_h, grid_w, r2_max, tile_h, tile_w, sub_h, sub_w, key_h, key_w, window);
  *n_entries = tile_map_count(g);
  rc = tile_map_check_entries(*n_entries);
  if (rc) return rc;
  if (*n_entries > cap)
    return set_error(CLEAR_ENOMEM, "tile map needs %zu entries (capacity %zu)", *n_entries, cap);
  if (!offsets || (*n_entries && (!key_tiles || !flags)))
    return set_error(CLEAR_EINVAL, "tile map output pointers must not be NULL");
  const size_t filled = tile_map_fill_host(g, offsets, key_tiles, flags, *n_entries);
  if (filled != *n_entries)
    return set_error(CLEAR_EINVAL, "internal: tile map count %zu differs from the %zu entries listed", *n_entries,
                     filled);
  return CLEAR_OK;
}

extern "C" int clear_tile_map_size(int grid_h, int grid_w, int r2_max, int tile_h, int tile_w,
                                   int sub_h, int sub_w, int key_h, int key_w, size_t* n_entries) {
  return clear_tile_map_size_ex(CLEAR_WINDOW_CIRCLE, grid_h, grid_w, r2_max, tile_h, tile_w, sub_h,
                                sub_w, key_h, key_w, n_entries);
}

extern "C" int clear_tile_map_build(int grid_h, int grid_w, int r2_max, int tile_h, int tile_w,
                                    int sub_h, int sub_w, int key_h, int key_w, uint32_t* offsets,
                                    uint32_t* key_tiles, uint16_t* flags, size_t cap,
                                    size_t* n_entries) {
  return clear_tile_map_build_ex(CLEAR_WINDOW_CIRCLE, grid_h, grid_w, r2_max, tile_h, tile_w, sub_h,
                                 sub_w, key_h, key_w, offsets, key_tiles, flags, cap, n_entries);
}
