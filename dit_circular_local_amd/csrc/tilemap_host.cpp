// tilemap_host.cpp -- host builder of the CLEAR tile map (closed form).
//
// For each query tile: one run of admitted key columns per key row within
// reach (the union of the tile's circular windows on that row, see
// tile_geom.h), the concatenated key list cut into chunks, and per chunk and
// sub-tile the "touched" / "full" bits.  Layout documented in clear_attn.h.
#include <vector>

#include "clear_internal.h"
#include "tile_geom.h"

namespace clear {

int tile_map_validate(int gh, int gw, int r2, int th, int tw, int sh, int sw, int chunk) {
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
  if (chunk < 1 || chunk > 4096)
    return set_error(CLEAR_EINVAL, "chunk must be in 1..4096 (got %d)", chunk);
  return CLEAR_OK;
}

void tile_map_counts(const TileGeom& g, size_t* n_runs, size_t* n_chunks,
                     std::vector<uint32_t>* tile_runs, std::vector<uint32_t>* tile_chunks) {
  size_t nr = 0, nc = 0;
  int nt = g.nty * g.ntx;
  if (tile_runs) tile_runs->assign(nt, 0);
  if (tile_chunks) tile_chunks->assign(nt, 0);
  for (int t = 0; t < nt; ++t) {
    int y0, y1, x0, x1, lo, hi;
    tile_rect(g, t, y0, y1, x0, x1);
    tile_key_rows(g, y0, y1, lo, hi);
    size_t keys = 0;
    for (int ky = lo; ky <= hi; ++ky) {
      int a, b;
      row_run(g, y0, y1, x0, x1, ky, a, b);
      keys += (size_t)(b - a + 1);
    }
    size_t runs_t = hi >= lo ? (size_t)(hi - lo + 1) : 0;
    size_t ch_t = (keys + g.chunk - 1) / g.chunk;
    if (tile_runs) (*tile_runs)[t] = (uint32_t)runs_t;
    if (tile_chunks) (*tile_chunks)[t] = (uint32_t)ch_t;
    nr += runs_t;
    nc += ch_t;
  }
  *n_runs = nr;
  *n_chunks = nc;
}

// Flags of the chunk covering flat positions [f0, f1) of a tile whose runs are
// given by (first row lo, per-run columns a[i], flat offsets off[i]).
uint16_t chunk_flags_host(const TileGeom& g, int ty0, int tx0, int lo, const int* a,
                          const int* b, const uint32_t* off, int nr, uint32_t f0,
                          uint32_t f1, int first_run) {
  int nsub = g.nsy * g.nsx;
  unsigned touched = 0, full_ok = 0;
  int sy0[8], sy1[8], sx0[8], sx1[8];
  bool on[8];
  for (int s = 0; s < nsub; ++s) {
    on[s] = sub_rect(g, ty0, tx0, s, sy0[s], sy1[s], sx0[s], sx1[s]);
    if (on[s]) full_ok |= 1u << s;
  }
  if (f1 - f0 != (uint32_t)g.chunk) full_ok = 0;
  for (int i = first_run; i < nr && off[i] < f1; ++i) {
    uint32_t ps = off[i] > f0 ? off[i] : f0;
    uint32_t pe = off[i + 1] < f1 ? off[i + 1] : f1;
    if (ps >= pe) continue;
    int ky = lo + i;
    int xa = a[i] + (int)(ps - off[i]);
    int xb = a[i] + (int)(pe - 1 - off[i]);
    (void)b;
    for (int s = 0; s < nsub; ++s) {
      if (!on[s]) continue;
      int dmin2, dmax2;
      piece_minmax(ky, xa, xb, sy0[s], sy1[s], sx0[s], sx1[s], dmin2, dmax2);
      if (dmin2 <= g.r2) touched |= 1u << s;
      if (dmax2 > g.r2) full_ok &= ~(1u << s);
    }
  }
  return (uint16_t)(touched | (full_ok << 8));
}

void tile_map_fill_host(const TileGeom& g, uint32_t* run_offsets, uint32_t* runs,
                        uint32_t* chunk_offsets, uint16_t* flags) {
  int nt = g.nty * g.ntx;
  uint32_t ro = 0, co = 0;
  std::vector<int> a, b;
  std::vector<uint32_t> off;
  for (int t = 0; t < nt; ++t) {
    run_offsets[t] = ro;
    chunk_offsets[t] = co;
    int y0, y1, x0, x1, lo, hi;
    tile_rect(g, t, y0, y1, x0, x1);
    tile_key_rows(g, y0, y1, lo, hi);
    int nr = hi >= lo ? hi - lo + 1 : 0;
    a.resize(nr);
    b.resize(nr);
    off.resize(nr + 1);
    uint32_t flat = 0;
    for (int i = 0; i < nr; ++i) {
      int ky = lo + i;
      row_run(g, y0, y1, x0, x1, ky, a[i], b[i]);
      off[i] = flat;
      uint32_t len = (uint32_t)(b[i] - a[i] + 1);
      runs[2 * (size_t)(ro + i)] = (uint32_t)(ky * g.gw + a[i]);
      runs[2 * (size_t)(ro + i) + 1] = len;
      flat += len;
    }
    off[nr] = flat;
    uint32_t nch = (flat + g.chunk - 1) / g.chunk;
    int cur = 0;
    for (uint32_t j = 0; j < nch; ++j) {
      uint32_t f0 = j * (uint32_t)g.chunk;
      uint32_t f1 = f0 + (uint32_t)g.chunk < flat ? f0 + (uint32_t)g.chunk : flat;
      while (cur < nr && off[cur + 1] <= f0) ++cur;
      flags[co + j] = chunk_flags_host(g, y0, x0, lo, a.data(), b.data(), off.data(), nr,
                                       f0, f1, cur);
    }
    ro += (uint32_t)nr;
    co += nch;
  }
  run_offsets[nt] = ro;
  chunk_offsets[nt] = co;
}

}  // namespace clear

using namespace clear;

extern "C" int clear_tile_map_size(int grid_h, int grid_w, int r2_max, int tile_h,
                                   int tile_w, int sub_h, int sub_w, int chunk,
                                   size_t* n_runs, size_t* n_chunks) {
  clear_error_reset();
  int rc = tile_map_validate(grid_h, grid_w, r2_max, tile_h, tile_w, sub_h, sub_w, chunk);
  if (rc) return rc;
  if (!n_runs || !n_chunks) return set_error(CLEAR_EINVAL, "n_runs / n_chunks must not be NULL");
  TileGeom g = make_geom(grid_h, grid_w, r2_max, tile_h, tile_w, sub_h, sub_w, chunk);
  tile_map_counts(g, n_runs, n_chunks, nullptr, nullptr);
  return CLEAR_OK;
}

extern "C" int clear_tile_map_build(int grid_h, int grid_w, int r2_max, int tile_h,
                                    int tile_w, int sub_h, int sub_w, int chunk,
                                    uint32_t* run_offsets, uint32_t* runs, size_t runs_cap,
                                    uint32_t* chunk_offsets, uint16_t* flags,
                                    size_t flags_cap, size_t* n_runs, size_t* n_chunks) {
  clear_error_reset();
  int rc = tile_map_validate(grid_h, grid_w, r2_max, tile_h, tile_w, sub_h, sub_w, chunk);
  if (rc) return rc;
  if (!n_runs || !n_chunks) return set_error(CLEAR_EINVAL, "n_runs / n_chunks must not be NULL");
  TileGeom g = make_geom(grid_h, grid_w, r2_max, tile_h, tile_w, sub_h, sub_w, chunk);
  tile_map_counts(g, n_runs, n_chunks, nullptr, nullptr);
  if (*n_runs > runs_cap || *n_chunks > flags_cap)
    return set_error(CLEAR_ENOMEM, "tile map needs %zu runs and %zu chunks (caps %zu, %zu)",
                     *n_runs, *n_chunks, runs_cap, flags_cap);
  if (!run_offsets || !chunk_offsets || (*n_runs && !runs) || (*n_chunks && !flags))
    return set_error(CLEAR_EINVAL, "tile map output pointers must not be NULL");
  tile_map_fill_host(g, run_offsets, runs, chunk_offsets, flags);
  return CLEAR_OK;
}
