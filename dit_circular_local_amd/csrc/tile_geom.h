// tile_geom.h -- closed-form geometry of CLEAR's circular window (and of the
// square-window variant) over tiles.
//
// Shared by the host and the device tile-map builders (which must agree bit for
// bit).  The window is the image part of CLEAR's mask (pith.science review of
// arXiv 2412.16112, "Core claim"): key cell (ky, kx) is admitted by query cell
// (qy, qx) when (qy-ky)^2 + (qx-kx)^2 <= r2.
//
// Why the closed forms are exact: for a query rectangle Qy x Qx and a key
// rectangle Ky x Kx, the squared distance of a pair splits as dy^2 + dx^2 with
// dy depending only on (qy, ky) and dx only on (qx, kx).  The minimum (maximum)
// of the squared distance over all pairs is therefore the minimum (maximum) of
// dy^2 plus that of dx^2, and those are attained at interval ends.  So a
// sub-tile touches a key tile iff dymin^2 + dxmin^2 <= r2, and admits every pair
// iff dymax^2 + dxmax^2 <= r2.
//
// Square-window variant (the square the circle is inscribed in, against which
// the same review's "What carries the argument" prices the circle at about
// pi/4): key cell admitted when max((qy-ky)^2, (qx-kx)^2) <= r2.  The same
// argument gives touched iff max(dymin^2, dxmin^2) <= r2 and full iff
// max(dymax^2, dxmax^2) <= r2.
#pragma once

#include <stdint.h>

#if defined(__HIP__)
#define CLEAR_HD __host__ __device__ inline
#else
#define CLEAR_HD inline
#endif

namespace clear {

enum { kWindowCircle = 0, kWindowSquare = 1 };

struct TileGeom {
  int gh, gw, r2;     // grid and squared radius (r2 already clamped to the grid diagonal)
  int window;         // kWindowCircle or kWindowSquare
  int th, tw;         // query tile
  int sh, sw;         // sub-tile (one wavefront)
  int kh, kw;         // key tile
  int nty, ntx;       // query tiles per column / row
  int nsy, nsx;       // sub-tiles per tile along y / x
  int nky, nkx;       // key tiles per column / row
  int wmax;           // isqrt(r2) (or -1 when r2 < 0)
};

CLEAR_HD int imax(int a, int b) { return a > b ? a : b; }
CLEAR_HD int imin(int a, int b) { return a < b ? a : b; }
CLEAR_HD int iabs(int a) { return a < 0 ? -a : a; }

// floor(sqrt(x)) for 0 <= x < 2^31, exact.
CLEAR_HD int isqrt_exact(int x) {
  if (x <= 0) return 0;
  int r = (int)__builtin_sqrt((double)x);
  while ((int64_t)r * r > x) --r;
  while ((int64_t)(r + 1) * (r + 1) <= x) ++r;
  return r;
}

CLEAR_HD TileGeom make_geom(int gh, int gw, int r2, int th, int tw, int sh, int sw, int kh,
                            int kw, int window = kWindowCircle) {
  TileGeom g;
  g.gh = gh; g.gw = gw;
  g.window = window;
  // Admitting every pair needs at most the grid diagonal (either window);
  // clamping keeps all squares in 32-bit range without changing the mask.
  int64_t diag = (int64_t)(gh - 1) * (gh - 1) + (int64_t)(gw - 1) * (gw - 1);
  g.r2 = (int64_t)r2 > diag ? (int)diag : r2;
  g.th = th; g.tw = tw; g.sh = sh; g.sw = sw; g.kh = kh; g.kw = kw;
  g.nty = (gh + th - 1) / th;
  g.ntx = (gw + tw - 1) / tw;
  g.nsy = th / sh;
  g.nsx = tw / sw;
  g.nky = (gh + kh - 1) / kh;
  g.nkx = (gw + kw - 1) / kw;
  g.wmax = g.r2 < 0 ? -1 : isqrt_exact(g.r2);
  return g;
}

// Inclusive cell rectangle of query tile t, clipped to the grid.
CLEAR_HD void tile_rect(const TileGeom& g, int t, int& y0, int& y1, int& x0, int& x1) {
  int ty = t / g.ntx, tx = t - ty * g.ntx;
  y0 = ty * g.th; y1 = imin(g.gh, y0 + g.th) - 1;
  x0 = tx * g.tw; x1 = imin(g.gw, x0 + g.tw) - 1;
}

// Candidate key tiles of a query tile: rows [ky_lo, ky_hi] x columns
// [kx_lo, kx_hi] of key tiles meeting the tile's box widened by wmax (no key
// outside it can be admitted).  Empty (ky_lo > ky_hi) when r2 < 0.
CLEAR_HD void candidate_key_tiles(const TileGeom& g, int y0, int y1, int x0, int x1, int& ky_lo,
                                  int& ky_hi, int& kx_lo, int& kx_hi) {
  if (g.wmax < 0) { ky_lo = 0; ky_hi = -1; kx_lo = 0; kx_hi = -1; return; }
  ky_lo = imax(0, y0 - g.wmax) / g.kh;
  ky_hi = imin(g.gh - 1, y1 + g.wmax) / g.kh;
  kx_lo = imax(0, x0 - g.wmax) / g.kw;
  kx_hi = imin(g.gw - 1, x1 + g.wmax) / g.kw;
}

// The window predicate on squared offsets.
CLEAR_HD bool window_admits(const TileGeom& g, int dy2, int dx2) {
  return g.window == kWindowSquare ? imax(dy2, dx2) <= g.r2 : dy2 + dx2 <= g.r2;
}

// Min / max of |a - b| over a in [a0, a1], b in [b0, b1].
CLEAR_HD void interval_dist(int a0, int a1, int b0, int b1, int& dmin, int& dmax) {
  dmin = imax(0, imax(b0 - a1, a0 - b1));
  dmax = imax(iabs(b1 - a0), iabs(a1 - b0));
}

// Number of key tiles listed for the query tile with clipped rectangle
// [y0, y1] x [x0, x1], i.e. of key tiles some sub-tile on the grid touches.
// Those sub-tiles form a product of row ranges and column ranges whose union
// is the clipped rectangle, so one of them reaches both the tile's smallest
// row distance and its smallest column distance to any key tile: a key tile is
// listed iff the rectangle touches it.  In a key-tile row at row distance dy
// that holds for the run of columns meeting [x0 - w, x1 + w], w being the
// largest column distance the window admits there: isqrt(r2 - dy^2) for the
// circle, isqrt(r2) for the square (dy^2 <= r2 in both).  O(key-tile rows).
CLEAR_HD uint32_t listed_key_tiles(const TileGeom& g, int y0, int y1, int x0, int x1) {
  if (g.wmax < 0) return 0;
  const int ky_lo = imax(0, y0 - g.wmax) / g.kh, ky_hi = imin(g.gh - 1, y1 + g.wmax) / g.kh;
  uint32_t n = 0;
  for (int ky = ky_lo; ky <= ky_hi; ++ky) {
    const int ky0 = ky * g.kh, ky1 = imin(g.gh, ky0 + g.kh) - 1;
    int dymin, dymax;
    interval_dist(y0, y1, ky0, ky1, dymin, dymax);
    const int dy2 = dymin * dymin;
    if (dy2 > g.r2) continue;
    const int w = g.window == kWindowSquare ? g.wmax : isqrt_exact(g.r2 - dy2);
    n += (uint32_t)(imin(g.gw - 1, x1 + w) / g.kw - imax(0, x0 - w) / g.kw + 1);
  }
  return n;
}

// Flags (bit s touched, bit 8+s full) of key tile (kty, ktx) for the query tile
// whose top-left cell is (ty0, tx0).
CLEAR_HD unsigned key_tile_flags(const TileGeom& g, int ty0, int tx0, int kty, int ktx) {
  const int ky0 = kty * g.kh, kx0 = ktx * g.kw;
  const int ky1 = imin(g.gh, ky0 + g.kh) - 1, kx1 = imin(g.gw, kx0 + g.kw) - 1;
  const bool on_grid = ky0 + g.kh <= g.gh && kx0 + g.kw <= g.gw;
  unsigned f = 0;
  const int nsub = g.nsy * g.nsx;
  for (int s = 0; s < nsub; ++s) {
    const int sy = s / g.nsx, sx = s - sy * g.nsx;
    const int sy0 = ty0 + sy * g.sh, sx0 = tx0 + sx * g.sw;
    if (sy0 >= g.gh || sx0 >= g.gw) continue;
    const int sy1 = imin(g.gh, sy0 + g.sh) - 1, sx1 = imin(g.gw, sx0 + g.sw) - 1;
    int dymin, dymax, dxmin, dxmax;
    interval_dist(sy0, sy1, ky0, ky1, dymin, dymax);
    interval_dist(sx0, sx1, kx0, kx1, dxmin, dxmax);
    if (window_admits(g, dymin * dymin, dxmin * dxmin)) {
      f |= 1u << s;
      if (on_grid && window_admits(g, dymax * dymax, dxmax * dxmax)) f |= 1u << (8 + s);
    }
  }
  return f;
}

}  // namespace clear
