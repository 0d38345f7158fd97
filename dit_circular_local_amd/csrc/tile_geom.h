// tile_geom.h -- closed-form geometry of CLEAR's circular window over query tiles.
//
// Shared by the host and the device tile-map builders (which must agree bit for
// bit).  The window is the image part of CLEAR's mask (pith.science review of
// arXiv 2412.16112, "Core claim"): key cell (ky, kx) is admitted by query cell
// (qy, qx) when (qy-ky)^2 + (qx-kx)^2 <= r2.
//
// Why the closed forms are exact: for a set of queries Qy x Qx (a rectangle)
// and keys Ky x Kx (one key row segment, or another rectangle), the squared
// distance splits as dy^2 + dx^2 with dy depending only on (qy, ky) and dx only
// on (qx, kx).  Hence the minimum (maximum) of the squared distance over all
// pairs is the minimum (maximum) of dy^2 plus the minimum (maximum) of dx^2, and
// those are attained at interval ends.  For one key row ky and a query
// rectangle [y0, y1] x [x0, x1], some query admits key (ky, kx) iff
// dymin^2 + dxmin^2 <= r2, i.e. iff kx lies in [x0 - w, x1 + w] with
// w = isqrt(r2 - dymin^2): the union of the windows on a key row is one
// interval.
#pragma once

#include <stdint.h>

#if defined(__HIP__)
#define CLEAR_HD __host__ __device__ inline
#else
#define CLEAR_HD inline
#endif

namespace clear {

struct TileGeom {
  int gh, gw, r2;     // grid and squared radius (r2 already clamped to the grid diagonal)
  int th, tw;         // query tile
  int sh, sw;         // sub-tile (one wavefront)
  int chunk;          // keys per chunk
  int nty, ntx;       // tiles per column / row
  int nsy, nsx;       // sub-tiles per tile along y / x
  int wmax;           // isqrt(r2) (or -1 when r2 < 0)
};

CLEAR_HD int imax(int a, int b) { return a > b ? a : b; }
CLEAR_HD int imin(int a, int b) { return a < b ? a : b; }

// floor(sqrt(x)) for 0 <= x < 2^31, exact.
CLEAR_HD int isqrt_exact(int x) {
  if (x <= 0) return 0;
  int r = (int)__builtin_sqrt((double)x);
  while ((int64_t)r * r > x) --r;
  while ((int64_t)(r + 1) * (r + 1) <= x) ++r;
  return r;
}

CLEAR_HD TileGeom make_geom(int gh, int gw, int r2, int th, int tw, int sh, int sw,
                            int chunk) {
  TileGeom g;
  g.gh = gh; g.gw = gw;
  // Admitting every pair needs at most the grid diagonal; clamping keeps all
  // squares in 32-bit range without changing the mask.
  int64_t diag = (int64_t)(gh - 1) * (gh - 1) + (int64_t)(gw - 1) * (gw - 1);
  g.r2 = (int64_t)r2 > diag ? (int)diag : r2;
  g.th = th; g.tw = tw; g.sh = sh; g.sw = sw; g.chunk = chunk;
  g.nty = (gh + th - 1) / th;
  g.ntx = (gw + tw - 1) / tw;
  g.nsy = th / sh;
  g.nsx = tw / sw;
  g.wmax = g.r2 < 0 ? -1 : isqrt_exact(g.r2);
  return g;
}

// Inclusive cell rectangle of query tile t, clipped to the grid.
CLEAR_HD void tile_rect(const TileGeom& g, int t, int& y0, int& y1, int& x0, int& x1) {
  int ty = t / g.ntx, tx = t - ty * g.ntx;
  y0 = ty * g.th; y1 = imin(g.gh, y0 + g.th) - 1;
  x0 = tx * g.tw; x1 = imin(g.gw, x0 + g.tw) - 1;
}

// Key rows touched by the tile: [ky_lo, ky_hi]; empty (ky_lo > ky_hi) when r2 < 0.
// Every key row within wmax of the tile's rows holds a non-empty run, because
// the run always contains the tile's own columns.
CLEAR_HD void tile_key_rows(const TileGeom& g, int y0, int y1, int& ky_lo, int& ky_hi) {
  if (g.wmax < 0) { ky_lo = 0; ky_hi = -1; return; }
  ky_lo = imax(0, y0 - g.wmax);
  ky_hi = imin(g.gh - 1, y1 + g.wmax);
}

// Run of admitted columns [a, b] on key row ky for the query rectangle.
CLEAR_HD void row_run(const TileGeom& g, int y0, int y1, int x0, int x1, int ky, int& a,
                      int& b) {
  int dy = imax(0, imax(y0 - ky, ky - y1));
  int w = isqrt_exact(g.r2 - dy * dy);
  a = imax(0, x0 - w);
  b = imin(g.gw - 1, x1 + w);
}

// Flags contribution of one piece of a chunk (key row ky, columns [xa, xb])
// for one sub-tile rectangle (already clipped, non-empty).
CLEAR_HD void piece_minmax(int ky, int xa, int xb, int sy0, int sy1, int sx0, int sx1,
                           int& dmin2, int& dmax2) {
  int dymin = imax(0, imax(sy0 - ky, ky - sy1));
  int dxmin = imax(0, imax(sx0 - xb, xa - sx1));
  int dymax = imax(ky - sy0 >= 0 ? ky - sy0 : sy0 - ky, ky - sy1 >= 0 ? ky - sy1 : sy1 - ky);
  int dxmax = imax(xb - sx0 >= 0 ? xb - sx0 : sx0 - xb, sx1 - xa >= 0 ? sx1 - xa : xa - sx1);
  dmin2 = dymin * dymin + dxmin * dxmin;
  dmax2 = dymax * dymax + dxmax * dxmax;
}

// Clipped rectangle of sub-tile s of the tile whose top-left cell is (y0, x0).
// Returns false when the sub-tile has no cell on the grid.
CLEAR_HD bool sub_rect(const TileGeom& g, int ty0, int tx0, int s, int& sy0, int& sy1,
                       int& sx0, int& sx1) {
  int sy = s / g.nsx, sx = s - sy * g.nsx;
  sy0 = ty0 + sy * g.sh;
  sx0 = tx0 + sx * g.sw;
  if (sy0 >= g.gh || sx0 >= g.gw) return false;
  sy1 = imin(g.gh, sy0 + g.sh) - 1;
  sx1 = imin(g.gw, sx0 + g.sw) - 1;
  return true;
}

}  // namespace clear
