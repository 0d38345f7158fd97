// tilemap_device.hip -- device builder of the CLEAR tile map.
//
// Three kernels on the caller's stream, from the same closed forms as the host
// builder (tile_geom.h), so the two agree bit for bit:
//   1. one thread per tile: number of runs and of chunks of the tile, written
//      into run_offsets[t] / chunk_offsets[t];
//   2. one workgroup: in-place exclusive scan of both arrays (entry ntiles
//      receives the totals);
//   3. one workgroup per tile: the runs, an exclusive scan of their lengths in
//      LDS (the flat position of each run in the tile's key list), then the
//      touched / full flags of every chunk.
#include <hip/hip_runtime.h>

#include "clear_internal.h"
#include "tile_geom.h"

namespace clear {

namespace {

__global__ void __launch_bounds__(256) k_tile_counts(TileGeom g, uint32_t* run_offsets,
                                                     uint32_t* chunk_offsets) {
  int t = blockIdx.x * blockDim.x + threadIdx.x;
  int nt = g.nty * g.ntx;
  if (t >= nt) return;
  int y0, y1, x0, x1, lo, hi;
  tile_rect(g, t, y0, y1, x0, x1);
  tile_key_rows(g, y0, y1, lo, hi);
  uint32_t keys = 0;
  for (int ky = lo; ky <= hi; ++ky) {
    int a, b;
    row_run(g, y0, y1, x0, x1, ky, a, b);
    keys += (uint32_t)(b - a + 1);
  }
  run_offsets[t] = hi >= lo ? (uint32_t)(hi - lo + 1) : 0u;
  chunk_offsets[t] = (keys + (uint32_t)g.chunk - 1) / (uint32_t)g.chunk;
}

constexpr int kScanThreads = 1024;

// In-place exclusive scan of x[0..n) with x[n] = total, by one workgroup.
__device__ void block_exclusive_scan_inplace(uint32_t* x, int n, uint32_t* sh) {
  int tid = threadIdx.x;
  int per = (n + kScanThreads - 1) / kScanThreads;
  int s0 = tid * per;
  int s1 = s0 + per < n ? s0 + per : n;
  uint32_t sum = 0;
  for (int i = s0; i < s1; ++i) sum += x[i];
  sh[tid] = sum;
  __syncthreads();
  // Hillis-Steele inclusive scan of the per-thread sums
  for (int off = 1; off < kScanThreads; off <<= 1) {
    uint32_t v = tid >= off ? sh[tid - off] : 0u;
    __syncthreads();
    sh[tid] += v;
    __syncthreads();
  }
  uint32_t run = sh[tid] - sum;  // exclusive prefix of this segment
  for (int i = s0; i < s1; ++i) {
    uint32_t v = x[i];
    x[i] = run;
    run += v;
  }
  if (tid == kScanThreads - 1) x[n] = sh[tid];
}

__global__ void __launch_bounds__(kScanThreads) k_scan_offsets(uint32_t* run_offsets,
                                                               uint32_t* chunk_offsets, int nt) {
  __shared__ uint32_t sh[kScanThreads];
  block_exclusive_scan_inplace(run_offsets, nt, sh);
  __syncthreads();
  block_exclusive_scan_inplace(chunk_offsets, nt, sh);
}

constexpr int kFillThreads = 256;

__global__ void __launch_bounds__(kFillThreads) k_tile_fill(TileGeom g, const uint32_t* run_offsets,
                                                            uint32_t* runs,
                                                            const uint32_t* chunk_offsets,
                                                            uint16_t* flags) {
  // flat offset of each run in the tile's key list (a tile has at most
  // CLEAR_MAX_GRID key rows)
  __shared__ uint32_t off[CLEAR_MAX_GRID + 1];
  __shared__ uint32_t tsum[kFillThreads];
  const int t = blockIdx.x;
  const int tid = threadIdx.x;
  int y0, y1, x0, x1, lo, hi;
  tile_rect(g, t, y0, y1, x0, x1);
  tile_key_rows(g, y0, y1, lo, hi);
  const int nr = hi >= lo ? hi - lo + 1 : 0;
  const uint32_t ro = run_offsets[t];
  const uint32_t co = chunk_offsets[t];
  const uint32_t nch = chunk_offsets[t + 1] - co;

  // runs, and their lengths into off[]
  for (int i = tid; i < nr; i += kFillThreads) {
    int a, b;
    row_run(g, y0, y1, x0, x1, lo + i, a, b);
    runs[2 * (size_t)(ro + i)] = (uint32_t)((lo + i) * g.gw + a);
    runs[2 * (size_t)(ro + i) + 1] = (uint32_t)(b - a + 1);
    off[i] = (uint32_t)(b - a + 1);
  }
  __syncthreads();
  // exclusive scan of off[0..nr) in place, off[nr] = total
  {
    int per = (nr + kFillThreads - 1) / kFillThreads;
    int s0 = tid * per;
    int s1 = s0 + per < nr ? s0 + per : nr;
    uint32_t sum = 0;
    for (int i = s0; i < s1; ++i) sum += off[i];
    tsum[tid] = sum;
    __syncthreads();
    for (int d = 1; d < kFillThreads; d <<= 1) {
      uint32_t v = tid >= d ? tsum[tid - d] : 0u;
      __syncthreads();
      tsum[tid] += v;
      __syncthreads();
    }
    uint32_t run = tsum[tid] - sum;
    for (int i = s0; i < s1; ++i) {
      uint32_t v = off[i];
      off[i] = run;
      run += v;
    }
    if (tid == kFillThreads - 1) off[nr] = tsum[tid];
    __syncthreads();
  }
  const uint32_t total = off[nr];
  const int nsub = g.nsy * g.nsx;

  for (uint32_t j = tid; j < nch; j += kFillThreads) {
    uint32_t f0 = j * (uint32_t)g.chunk;
    uint32_t f1 = f0 + (uint32_t)g.chunk < total ? f0 + (uint32_t)g.chunk : total;
    // last run whose start is <= f0
    int lo_i = 0, hi_i = nr - 1;
    while (lo_i < hi_i) {
      int mid = (lo_i + hi_i + 1) >> 1;
      if (off[mid] <= f0) lo_i = mid; else hi_i = mid - 1;
    }
    unsigned touched = 0, full_ok = 0;
    int sy0[8], sy1[8], sx0[8], sx1[8];
    bool on[8];
    for (int s = 0; s < nsub; ++s) {
      on[s] = sub_rect(g, y0, x0, s, sy0[s], sy1[s], sx0[s], sx1[s]);
      if (on[s]) full_ok |= 1u << s;
    }
    if (f1 - f0 != (uint32_t)g.chunk) full_ok = 0;
    for (int i = lo_i; i < nr && off[i] < f1; ++i) {
      uint32_t ps = off[i] > f0 ? off[i] : f0;
      uint32_t pe = off[i + 1] < f1 ? off[i + 1] : f1;
      if (ps >= pe) continue;
      int a, b;
      row_run(g, y0, y1, x0, x1, lo + i, a, b);
      int xa = a + (int)(ps - off[i]);
      int xb = a + (int)(pe - 1 - off[i]);
      for (int s = 0; s < nsub; ++s) {
        if (!on[s]) continue;
        int dmin2, dmax2;
        piece_minmax(lo + i, xa, xb, sy0[s], sy1[s], sx0[s], sx1[s], dmin2, dmax2);
        if (dmin2 <= g.r2) touched |= 1u << s;
        if (dmax2 > g.r2) full_ok &= ~(1u << s);
      }
    }
    flags[co + j] = (uint16_t)(touched | (full_ok << 8));
  }
}

}  // namespace

int tile_map_build_device_launch(const TileGeom& g, uint32_t* run_offsets, uint32_t* runs,
                                 uint32_t* chunk_offsets, uint16_t* flags, uint32_t* scratch,
                                 void* stream) {
  (void)scratch;
  hipStream_t s = (hipStream_t)stream;
  int nt = g.nty * g.ntx;
  hipLaunchKernelGGL(k_tile_counts, dim3((nt + 255) / 256), dim3(256), 0, s, g, run_offsets,
                     chunk_offsets);
  hipLaunchKernelGGL(k_scan_offsets, dim3(1), dim3(kScanThreads), 0, s, run_offsets,
                     chunk_offsets, nt);
  hipLaunchKernelGGL(k_tile_fill, dim3(nt), dim3(kFillThreads), 0, s, g, run_offsets, runs,
                     chunk_offsets, flags);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return set_error(CLEAR_EHIP, "tile map kernels: %s", hipGetErrorString(e));
  return CLEAR_OK;
}

}  // namespace clear
