// tilemap_device.hip -- device builder of the CLEAR tile map.
//
// Three kernels on the caller's stream, from the same closed forms as the host
// builder (tile_geom.h), so the two agree bit for bit:
//   1. one thread per query tile: number of listed key tiles (the closed form
//      listed_key_tiles), written to offsets[t];
//   2. one workgroup: in-place exclusive scan of offsets (entry ntiles
//      receives the total);
//   3. one workgroup per query tile: the flags of every candidate key tile, in
//      blocks of 256 candidates (ascending id), compacted in order with a
//      wavefront ballot and a prefix over the four wavefronts; optionally also
//      each entry's descriptor for the attention kernels (see tile_desc below).
#include <hip/hip_runtime.h>

#include "clear_internal.h"
#include "tile_geom.h"

namespace clear {

namespace {

constexpr int kThreads = 256;
constexpr int kScanThreads = 1024;

__global__ void __launch_bounds__(kThreads) k_tile_counts(TileGeom g, uint32_t* offsets) {
  const int nt = g.nty * g.ntx;
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= nt) return;
  int y0, y1, x0, x1;
  tile_rect(g, t, y0, y1, x0, x1);
  offsets[t] = listed_key_tiles(g, y0, y1, x0, x1);
}

// In-place exclusive scan of x[0..n) with x[n] = total, by one workgroup.
__global__ void __launch_bounds__(kScanThreads) k_scan_offsets(uint32_t* x, int n) {
  __shared__ uint32_t sh[kScanThreads];
  const int tid = threadIdx.x;
  const int per = (n + kScanThreads - 1) / kScanThreads;
  const int s0 = tid * per;
  const int s1 = s0 + per < n ? s0 + per : n;
  uint32_t sum = 0;
  for (int i = s0; i < s1; ++i) sum += x[i];
  sh[tid] = sum;
  __syncthreads();
  for (int off = 1; off < kScanThreads; off <<= 1) {
    const uint32_t v = tid >= off ? sh[tid - off] : 0u;
    __syncthreads();
    sh[tid] += v;
    __syncthreads();
  }
  uint32_t run = sh[tid] - sum;
  for (int i = s0; i < s1; ++i) {
    const uint32_t v = x[i];
    x[i] = run;
    run += v;
  }
  if (tid == kScanThreads - 1) x[n] = sh[tid];
}

__global__ void __launch_bounds__(kThreads) k_tile_fill(TileGeom g, const uint32_t* offsets,
                                                         uint32_t* key_tiles, uint16_t* flags, uint32_t* desc) {
  __shared__ uint32_t wcnt[kThreads / 64];
  const int t = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int y0, y1, x0, x1, kylo, kyhi, kxlo, kxhi;
  tile_rect(g, t, y0, y1, x0, x1);
  candidate_key_tiles(g, y0, y1, x0, x1, kylo, kyhi, kxlo, kxhi);
  const int ncx = kxhi - kxlo + 1;
  const int ncand = kyhi >= kylo ? (kyhi - kylo + 1) * ncx : 0;
  uint32_t base = offsets[t];
  const uint32_t end = offsets[t + 1];  // entries are written only inside this tile's range
  for (int c0 = 0; c0 < ncand; c0 += kThreads) {
    const int c = c0 + (int)threadIdx.x;
    unsigned f = 0;
    int ky = 0, kx = 0;
    if (c < ncand) {
      ky = kylo + c / ncx;
      kx = kxlo + c % ncx;
      f = key_tile_flags(g, y0, x0, ky, kx);
    }
    const bool keep = (f & 0xFFu) != 0;
    const unsigned long long m = __ballot(keep);
    const uint32_t before = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wcnt[wave] = (uint32_t)__popcll(m);
    __syncthreads();
    uint32_t woff = 0;
    for (int w = 0; w < wave; ++w) woff += wcnt[w];
    const uint32_t total = wcnt[0] + wcnt[1] + wcnt[2] + wcnt[3];
    const uint32_t e = base + woff + before;
    if (keep && e < end) {
      key_tiles[e] = (uint32_t)(ky * g.nkx + kx);
      flags[e] = (uint16_t)f;
      if (desc) {
        const uint32_t tok = (uint32_t)(ky * g.kh * g.gw + kx * g.kw);
        const bool inside = ky * g.kh + g.kh <= g.gh && kx * g.kw + g.kw <= g.gw;
        desc[4 * (size_t)e + 0] = tok;
        desc[4 * (size_t)e + 1] = f | (inside ? kTileInside : 0u);
        desc[4 * (size_t)e + 2] = ((uint32_t)ky << 16) | (uint32_t)kx;
        desc[4 * (size_t)e + 3] = (uint32_t)(g.gh * g.gw) - tok;
      }
    }
    base += total;
    __syncthreads();
  }
}

}  // namespace

int tile_map_build_device_launch(const TileGeom& g, uint32_t* offsets, uint32_t* key_tiles,
                                 uint16_t* flags, uint32_t* desc, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int nt = g.nty * g.ntx;
  hipLaunchKernelGGL(k_tile_counts, dim3((nt + kThreads - 1) / kThreads), dim3(kThreads), 0, s, g, offsets);
  hipLaunchKernelGGL(k_scan_offsets, dim3(1), dim3(kScanThreads), 0, s, offsets, nt);
  hipLaunchKernelGGL(k_tile_fill, dim3(nt), dim3(kThreads), 0, s, g, offsets, key_tiles, flags, desc);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(CLEAR_EHIP, "tile map kernels: %s", hipGetErrorString(e));
  return CLEAR_OK;
}

}  // namespace clear
