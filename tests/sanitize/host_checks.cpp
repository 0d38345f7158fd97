// host_checks.cpp -- drives the library's host code (argument checks, tile-map
// cache and builders, split choice, workspace and scratch sizing, the
// lane-mask table) under AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Built with the host compiler from clear_attn.cpp and tilemap_host.cpp only;
// the HIP runtime and the device-side launchers are replaced here by host
// stand-ins: "device" memory is host memory, the tile-map "kernels" fill the
// map with the host builder, and the attention "launches" write the last
// element of every buffer the real kernels would write, so that a buffer the
// host code sized too small is reported by the sanitizer.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "clear_attn.h"
#include "clear_internal.h"

static bool g_device = true;
static int g_events[256];
static int g_event_next = 0;

extern "C" {
hipError_t hipGetDevice(int* d) {
  if (!g_device) return hipErrorNoDevice;
  *d = 0;
  return hipSuccess;
}
hipError_t hipDeviceGetAttribute(int* pi, hipDeviceAttribute_t, int) {
  *pi = 256;
  return hipSuccess;
}
hipError_t hipMalloc(void** p, size_t n) {
  *p = malloc(n ? n : 1);
  return *p ? hipSuccess : hipErrorOutOfMemory;
}
hipError_t hipFree(void* p) {
  free(p);
  return hipSuccess;
}
hipError_t hipMallocAsync(void** p, size_t n, hipStream_t) { return hipMalloc(p, n); }
hipError_t hipFreeAsync(void* p, hipStream_t) { return hipFree(p); }
hipError_t hipMemcpyAsync(void* d, const void* s, size_t n, hipMemcpyKind, hipStream_t) {
  memcpy(d, s, n);
  return hipSuccess;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipSuccess; }
hipError_t hipDeviceSynchronize(void) { return hipSuccess; }
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipEventCreateWithFlags(hipEvent_t* e, unsigned) {
  *e = (hipEvent_t)&g_events[g_event_next++ % 256];
  return hipSuccess;
}
hipError_t hipEventDestroy(hipEvent_t) { return hipSuccess; }
hipError_t hipEventRecord(hipEvent_t, hipStream_t) { return hipSuccess; }
hipError_t hipStreamWaitEvent(hipStream_t, hipEvent_t, unsigned) { return hipSuccess; }
hipError_t hipGetLastError(void) { return hipSuccess; }
const char* hipGetErrorString(hipError_t) { return "host stand-in"; }
}

namespace clear {

int tile_map_build_device_launch(const TileGeom& g, uint32_t* offsets, uint32_t* key_tiles, uint16_t* flags,
                                 uint32_t* desc, void*) {
  const size_t n = tile_map_count(g);
  if (tile_map_fill_host(g, offsets, key_tiles, flags, n) != n) abort();
  if (desc)
    for (size_t e = 0; e < n; ++e) {
      const uint32_t ky = key_tiles[e] / (uint32_t)g.nkx, kx = key_tiles[e] % (uint32_t)g.nkx;
      desc[4 * e] = ky * g.kh * g.gw + kx * g.kw;
      desc[4 * e + 1] = flags[e];
      desc[4 * e + 2] = (ky << 16) | kx;
      desc[4 * e + 3] = (uint32_t)(g.gh * g.gw) - desc[4 * e];
    }
  return CLEAR_OK;
}

int attn_launch(const AttnLaunch& a, void*) {
  const size_t bh = (size_t)a.B * a.H;
  const int nall = (a.n_text + a.gh * a.gw + CLEAR_CHUNK - 1) / CLEAR_CHUNK;
  int splits = a.text_splits < 1 ? 1 : a.text_splits;
  if (splits > nall || a.strip) splits = a.strip ? 1 : nall;
  const int per = (nall + splits - 1) / splits;
  splits = (nall + per - 1) / per;
  if ((a.strip || splits > 1) && a.n_text > 0) {
    if (!a.ws_o || !a.ws_ml) abort();
    a.ws_o[(size_t)splits * bh * a.n_text * a.d - 1] = 0.0f;
    a.ws_ml[(size_t)splits * bh * a.n_text * 2 - 1] = 0.0f;
  }
  if (a.tm_offsets == nullptr || (a.mask_tbl == nullptr) != (a.mt_ky == 0 && a.mt_kx == 0 && a.mask_tbl == nullptr))
    abort();
  return CLEAR_OK;
}

int attn_bwd_launch(const BwdLaunch& a, void*) {
  const size_t bh = (size_t)a.B * a.H, n = (size_t)a.n_text + (size_t)a.gh * a.gw;
  a.ws_stats[bh * n * 2 - 1] = 0.0f;
  if (a.n_text > 0) {
    const size_t part = (size_t)(a.text_splits < 1 ? 1 : a.text_splits) * bh * a.n_text * a.d;
    a.ws_dq[part - 1] = a.ws_dk[part - 1] = a.ws_dv[part - 1] = 0.0f;
  }
  return CLEAR_OK;
}

int text_merge_launch(const float*, const float*, int, int, void*, float*, int, int, int, int, int, void*) {
  return CLEAR_OK;
}

int noalloc_scratch(int, void** ptr) {
  static void* s = malloc(CLEAR_NOALLOC_SCRATCH_BYTES);
  *ptr = s;
  return s ? CLEAR_OK : CLEAR_ENOMEM;
}

}  // namespace clear

static int g_fail = 0;
#define EXPECT(cond)                                                              \
  do {                                                                            \
    if (!(cond)) {                                                                \
      fprintf(stderr, "line %d: expected %s (last error: %s)\n", __LINE__, #cond, \
              clear_last_error());                                                \
      ++g_fail;                                                                   \
    }                                                                             \
  } while (0)

// fake device addresses, 16-byte aligned, far apart (never dereferenced)
static const void* addr(int i) { return (const void*)(uintptr_t)(0x100000000000ull * (uintptr_t)(i + 1)); }

int main() {
  // ---- host tile-map builders over many geometries, both windows
  const int tilings[][6] = {{16, 8, 4, 8, 4, 8}, {8, 8, 4, 4, 4, 4}, {6, 9, 3, 3, 5, 2}, {1, 1, 1, 1, 1, 1}};
  const int grids[][2] = {{1, 1}, {1, 9}, {7, 1}, {17, 9}, {64, 64}, {33, 130}};
  const int r2s[] = {-1, 0, 1, 2, 5, 64, 1023, 1024, 100000};
  for (int window = 0; window < 2; ++window)
    for (const auto& t : tilings)
      for (const auto& gd : grids)
        for (int r2 : r2s) {
          size_t n = 0;
          EXPECT(clear_tile_map_size_ex(window, gd[0], gd[1], r2, t[0], t[1], t[2], t[3], t[4], t[5], &n) == 0);
          const size_t nt = (size_t)((gd[0] + t[0] - 1) / t[0]) * ((gd[1] + t[1] - 1) / t[1]);
          std::vector<uint32_t> off(nt + 1), kt(n);
          std::vector<uint16_t> fl(n);
          size_t got = 0;
          if (n > 0)
            EXPECT(clear_tile_map_build_ex(window, gd[0], gd[1], r2, t[0], t[1], t[2], t[3], t[4], t[5], off.data(),
                                           kt.data(), fl.data(), n - 1, &got) == CLEAR_ENOMEM);
          EXPECT(clear_tile_map_build_ex(window, gd[0], gd[1], r2, t[0], t[1], t[2], t[3], t[4], t[5], off.data(),
                                         n ? kt.data() : nullptr, n ? fl.data() : nullptr, n, &got) == 0);
          EXPECT(got == n && off[nt] == n);
        }
  // the lane-mask table at every radius it is built for
  for (int r = 0; r <= 40; ++r)
    for (int window = 0; window < 2; ++window) {
      clear::TileGeom g = clear::make_geom(512, 512, r * r, 16, 8, 4, 8, 4, 8, window);
      int ky = 0, kx = 0;
      if (clear::mask_table_dims(g, ky, kx)) {
        std::vector<uint64_t> tbl((size_t)(2 * ky + 1) * (2 * kx + 1) * 16);
        clear::mask_table_fill(g, ky, kx, tbl.data());
      }
    }

  // ---- layer entry points: argument checks, cache, splits, workspace (host stand-ins)
  clear_opts o{CLEAR_BF16, 1024, nullptr, 0, CLEAR_WINDOW_CIRCLE};
  EXPECT(clear_attn_fwd(addr(0), addr(1), addr(2), (void*)addr(3), 1, 24, 96, 512, 64, 64, 32, nullptr) ==
         CLEAR_EINVAL);
  const int geoms[][3] = {{512, 64, 64}, {0, 37, 21}, {130, 1, 1}, {8, 16, 16}, {512, 512, 512}};
  const int splits[] = {0, 1, 2, 7, 64};
  for (const auto& gm : geoms)
    for (int sp : splits)
      for (int window = 0; window < 2; ++window) {
        o.text_splits = sp;
        o.window = window;
        o.r2_max = gm[0] == 0 && sp == 0 ? 0 : 1024;
        EXPECT(clear_attn_fwd_ex(addr(0), addr(1), addr(2), (void*)addr(3), 1, 24, 128, gm[0], gm[1], gm[2], &o,
                                 nullptr) == 0);
        EXPECT(clear_attn_bwd(addr(0), addr(1), addr(2), addr(3), addr(4), (const float*)addr(5), (void*)addr(6),
                              (void*)addr(7), (void*)addr(8), 1, 24, 128, gm[0], gm[1], gm[2], &o, nullptr) == 0);
        const int rc = clear_attn_fwd_noalloc(addr(0), addr(1), addr(2), (void*)addr(3), 1, 24, 128, gm[0], gm[1],
                                              gm[2], &o, nullptr);
        EXPECT(rc == 0 || (rc == CLEAR_ENOMEM && sp > 8));
      }
  o.text_splits = 0;
  o.window = 0;
  std::vector<float> po(24 * 512 * 128), pml(24 * 512 * 2);
  EXPECT(clear_attn_fwd_strip(addr(0), addr(1), addr(2), (void*)addr(3), 1, 24, 128, 512, 64, 64, &o, 8, 40, 1,
                              po.data(), pml.data(), nullptr) == 0);
  EXPECT(clear_attn_fwd_strip(addr(0), addr(1), addr(2), (void*)addr(3), 1, 24, 128, 512, 64, 64, &o, 40, 8, 1,
                              po.data(), pml.data(), nullptr) == CLEAR_EINVAL);
  EXPECT(clear_text_merge(po.data(), pml.data(), 1, CLEAR_MERGE_EXACT, (void*)addr(3), nullptr, 1, 24, 128, 512,
                          64, 64, CLEAR_BF16, nullptr) == 0);
  {
    size_t n = 0;
    EXPECT(clear_tile_map_descriptors(0, 300, 17, 500, nullptr, nullptr, nullptr, nullptr, 0, &n, nullptr) ==
           CLEAR_ENOMEM);
    const size_t nt = (size_t)((300 + 15) / 16) * ((17 + 7) / 8);
    std::vector<uint32_t> off(nt + 1), kt(n), desc(4 * n);
    std::vector<uint16_t> fl(n);
    EXPECT(clear_tile_map_descriptors(0, 300, 17, 500, off.data(), kt.data(), fl.data(), desc.data(), n, &n,
                                      nullptr) == 0);
  }
  clear_release_cache();

  // ---- no device: every call that reaches the runtime reports CLEAR_EHIP
  g_device = false;
  EXPECT(clear_attn_fwd(addr(0), addr(1), addr(2), (void*)addr(3), 1, 2, 128, 8, 16, 16, 2, nullptr) == CLEAR_EHIP);
  EXPECT(clear_attn_fwd_noalloc(addr(0), addr(1), addr(2), (void*)addr(3), 1, 2, 128, 8, 16, 16, &o, nullptr) ==
         CLEAR_EHIP);
  clear_release_cache();
  if (g_fail) fprintf(stderr, "%d checks failed\n", g_fail);
  else printf("host checks passed\n");
  return g_fail ? 1 : 0;
}
