// clear_attn.cpp -- C ABI of libclear_attn.so: argument checks, tile-map cache,
// text-row workspace and launch sequencing.  See include/clear_attn.h.
#include <hip/hip_runtime_api.h>

#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <tuple>
#include <vector>

#include "clear_internal.h"

namespace clear {

namespace {
thread_local char g_err[512];

struct TileMapDev {
  void* block = nullptr;  // one allocation holding the four arrays
  uint32_t* offsets = nullptr;
  uint32_t* key_tiles = nullptr;
  uint16_t* flags = nullptr;
  uint32_t* desc = nullptr;  // 4 words per entry (tile_map_build_device_launch)
  size_t n_entries = 0;
  hipEvent_t ready = nullptr;  // recorded after the build kernels
  // lane-mask table of partly admitted chunks (null when not built); the host
  // copy lives as long as the entry, so the upload may run asynchronously
  uint64_t* mask_tbl = nullptr;
  int mt_ky = 0, mt_kx = 0;
  std::vector<uint64_t>* mask_host = nullptr;
};

struct DevState {
  std::map<std::tuple<int, int, int, int>, TileMapDev> maps;  // (gh, gw, r2, window)
  void* ws = nullptr;
  size_t ws_bytes = 0;
  // the last call that used the workspace: its stream and an event recorded
  // after its kernels, which a call on another stream waits for
  hipEvent_t ws_done = nullptr;
  hipStream_t ws_stream = nullptr;
  // compute units of the device (a partitioned MI355X exposes fewer than 256)
  int n_cu = 0;
};


std::mutex g_mu;
std::map<int, DevState> g_dev;

// The device's state, with its compute-unit count read on first use.  Caller
// holds g_mu.
int dev_state(int dev, DevState** out) {
  DevState& ds = g_dev[dev];
  if (ds.n_cu <= 0) {
    int n = 0;
    hipError_t e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return set_error(CLEAR_EHIP, "hipDeviceGetAttribute: %s", hipGetErrorString(e));
    ds.n_cu = n > 0 ? n : 256;
  }
  *out = &ds;
  return CLEAR_OK;
}

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

int hip_fail(hipError_t e, const char* what) {
  return set_error(CLEAR_EHIP, "%s: %s", what, hipGetErrorString(e));
}

// Tile map of the kernels' fixed tiling for (gh, gw, r2, window) on the current
// device; built on `stream` on first use.  Caller holds g_mu.
int get_tile_map(DevState& ds, int gh, int gw, int r2, int window, hipStream_t stream,
                 TileMapDev** out) {
  TileGeom g = make_geom(gh, gw, r2, CLEAR_TILE_H, CLEAR_TILE_W, CLEAR_SUB_H, CLEAR_SUB_W, CLEAR_KEY_H,
                         CLEAR_KEY_W, window);
  auto key = std::make_tuple(gh, gw, g.r2, window);
  auto it = ds.maps.find(key);
  if (it != ds.maps.end()) {
    *out = &it->second;
    return CLEAR_OK;
  }
  TileMapDev m;
  m.n_entries = tile_map_count(g);
  if (m.n_entries > (size_t)kMaxKernelEntries)
    return set_error(CLEAR_ENOTSUP,
                     "the tile map of a %d x %d grid at r2 %d holds %zu key tiles; the attention kernels "
                     "index at most %d",
                     gh, gw, g.r2, m.n_entries, kMaxKernelEntries);
  const size_t nt = (size_t)g.nty * g.ntx;
  const size_t o_kt = align_up((nt + 1) * 4, 256);
  const size_t o_fl = align_up(o_kt + m.n_entries * 4, 256);
  const size_t o_ds = align_up(o_fl + m.n_entries * 2 + 2, 256);
  const size_t bytes = align_up(o_ds + m.n_entries * 16, 256);
  hipError_t e = hipMalloc(&m.block, bytes);
  if (e != hipSuccess)
    return set_error(CLEAR_ENOMEM, "tile map allocation (%zu bytes): %s", bytes, hipGetErrorString(e));
  char* b = (char*)m.block;
  m.offsets = (uint32_t*)b;
  m.key_tiles = (uint32_t*)(b + o_kt);
  m.flags = (uint16_t*)(b + o_fl);
  m.desc = (uint32_t*)(b + o_ds);
  int rc = tile_map_build_device_launch(g, m.offsets, m.key_tiles, m.flags, m.desc, stream);
  if (rc) {
    (void)hipFree(m.block);
    return rc;
  }
  if (mask_table_dims(g, m.mt_ky, m.mt_kx)) {
    const size_t words = (size_t)(2 * m.mt_ky + 1) * (2 * m.mt_kx + 1) * 16;
    m.mask_host = new std::vector<uint64_t>(words);
    mask_table_fill(g, m.mt_ky, m.mt_kx, m.mask_host->data());
    if ((e = hipMalloc(&m.mask_tbl, words * 8)) != hipSuccess ||
        (e = hipMemcpyAsync(m.mask_tbl, m.mask_host->data(), words * 8, hipMemcpyHostToDevice, stream)) !=
            hipSuccess) {
      (void)hipStreamSynchronize(stream);
      if (m.mask_tbl) (void)hipFree(m.mask_tbl);
      delete m.mask_host;
      (void)hipFree(m.block);
      return hip_fail(e, "mask table");
    }
  }
  if ((e = hipEventCreateWithFlags(&m.ready, hipEventDisableTiming)) != hipSuccess ||
      (e = hipEventRecord(m.ready, stream)) != hipSuccess) {
    (void)hipStreamSynchronize(stream);
    (void)hipFree(m.block);
    return hip_fail(e, "tile map event");
  }
  auto ins = ds.maps.emplace(key, m);
  *out = &ins.first->second;
  return CLEAR_OK;
}

// The device's library workspace, grown to at least `need` bytes, for kernels
// about to be enqueued on stream s.  If the previous user ran on another
// stream, s first waits (on the device) for that user's kernels, so calls on
// different streams take turns with the buffer; workspace_done records the
// end of this call's use.  Growth is stream-ordered and never blocks the host:
// once s has waited for the last user, the old buffer is released with
// hipFreeAsync on s and the new one taken with hipMallocAsync on s, so both
// happen after every kernel that used the old buffer and before the kernels
// of this call.  Caller holds g_mu.
int workspace(DevState& ds, size_t need, hipStream_t s, void** out) {
  hipError_t e;
  if (ds.ws_done && ds.ws_stream != s) {
    if ((e = hipStreamWaitEvent(s, ds.ws_done, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent (workspace)");
  }
  if (need > ds.ws_bytes) {
    if (ds.ws) {
      if ((e = hipFreeAsync(ds.ws, s)) != hipSuccess) return hip_fail(e, "hipFreeAsync (workspace)");
      ds.ws = nullptr;
      ds.ws_bytes = 0;
    }
    if ((e = hipMallocAsync(&ds.ws, need, s)) != hipSuccess) {
      ds.ws = nullptr;
      return set_error(CLEAR_ENOMEM, "workspace (%zu bytes): %s", need, hipGetErrorString(e));
    }
    ds.ws_bytes = need;
  }
  *out = ds.ws;
  return CLEAR_OK;
}

int workspace_done(DevState& ds, hipStream_t s) {
  hipError_t e;
  if (!ds.ws_done && (e = hipEventCreateWithFlags(&ds.ws_done, hipEventDisableTiming)) != hipSuccess)
    return hip_fail(e, "hipEventCreateWithFlags (workspace)");
  if ((e = hipEventRecord(ds.ws_done, s)) != hipSuccess) return hip_fail(e, "hipEventRecord (workspace)");
  ds.ws_stream = s;
  return CLEAR_OK;
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

}  // namespace

// Text-row split count: make a text workgroup's key range (its critical path)
// at most about half of the ideal time of the whole launch.  With fill_slots
// (the forward), also at least enough splits for the text workgroups to take
// one workgroup slot each across the chip: on the 512x512 + 512 FLUX shape
// (24 heads) that is 8 splits, measured 1.5-3 % faster than the 2 (r = 32) and
// 5 (r = 8) of the critical-path rule alone, and neutral on 256x256 + 512.
int choose_text_splits(int B, int H, int n_text, int N, int ntiles, size_t img_chunks, int n_cu,
                       double waves_per_simd, bool fill_slots) {
  // img_chunks: listed key tiles (32 keys each) over all query tiles
  if (n_text == 0) return 1;
  const double nall = (N + CLEAR_CHUNK - 1) / CLEAR_CHUNK;
  const double text_blocks = (n_text + 127) / 128;
  const double nt_ch = (n_text + CLEAR_CHUNK - 1) / CLEAR_CHUNK;
  // wavefront-chunks of work (each = 32 queries x 32 keys)
  const double w_img = (double)B * H * (4.0 * ntiles * nt_ch + 3.0 * (double)img_chunks);
  const double w_text = (double)B * H * text_blocks * 4.0 * nall;
  const double slots = (double)n_cu * 4.0 * waves_per_simd;  // CUs x SIMDs x resident waves
  const double t_ideal = (w_img + w_text) / slots;
  int s = (int)(2.0 * nall / (t_ideal > 1.0 ? t_ideal : 1.0)) + 1;
  if (fill_slots) {
    const double wg_slots = (double)n_cu * waves_per_simd;  // workgroups of 4 wavefronts resident on the device
    const int s_fill = (int)(wg_slots / ((double)B * H * text_blocks));
    if (s_fill > s) s = s_fill;
  }
  int smax = (int)(nall / 8.0);
  if (s > smax) s = smax;
  if (s > 64) s = 64;
  if (s < 1) s = 1;
  return s;
}

int set_error(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

void clear_error_reset() { g_err[0] = 0; }

bool debug_sync_enabled() {
  static int v = -1;
  if (v < 0) {
    const char* e = getenv("CLEAR_DEBUG");
    v = (e && e[0] == '1') ? 1 : 0;
  }
  return v == 1;
}

}  // namespace clear

using namespace clear;

extern "C" const char* clear_last_error(void) { return g_err; }

extern "C" int clear_version(void) { return 10500; }

namespace {

// The forward pass behind clear_attn_fwd_ex (whole layer: strip == nullptr) and
// clear_attn_fwd_strip (one strip: image rows [row_begin, row_end) and the text
// partial into the caller's buffers).
struct StripArgs {
  int row_begin, row_end, text_keys;
  float* part_o;
  float* part_ml;
};

}  // namespace

// Argument checks of the forward entry points (see clear_attn.h); *o receives
// the options with their defaults filled in.
int validate_forward(const void* q, const void* k, const void* v, void* out, int B, int H, int d, int n_text,
                     int grid_h, int grid_w, const clear_opts* opts, const StripArgs* strip, clear_opts* o_out) {
  clear_opts o = opts ? *opts : clear_opts{CLEAR_BF16, 0, nullptr, 0, CLEAR_WINDOW_CIRCLE};
  if (!q || !k || !v || !out) return set_error(CLEAR_EINVAL, "q, k, v and out must not be NULL");
  if (B < 1 || H < 1) return set_error(CLEAR_EINVAL, "B and H must be >= 1 (got %d, %d)", B, H);
  if (d != 64 && d != 128) return set_error(CLEAR_EINVAL, "d must be 64 or 128 (got %d)", d);
  if (n_text < 0) return set_error(CLEAR_EINVAL, "n_text must be >= 0 (got %d)", n_text);
  if (grid_h < 1 || grid_w < 1 || grid_h > CLEAR_MAX_GRID || grid_w > CLEAR_MAX_GRID)
    return set_error(CLEAR_EINVAL, "grid sides must be in 1..%d (got %d x %d)", CLEAR_MAX_GRID, grid_h, grid_w);
  if (o.dtype != CLEAR_BF16 && o.dtype != CLEAR_FP32)
    return set_error(CLEAR_EINVAL, "dtype must be CLEAR_BF16 or CLEAR_FP32 (got %d)", o.dtype);
  if (o.r2_max < -1) return set_error(CLEAR_EINVAL, "r2_max must be >= -1 (got %d)", o.r2_max);
  if (o.window != CLEAR_WINDOW_CIRCLE && o.window != CLEAR_WINDOW_SQUARE)
    return set_error(CLEAR_EINVAL, "window must be CLEAR_WINDOW_CIRCLE or CLEAR_WINDOW_SQUARE (got %d)",
                     o.window);
  if (n_text == 0 && o.r2_max < 0)
    return set_error(CLEAR_EINVAL, "n_text == 0 and r2_max < 0: every query row would be empty");
  if (o.text_splits < 0 || o.text_splits > 64)
    return set_error(CLEAR_EINVAL, "text_splits must be in 0..64 (got %d)", o.text_splits);
  if (strip) {
    if (strip->row_begin < 0 || strip->row_end > grid_h || strip->row_begin >= strip->row_end)
      return set_error(CLEAR_EINVAL, "strip rows [%d, %d) must be a non-empty range inside 0..%d",
                       strip->row_begin, strip->row_end, grid_h);
    if (o.text_splits != 0) return set_error(CLEAR_EINVAL, "a strip computes its text partial in one part");
    if (n_text > 0 && (!strip->part_o || !strip->part_ml))
      return set_error(CLEAR_EINVAL, "text_part_o and text_part_ml must not be NULL when n_text > 0");
    if (((uintptr_t)strip->part_o | (uintptr_t)strip->part_ml) & 3)
      return set_error(CLEAR_EINVAL, "text partial buffers must be 4-byte aligned");
  }
  const long long N = (long long)n_text + (long long)grid_h * grid_w;
  if (N > kMaxTokens) return set_error(CLEAR_EINVAL, "sequence too long (N = %lld; at most %lld)", N, kMaxTokens);
  const size_t elem = o.dtype == CLEAR_BF16 ? 2 : 4;
  const size_t bytes = (size_t)B * H * (size_t)N * d * elem;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out) & 15)
    return set_error(CLEAR_EINVAL, "q, k, v and out must be 16-byte aligned");
  if (ranges_overlap(out, bytes, q, bytes) || ranges_overlap(out, bytes, k, bytes) ||
      ranges_overlap(out, bytes, v, bytes))
    return set_error(CLEAR_EINVAL, "out must not overlap q, k or v");
  if (o.lse_out && ((uintptr_t)o.lse_out & 3)) return set_error(CLEAR_EINVAL, "lse_out must be 4-byte aligned");

  *o_out = o;
  return CLEAR_OK;
}

namespace {

int run_forward(const void* q, const void* k, const void* v, void* out, int B, int H, int d,
                int n_text, int grid_h, int grid_w, const clear_opts* opts, const StripArgs* strip,
                void* stream) {
  clear_opts o;
  int rc0 = validate_forward(q, k, v, out, B, H, d, n_text, grid_h, grid_w, opts, strip, &o);
  if (rc0) return rc0;
  const long long N = (long long)n_text + (long long)grid_h * grid_w;
  hipStream_t s = (hipStream_t)stream;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");

  std::lock_guard<std::mutex> lock(g_mu);
  DevState* dsp = nullptr;
  int rc = dev_state(dev, &dsp);
  if (rc) return rc;
  DevState& ds = *dsp;
  TileMapDev* tm = nullptr;
  rc = get_tile_map(ds, grid_h, grid_w, o.r2_max, o.window, s, &tm);
  if (rc) return rc;
  if ((e = hipStreamWaitEvent(s, tm->ready, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");

  TileGeom g = make_geom(grid_h, grid_w, o.r2_max, CLEAR_TILE_H, CLEAR_TILE_W, CLEAR_SUB_H, CLEAR_SUB_W,
                         CLEAR_KEY_H, CLEAR_KEY_W, o.window);
  int splits = strip ? 1
                     : o.text_splits ? o.text_splits
                                     : choose_text_splits(B, H, n_text, (int)N, g.nty * g.ntx, tm->n_entries,
                                                          ds.n_cu, 3.0, true);
  AttnLaunch a;
  memset(&a, 0, sizeof a);
  a.q = q; a.k = k; a.v = v; a.out = out; a.lse = o.lse_out;
  a.tm_offsets = tm->offsets; a.tm_desc = tm->desc;
  a.mask_tbl = tm->mask_tbl; a.mt_ky = tm->mt_ky; a.mt_kx = tm->mt_kx;
  a.B = B; a.H = H; a.d = d; a.n_text = n_text; a.gh = grid_h; a.gw = grid_w; a.r2 = g.r2;
  a.dtype = o.dtype; a.text_splits = splits; a.window = o.window;
  a.row_begin = strip ? strip->row_begin : 0;
  a.row_end = strip ? strip->row_end : grid_h;
  if (strip) {
    a.strip = 1;
    a.strip_text_keys = strip->text_keys ? 1 : 0;
    a.ws_o = strip->part_o;
    a.ws_ml = strip->part_ml;
  } else if (splits > 1 && n_text > 0) {
    const size_t o_bytes = align_up((size_t)splits * B * H * n_text * d * 4, 256);
    const size_t need = o_bytes + (size_t)splits * B * H * n_text * 2 * 4;
    void* ws = nullptr;
    if ((rc = workspace(ds, need, s, &ws)) != CLEAR_OK) return rc;
    a.ws_o = (float*)ws;
    a.ws_ml = (float*)((char*)ws + o_bytes);
  }
  rc = attn_launch(a, stream);
  if (rc) return rc;
  if (a.ws_o && !strip && (rc = workspace_done(ds, s)) != CLEAR_OK) return rc;
  if (debug_sync_enabled()) {
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "CLEAR_DEBUG sync");
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "CLEAR_DEBUG check");
  }
  return CLEAR_OK;
}

int run_backward(const void* q, const void* k, const void* v, const void* out, const void* dout,
                 const float* lse, void* dq, void* dk, void* dv, int B, int H, int d, int n_text,
                 int grid_h, int grid_w, const clear_opts* opts, void* stream) {
  clear_opts o = opts ? *opts : clear_opts{CLEAR_BF16, 0, nullptr, 0, CLEAR_WINDOW_CIRCLE};
  if (!q || !k || !v || !out || !dout || !lse || !dq || !dk || !dv)
    return set_error(CLEAR_EINVAL, "q, k, v, out, dout, lse, dq, dk and dv must not be NULL");
  if (B < 1 || H < 1) return set_error(CLEAR_EINVAL, "B and H must be >= 1 (got %d, %d)", B, H);
  if (d != 64 && d != 128) return set_error(CLEAR_EINVAL, "d must be 64 or 128 (got %d)", d);
  if (n_text < 0) return set_error(CLEAR_EINVAL, "n_text must be >= 0 (got %d)", n_text);
  if (grid_h < 1 || grid_w < 1 || grid_h > CLEAR_MAX_GRID || grid_w > CLEAR_MAX_GRID)
    return set_error(CLEAR_EINVAL, "grid sides must be in 1..%d (got %d x %d)", CLEAR_MAX_GRID, grid_h, grid_w);
  if (o.dtype != CLEAR_BF16 && o.dtype != CLEAR_FP32)
    return set_error(CLEAR_EINVAL, "dtype must be CLEAR_BF16 or CLEAR_FP32 (got %d)", o.dtype);
  if (o.r2_max < -1) return set_error(CLEAR_EINVAL, "r2_max must be >= -1 (got %d)", o.r2_max);
  if (o.window != CLEAR_WINDOW_CIRCLE && o.window != CLEAR_WINDOW_SQUARE)
    return set_error(CLEAR_EINVAL, "window must be CLEAR_WINDOW_CIRCLE or CLEAR_WINDOW_SQUARE (got %d)",
                     o.window);
  if (n_text == 0 && o.r2_max < 0)
    return set_error(CLEAR_EINVAL, "n_text == 0 and r2_max < 0: every query row would be empty");
  if (o.text_splits < 0 || o.text_splits > 64)
    return set_error(CLEAR_EINVAL, "text_splits must be in 0..64 (got %d)", o.text_splits);
  if (o.lse_out) return set_error(CLEAR_EINVAL, "lse_out is a forward output; pass NULL to the backward");
  const long long N = (long long)n_text + (long long)grid_h * grid_w;
  if (N > kMaxTokens) return set_error(CLEAR_EINVAL, "sequence too long (N = %lld; at most %lld)", N, kMaxTokens);
  const size_t elem = o.dtype == CLEAR_BF16 ? 2 : 4;
  const size_t bytes = (size_t)B * H * (size_t)N * d * elem;
  const size_t lse_bytes = (size_t)B * H * (size_t)N * 4;
  if (((uintptr_t)q | (uintptr_t)k | (uintptr_t)v | (uintptr_t)out | (uintptr_t)dout | (uintptr_t)dq |
       (uintptr_t)dk | (uintptr_t)dv) & 15)
    return set_error(CLEAR_EINVAL, "q, k, v, out, dout, dq, dk and dv must be 16-byte aligned");
  if ((uintptr_t)lse & 3) return set_error(CLEAR_EINVAL, "lse must be 4-byte aligned");
  const void* ins[5] = {q, k, v, out, dout};
  void* grads[3] = {dq, dk, dv};
  for (int i = 0; i < 3; ++i) {
    for (int j = 0; j < 5; ++j)
      if (ranges_overlap(grads[i], bytes, ins[j], bytes))
        return set_error(CLEAR_EINVAL, "dq, dk and dv must not overlap q, k, v, out or dout");
    if (ranges_overlap(grads[i], bytes, lse, lse_bytes))
      return set_error(CLEAR_EINVAL, "dq, dk and dv must not overlap lse");
    for (int j = i + 1; j < 3; ++j)
      if (ranges_overlap(grads[i], bytes, grads[j], bytes))
        return set_error(CLEAR_EINVAL, "dq, dk and dv must not overlap each other");
  }

  hipStream_t s = (hipStream_t)stream;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");

  std::lock_guard<std::mutex> lock(g_mu);
  DevState* dsp = nullptr;
  int rc = dev_state(dev, &dsp);
  if (rc) return rc;
  DevState& ds = *dsp;
  TileMapDev* tm = nullptr;
  rc = get_tile_map(ds, grid_h, grid_w, o.r2_max, o.window, s, &tm);
  if (rc) return rc;
  if ((e = hipStreamWaitEvent(s, tm->ready, 0)) != hipSuccess) return hip_fail(e, "hipStreamWaitEvent");

  TileGeom g = make_geom(grid_h, grid_w, o.r2_max, CLEAR_TILE_H, CLEAR_TILE_W, CLEAR_SUB_H, CLEAR_SUB_W,
                         CLEAR_KEY_H, CLEAR_KEY_W, o.window);
  const int splits = o.text_splits ? o.text_splits
                                   : choose_text_splits(B, H, n_text, (int)N, g.nty * g.ntx, tm->n_entries,
                                                        ds.n_cu, 2.0);
  const size_t stats_bytes = align_up((size_t)B * H * (size_t)N * 8, 256);
  const size_t part_bytes = n_text > 0 ? align_up((size_t)splits * B * H * n_text * d * 4, 256) : 0;
  void* ws = nullptr;
  if ((rc = workspace(ds, stats_bytes + 3 * part_bytes, s, &ws)) != CLEAR_OK) return rc;

  BwdLaunch a;
  memset(&a, 0, sizeof a);
  a.q = q; a.k = k; a.v = v; a.out = out; a.dout = dout; a.lse = lse;
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.ws_stats = (float*)ws;
  if (n_text > 0) {
    a.ws_dq = (float*)((char*)ws + stats_bytes);
    a.ws_dk = (float*)((char*)ws + stats_bytes + part_bytes);
    a.ws_dv = (float*)((char*)ws + stats_bytes + 2 * part_bytes);
  }
  a.tm_offsets = tm->offsets; a.tm_desc = tm->desc;
  a.mask_tbl = tm->mask_tbl; a.mt_ky = tm->mt_ky; a.mt_kx = tm->mt_kx;
  a.B = B; a.H = H; a.d = d; a.n_text = n_text; a.gh = grid_h; a.gw = grid_w; a.r2 = g.r2;
  a.dtype = o.dtype; a.text_splits = splits; a.window = o.window;
  rc = attn_bwd_launch(a, stream);
  if (rc) return rc;
  if ((rc = workspace_done(ds, s)) != CLEAR_OK) return rc;
  if (debug_sync_enabled()) {
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "CLEAR_DEBUG sync");
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "CLEAR_DEBUG check");
  }
  return CLEAR_OK;
}

}  // namespace

extern "C" int clear_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                              const void* dout, const float* lse, void* dq, void* dk, void* dv, int B,
                              int H, int d, int n_text, int grid_h, int grid_w, const clear_opts* opts,
                              void* stream) {
  clear_error_reset();
  return run_backward(q, k, v, out, dout, lse, dq, dk, dv, B, H, d, n_text, grid_h, grid_w, opts, stream);
}

extern "C" int clear_attn_fwd_ex(const void* q, const void* k, const void* v, void* out, int B,
                                 int H, int d, int n_text, int grid_h, int grid_w,
                                 const clear_opts* opts, void* stream) {
  clear_error_reset();
  return run_forward(q, k, v, out, B, H, d, n_text, grid_h, grid_w, opts, nullptr, stream);
}

extern "C" int clear_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, int B, int H,
                                      int d, int n_text, int grid_h, int grid_w, const clear_opts* opts,
                                      void* stream) {
  clear_error_reset();
  clear_opts o;
  int rc = validate_forward(q, k, v, out, B, H, d, n_text, grid_h, grid_w, opts, nullptr, &o);
  if (rc) return rc;
  const long long N = (long long)n_text + (long long)grid_h * grid_w;
  const size_t cap = CLEAR_NOALLOC_SCRATCH_BYTES;

  // the tile map at the kernels' tiling, laid out as the cached copy (sized on
  // the host before any HIP call)
  TileGeom g = make_geom(grid_h, grid_w, o.r2_max, CLEAR_TILE_H, CLEAR_TILE_W, CLEAR_SUB_H, CLEAR_SUB_W,
                         CLEAR_KEY_H, CLEAR_KEY_W, o.window);
  const size_t n_entries = tile_map_count(g);
  if (n_entries > (size_t)kMaxKernelEntries)
    return set_error(CLEAR_ENOTSUP, "the tile map holds %zu key tiles; the attention kernels index at most %d",
                     n_entries, kMaxKernelEntries);
  const size_t nt = (size_t)g.nty * g.ntx;
  const size_t o_kt = align_up((nt + 1) * 4, 256);
  const size_t o_fl = align_up(o_kt + n_entries * 4, 256);
  const size_t o_ds = align_up(o_fl + n_entries * 2 + 2, 256);
  const size_t map_bytes = align_up(o_ds + n_entries * 16, 256);
  if (map_bytes > cap)
    return set_error(CLEAR_ENOMEM, "the tile map of a %d x %d grid at r2 %d needs %zu bytes; the no-alloc "
                     "scratch holds %zu", grid_h, grid_w, g.r2, map_bytes, cap);

  if (o.text_splits > 1 && n_text > 0 &&
      (size_t)o.text_splits * (align_up((size_t)B * H * n_text * d * 4, 256) +
                               align_up((size_t)B * H * n_text * 8, 256)) > cap - map_bytes)
    return set_error(CLEAR_ENOMEM, "%d text splits do not fit the no-alloc scratch beside the tile map",
                     o.text_splits);

  hipStream_t s = (hipStream_t)stream;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int n_cu = 0;
  if ((e = hipDeviceGetAttribute(&n_cu, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return hip_fail(e, "hipDeviceGetAttribute");
  void* base = nullptr;
  if ((rc = noalloc_scratch(dev, &base)) != CLEAR_OK) return rc;

  // text-row partials beside it
  const size_t per_split = align_up((size_t)B * H * n_text * d * 4, 256) + align_up((size_t)B * H * n_text * 8, 256);
  const size_t room = (cap - map_bytes) / (per_split ? per_split : 1);
  int splits = o.text_splits ? o.text_splits
                             : choose_text_splits(B, H, n_text, (int)N, (int)nt, n_entries, n_cu > 0 ? n_cu : 256,
                                                  3.0, true);
  if (n_text > 0 && splits > 1 && (size_t)splits > room) {
    if (o.text_splits)
      return set_error(CLEAR_ENOMEM, "%d text splits need %zu bytes of partials; the no-alloc scratch has %zu "
                       "left beside the tile map", splits, (size_t)splits * per_split, cap - map_bytes);
    splits = room > 1 ? (int)room : 1;
  }

  char* b = (char*)base;
  AttnLaunch a;
  memset(&a, 0, sizeof a);
  a.q = q; a.k = k; a.v = v; a.out = out; a.lse = o.lse_out;
  a.tm_offsets = (const uint32_t*)b;
  a.tm_desc = (const uint32_t*)(b + o_ds);
  a.mask_tbl = nullptr;
  a.B = B; a.H = H; a.d = d; a.n_text = n_text; a.gh = grid_h; a.gw = grid_w; a.r2 = g.r2;
  a.dtype = o.dtype; a.text_splits = splits; a.window = o.window;
  a.row_begin = 0;
  a.row_end = grid_h;
  if (splits > 1 && n_text > 0) {
    a.ws_o = (float*)(b + map_bytes);
    a.ws_ml = (float*)(b + map_bytes + (size_t)splits * align_up((size_t)B * H * n_text * d * 4, 256));
  }
  rc = tile_map_build_device_launch(g, (uint32_t*)b, (uint32_t*)(b + o_kt), (uint16_t*)(b + o_fl),
                                    (uint32_t*)(b + o_ds), stream);
  if (rc) return rc;
  rc = attn_launch(a, stream);
  if (rc) return rc;
  if (debug_sync_enabled()) {
    if ((e = hipStreamSynchronize(s)) != hipSuccess) return hip_fail(e, "CLEAR_DEBUG sync");
    if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "CLEAR_DEBUG check");
  }
  return CLEAR_OK;
}

extern "C" int clear_attn_fwd_strip(const void* q, const void* k, const void* v, void* out, int B,
                                    int H, int d, int n_text, int grid_h, int grid_w,
                                    const clear_opts* opts, int row_begin, int row_end,
                                    int with_text_keys, float* text_part_o, float* text_part_ml,
                                    void* stream) {
  clear_error_reset();
  StripArgs st{row_begin, row_end, with_text_keys, text_part_o, text_part_ml};
  return run_forward(q, k, v, out, B, H, d, n_text, grid_h, grid_w, opts, &st, stream);
}

extern "C" int clear_text_merge(const float* part_o, const float* part_ml, int nparts, int mode,
                                void* out, float* lse_out, int B, int H, int d, int n_text,
                                int grid_h, int grid_w, int dtype, void* stream) {
  clear_error_reset();
  if (!part_o || !part_ml || !out) return set_error(CLEAR_EINVAL, "part_o, part_ml and out must not be NULL");
  if (nparts < 1) return set_error(CLEAR_EINVAL, "nparts must be >= 1 (got %d)", nparts);
  if (mode != CLEAR_MERGE_EXACT && mode != CLEAR_MERGE_PATCH_AVERAGE)
    return set_error(CLEAR_EINVAL, "mode must be CLEAR_MERGE_EXACT or CLEAR_MERGE_PATCH_AVERAGE (got %d)", mode);
  if (mode == CLEAR_MERGE_PATCH_AVERAGE && lse_out)
    return set_error(CLEAR_EINVAL, "the patch average has no log-sum-exp; pass lse_out = NULL");
  if (B < 1 || H < 1) return set_error(CLEAR_EINVAL, "B and H must be >= 1 (got %d, %d)", B, H);
  if (d != 64 && d != 128) return set_error(CLEAR_EINVAL, "d must be 64 or 128 (got %d)", d);
  if (n_text < 0) return set_error(CLEAR_EINVAL, "n_text must be >= 0 (got %d)", n_text);
  if (grid_h < 1 || grid_w < 1 || grid_h > CLEAR_MAX_GRID || grid_w > CLEAR_MAX_GRID)
    return set_error(CLEAR_EINVAL, "grid sides must be in 1..%d (got %d x %d)", CLEAR_MAX_GRID, grid_h, grid_w);
  if (dtype != CLEAR_BF16 && dtype != CLEAR_FP32)
    return set_error(CLEAR_EINVAL, "dtype must be CLEAR_BF16 or CLEAR_FP32 (got %d)", dtype);
  const long long N = (long long)n_text + (long long)grid_h * grid_w;
  if (N > kMaxTokens) return set_error(CLEAR_EINVAL, "sequence too long (N = %lld; at most %lld)", N, kMaxTokens);
  int rc = text_merge_launch(part_o, part_ml, nparts, mode, out, lse_out, B * H, n_text, (int)N, d,
                             dtype, stream);
  if (rc) return rc;
  if (debug_sync_enabled()) {
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "CLEAR_DEBUG sync");
  }
  return CLEAR_OK;
}

extern "C" int clear_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int H,
                              int d, int n_text, int grid_h, int grid_w, int radius, void* stream) {
  clear_error_reset();
  if (radius < 0) return set_error(CLEAR_EINVAL, "radius must be >= 0 (got %d)", radius);
  long long r2 = (long long)radius * radius;
  if (r2 > 0x7fffffffLL) r2 = 0x7fffffffLL;
  clear_opts o{CLEAR_BF16, (int)r2, nullptr, 0, CLEAR_WINDOW_CIRCLE};
  return clear_attn_fwd_ex(q, k, v, out, B, H, d, n_text, grid_h, grid_w, &o, stream);
}

extern "C" int clear_tile_map_build_device_ex(int window, int grid_h, int grid_w, int r2_max,
                                              int tile_h, int tile_w, int sub_h, int sub_w, int key_h,
                                              int key_w, uint32_t* offsets, uint32_t* key_tiles,
                                              uint16_t* flags, size_t cap, size_t* n_entries,
                                              void* stream) {
  clear_error_reset();
  if (window != CLEAR_WINDOW_CIRCLE && window != CLEAR_WINDOW_SQUARE)
    return set_error(CLEAR_EINVAL, "window must be CLEAR_WINDOW_CIRCLE or CLEAR_WINDOW_SQUARE (got %d)",
                     window);
  int rc = tile_map_validate(grid_h, grid_w, r2_max, tile_h, tile_w, sub_h, sub_w, key_h, key_w);
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
  rc = tile_map_build_device_launch(g, offsets, key_tiles, flags, nullptr, stream);
  if (rc) return rc;
  if (debug_sync_enabled()) {
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "CLEAR_DEBUG sync");
  }
  return CLEAR_OK;
}

extern "C" int clear_tile_map_descriptors(int window, int grid_h, int grid_w, int r2_max, uint32_t* offsets,
                                          uint32_t* key_tiles, uint16_t* flags, uint32_t* desc, size_t cap,
                                          size_t* n_entries, void* stream) {
  clear_error_reset();
  if (window != CLEAR_WINDOW_CIRCLE && window != CLEAR_WINDOW_SQUARE)
    return set_error(CLEAR_EINVAL, "window must be CLEAR_WINDOW_CIRCLE or CLEAR_WINDOW_SQUARE (got %d)",
                     window);
  int rc = tile_map_validate(grid_h, grid_w, r2_max, CLEAR_TILE_H, CLEAR_TILE_W, CLEAR_SUB_H, CLEAR_SUB_W,
                             CLEAR_KEY_H, CLEAR_KEY_W);
  if (rc) return rc;
  if (!n_entries) return set_error(CLEAR_EINVAL, "n_entries must not be NULL");
  TileGeom g = make_geom(grid_h, grid_w, r2_max, CLEAR_TILE_H, CLEAR_TILE_W, CLEAR_SUB_H, CLEAR_SUB_W,
                         CLEAR_KEY_H, CLEAR_KEY_W, window);
  *n_entries = tile_map_count(g);
  rc = tile_map_check_entries(*n_entries);
  if (rc) return rc;
  if (*n_entries > cap)
    return set_error(CLEAR_ENOMEM, "tile map needs %zu entries (capacity %zu)", *n_entries, cap);
  if (!offsets || (*n_entries && (!key_tiles || !flags || !desc)))
    return set_error(CLEAR_EINVAL, "tile map output pointers must not be NULL");
  rc = tile_map_build_device_launch(g, offsets, key_tiles, flags, desc, stream);
  if (rc) return rc;
  if (debug_sync_enabled()) {
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "CLEAR_DEBUG sync");
  }
  return CLEAR_OK;
}

extern "C" int clear_tile_map_build_device(int grid_h, int grid_w, int r2_max, int tile_h, int tile_w,
                                           int sub_h, int sub_w, int key_h, int key_w, uint32_t* offsets,
                                           uint32_t* key_tiles, uint16_t* flags, size_t cap,
                                           size_t* n_entries, void* stream) {
  return clear_tile_map_build_device_ex(CLEAR_WINDOW_CIRCLE, grid_h, grid_w, r2_max, tile_h, tile_w,
                                        sub_h, sub_w, key_h, key_w, offsets, key_tiles, flags, cap,
                                        n_entries, stream);
}

extern "C" void clear_release_cache(void) {
  std::lock_guard<std::mutex> lock(g_mu);
  int cur = 0;
  (void)hipGetDevice(&cur);
  for (auto& kv : g_dev) {
    if (hipSetDevice(kv.first) != hipSuccess) continue;
    (void)hipDeviceSynchronize();
    for (auto& m : kv.second.maps) {
      if (m.second.ready) (void)hipEventDestroy(m.second.ready);
      (void)hipFree(m.second.block);
      if (m.second.mask_tbl) (void)hipFree(m.second.mask_tbl);
      delete m.second.mask_host;
    }
    kv.second.maps.clear();
    if (kv.second.ws) {
      (void)hipFreeAsync(kv.second.ws, nullptr);
      (void)hipDeviceSynchronize();
    }
    kv.second.ws = nullptr;
    kv.second.ws_bytes = 0;
    if (kv.second.ws_done) (void)hipEventDestroy(kv.second.ws_done);
    kv.second.ws_done = nullptr;
    kv.second.ws_stream = nullptr;
  }
  (void)hipSetDevice(cur);
}
