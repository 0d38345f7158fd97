// clear_internal.h -- internal declarations shared by the library's host sources.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include "clear_attn.h"
#include "tile_geom.h"

namespace clear {

// Thread-local error message; returns `code` so callers can `return set_error(...)`.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error_reset();
bool debug_sync_enabled();

int tile_map_validate(int gh, int gw, int r2, int th, int tw, int sh, int sw, int kh, int kw);
size_t tile_map_count(const TileGeom& g);
// CLEAR_ENOTSUP (with the message set) when a map of n_entries entries does
// not fit the 32-bit offsets of the exported layout.
int tile_map_check_entries(size_t n_entries);
// Largest accepted N = n_text + grid_h * grid_w: token indices, and N rounded
// up to whole 32-key chunks, stay in 32-bit signed range in host and kernels.
constexpr long long kMaxTokens = 0x7fffffffLL - 4096;
// The attention kernels index entries with 32-bit signed arithmetic.
constexpr int kMaxKernelEntries = 0x7fffffff;
// Fills the map (entries past cap are counted, not written); returns the
// number of entries listed, which equals tile_map_count(g).
size_t tile_map_fill_host(const TileGeom& g, uint32_t* offsets, uint32_t* key_tiles, uint16_t* flags,
                          size_t cap);

// Lane-mask table of partly admitted chunks (tilemap_host.cpp): entries for
// tile offsets D = (4 iy, 8 ix), |iy| <= ky, |ix| <= kx, 16 words each.  Not
// built (false) for r2 < 0 or radii above kMaskTableMaxRadius.
constexpr int kMaskTableMaxRadius = 256;
bool mask_table_dims(const TileGeom& g, int& ky, int& kx);
void mask_table_fill(const TileGeom& g, int ky, int kx, uint64_t* out);

// Device builder: enqueue the kernels that fill offsets / key_tiles / flags
// (capacity already checked against tile_map_count).
// desc (optional, 4 words per entry): the entry's descriptor for the attention
// kernels, read through the scalar cache in one load --
//   [0] token offset of the key tile's first cell from the first image token
//       (ky * key_h * gw + kx * key_w),
//   [1] the entry's flags, plus kTileInside when the key tile lies wholly on
//       the grid,
//   [2] (ky << 16) | kx, the key tile's row and column (16 bits each suffice:
//       grid sides are at most CLEAR_MAX_GRID),
//   [3] image tokens from the first cell to the end of the grid.
constexpr uint32_t kTileInside = 1u << 16;
int tile_map_build_device_launch(const TileGeom& g, uint32_t* offsets, uint32_t* key_tiles,
                                 uint16_t* flags, uint32_t* desc, void* stream);

// Attention launch description (all pointers are device pointers).
struct AttnLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;                 // optional
  float* ws_o;                // text partials [splits][B*H][n_text][d]   (splits > 1)
  float* ws_ml;               // text partials [splits][B*H][n_text][2]   (splits > 1)
  const uint32_t* tm_offsets;  // tile map: entry range of each query tile
  const uint32_t* tm_desc;     //   and each entry's descriptor
  const uint64_t* mask_tbl;   // lane-mask table (NULL: masks computed per element)
  int mt_ky, mt_kx;
  int B, H, d, n_text, gh, gw, r2;
  int dtype;
  int text_splits;
  int window;                 // CLEAR_WINDOW_CIRCLE or CLEAR_WINDOW_SQUARE
  int row_begin, row_end;     // image rows computed (0, gh for the whole layer)
  int strip;                  // text rows: write the strip's partial to ws_o / ws_ml
  int strip_text_keys;        //   ... including the text keys
};

int attn_launch(const AttnLaunch& a, void* stream);

// Text-row split count of the layer entry points (clear_attn.cpp).
int choose_text_splits(int B, int H, int n_text, int N, int ntiles, size_t img_chunks, int n_cu,
                       double waves_per_simd = 3.0, bool fill_slots = false);

// Device address of the allocation-free entry point's scratch on device dev
// (noalloc.hip): CLEAR_NOALLOC_SCRATCH_BYTES bytes, looked up on the first call
// for the device, which must be current.
int noalloc_scratch(int dev, void** ptr);

// Backward launch description (all pointers are device pointers).
struct BwdLaunch {
  const void* q;
  const void* k;
  const void* v;
  const void* out;    // forward output O
  const void* dout;   // upstream gradient dO
  const float* lse;   // forward LSE [B*H][N], natural log
  void* dq;
  void* dk;
  void* dv;
  float* ws_stats;    // [B*H][N][2]: (lse * log2(e), -(dO . O))
  float* ws_dq;       // text partials [splits][B*H][n_text][d]   (n_text > 0)
  float* ws_dk;
  float* ws_dv;
  const uint32_t* tm_offsets;
  const uint32_t* tm_desc;
  const uint64_t* mask_tbl;   // lane-mask table (NULL: masks computed per element)
  int mt_ky, mt_kx;
  int B, H, d, n_text, gh, gw, r2;
  int dtype;
  int text_splits;
  int window;
};

int attn_bwd_launch(const BwdLaunch& a, void* stream);
int text_merge_launch(const float* part_o, const float* part_ml, int nparts, int mode, void* out,
                      float* lse, int BH, int n_text, int N, int d, int dtype, void* stream);

}  // namespace clear
