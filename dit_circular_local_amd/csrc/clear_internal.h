// clear_internal.h -- internal declarations shared by the library's host sources.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <vector>

#include "clear_attn.h"
#include "tile_geom.h"

namespace clear {

// Thread-local error message; returns `code` so callers can `return set_error(...)`.
int set_error(int code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
void clear_error_reset();
bool debug_sync_enabled();

int tile_map_validate(int gh, int gw, int r2, int th, int tw, int sh, int sw, int chunk);
void tile_map_counts(const TileGeom& g, size_t* n_runs, size_t* n_chunks,
                     std::vector<uint32_t>* tile_runs, std::vector<uint32_t>* tile_chunks);
void tile_map_fill_host(const TileGeom& g, uint32_t* run_offsets, uint32_t* runs,
                        uint32_t* chunk_offsets, uint16_t* flags);

// Device builder: enqueue the fill of a tile map whose sizes are known.
// `scratch` must hold (ntiles) uint32 for the per-tile counts.
int tile_map_build_device_launch(const TileGeom& g, uint32_t* run_offsets, uint32_t* runs,
                                 uint32_t* chunk_offsets, uint16_t* flags,
                                 uint32_t* scratch, void* stream);

// Attention launch description (all pointers are device pointers).
struct AttnLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  float* lse;                 // optional
  float* ws_o;                // text partials [splits][B*H][n_text][d]   (splits > 1)
  float* ws_ml;               // text partials [splits][B*H][n_text][2]   (splits > 1)
  const uint32_t* run_off;    // tile map
  const uint32_t* runs;
  const uint32_t* chunk_off;
  const uint16_t* flags;
  int B, H, d, n_text, gh, gw, r2;
  int dtype;
  int text_splits;
};

int attn_launch(const AttnLaunch& a, void* stream);

}  // namespace clear
