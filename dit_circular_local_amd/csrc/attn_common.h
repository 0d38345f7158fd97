// attn_common.h -- device code shared by the attention kernels (forward and
// backward): vector types, tile geometry, the 32x32 MFMA accumulator layout,
// the walk over a workgroup's chunks (dense token ranges, then the 4 x 8 cell
// tiles the tile map lists for its tile) and the per-element window mask.
//
// The mask is CLEAR's (pith.science review of arXiv 2412.16112, "Core claim"),
// 0-based: M_ij = [i < n_text] | [j < n_text] | [dy^2 + dx^2 <= r2]; the square
// window of "What carries the argument" tests max(dy^2, dx^2) <= r2 instead.
#pragma once

#include <hip/hip_runtime.h>

#include "clear_internal.h"

namespace clear {
namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;
typedef __attribute__((ext_vector_type(2))) float f32x2_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((address_space(4))) const u32x4_t const_u32x4_t;
typedef __attribute__((ext_vector_type(2))) short s16x2_t;
typedef __attribute__((ext_vector_type(4))) short s16x4_t;
typedef __attribute__((ext_vector_type(8))) short s16x8_t;
typedef __attribute__((address_space(3))) char lds_char_t;
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kTileH = CLEAR_TILE_H;
constexpr int kTileW = CLEAR_TILE_W;
constexpr int kSubH = CLEAR_SUB_H;
constexpr int kChunk = CLEAR_CHUNK;
constexpr int kKeyH = CLEAR_KEY_H;
constexpr int kKeyW = CLEAR_KEY_W;

static_assert(kTileH == kWaves * kSubH && kTileW == CLEAR_SUB_W && kTileW * kSubH == 32,
              "one 32-query sub-tile per wavefront");
static_assert(kChunk == 32, "chunk = one 32-row MFMA block");
static_assert(kKeyH * kKeyW == kChunk && kKeyW == 8,
              "key tile = one chunk; key cell (a, c) is chunk position 8a + c");


// Key position m (0..31) of accumulator register i in lane group g: the row
// index of the 32x32 accumulator layout.
__device__ __forceinline__ int acc_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// Wave-wide combine of a value with its partner lane l ^ 32.
__device__ __forceinline__ float max_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_elementwise_maximum(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_xor32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------- key sources

// Maps (chunk j, position p) to a key token for the current workgroup.
// Chunks 0 .. n_dense-1 come from one or two dense token ranges (the text keys
// of an image tile; a key range of a text workgroup; or the text keys and one
// strip's image rows); chunk n_dense + e is the e-th key
// tile the tile map lists for the query tile, position p = 8a + c being its
// key cell (ky0 + a, kx0 + c).
typedef __attribute__((address_space(4))) const uint32_t const_u32_t;

struct KeySource {
  // dense chunks 0 .. n_dense1-1 cover tokens [dense_base, dense_limit), chunks
  // n_dense1 .. n_dense-1 cover [dense2_base, dense2_limit)
  int dense_base, dense_limit, n_dense1, dense2_base, dense2_limit, n_dense;
  int n_text, gh, gw;
  int e0;                // the query tile's first tile-map entry
  int window;            // 0 circle, 1 square
  int n_tok;             // tokens per head (N)
  const_u32x4_t* desc;   // tile-map entry descriptors, read through the scalar cache
};

// Buffer resource over `bytes` bytes from a uniform address (gfx9 resource
// word 3).  Loads at offsets >= bytes return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t byte_rsrc(const char* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), (short)0, (int)bytes, 0x00020000);
}

// Buffer resource words (gfx9 layout, stride 0) over `bytes` bytes from a
// uniform address: offsets at or past `bytes` read zeros.
__device__ __forceinline__ u32x4_t rsrc_words(const char* base, uint32_t bytes) {
  const uint64_t a = (uint64_t)(uintptr_t)base;
  return u32x4_t{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// One wavefront's direct-to-LDS copy of 64 x 16 bytes: lane l's piece at byte
// voff of the resource lands at LDS address lds + 16 l.  Written in assembly so
// that the compiler does not take it for a writer of the stage being read (it
// cannot tell the two stages apart and would wait for the next chunk's copies
// before the reads of the current one); the walk waits for the copies itself,
// before each barrier (stage_barrier).
__device__ __forceinline__ void lds_copy(uint32_t lds, const u32x4_t& rsrc, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc) : "memory");
}

__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(lds_char_t*)const_cast<char*>(p);
}

// As lds_copy, 64 x 4 bytes: lane l's word lands at lds + 4 l.
__device__ __forceinline__ void lds_copy_dword(uint32_t lds, const u32x4_t& rsrc, uint32_t voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :: "s"(lds), "v"(voff), "s"(rsrc) : "memory");
}

// Per-chunk description, uniform: where the chunk's keys start, and what the
// mask needs.
struct ChunkMeta {
  int tok0;       // first key token of the chunk
  int left;       // tokens from tok0 to the end of the head
  int limit;      // dense chunks: end of the chunk's token range
  unsigned flag;  // tile-map flags and kTileInside (0 for dense chunks)
  unsigned kt;    // key tiles: (row << 16) | column of the tile
};

// Chunk j >= n_dense: entry j - n_dense of the query tile's key-tile list,
// from its descriptor (one scalar load).
__device__ __forceinline__ ChunkMeta tile_chunk_meta(const KeySource& ks, int j) {
  const u32x4_t d = ks.desc[ks.e0 + j - ks.n_dense];
  return ChunkMeta{ks.n_text + (int)d[0], (int)d[3], 0, d[1], d[2]};
}

__device__ __forceinline__ ChunkMeta chunk_meta(const KeySource& ks, int j) {
  if (j >= ks.n_dense) return tile_chunk_meta(ks, j);
  const bool first = j < ks.n_dense1;
  const int tok0 = first ? ks.dense_base + j * kChunk : ks.dense2_base + (j - ks.n_dense1) * kChunk;
  return ChunkMeta{tok0, ks.n_tok - tok0, first ? ks.dense_limit : ks.dense2_limit, 0u, 0u};
}

// Offset of a padding slot: past any buffer bound, so its load returns zeros.
constexpr uint32_t kNoPiece = 0xfffffff0u;

typedef __attribute__((address_space(3))) void lds_void_t;

// What one wavefront does with chunk j: whether it computes it at all, and
// which mask applies (tail of a dense range, or the circular window).
struct ChunkInfo {
  bool active;
  bool coord;
  bool square;  // square-window variant
  bool inside;  // key tile wholly on the grid
  int tail;     // dense chunk: positions >= tail are masked
  int kty, ktx; // key tile's row and column (key-tile chunks)
  int ky0, kx0; // its first cell
};

// A dense chunk: every wavefront computes it; positions past the range's
// limit are masked.
__device__ __forceinline__ ChunkInfo dense_chunk_info(const ChunkMeta& m, const KeySource& ks) {
  const int rem = m.limit - m.tok0;
  return ChunkInfo{true, false, ks.window == 1, true, rem < kChunk ? rem : kChunk, 0, 0, 0, 0};
}

// A key tile: computed by the wavefronts whose sub-tile touches it, masked
// by coordinates unless the sub-tile admits all of it.
__device__ __forceinline__ ChunkInfo tile_chunk_info(const ChunkMeta& m, const KeySource& ks, int wave) {
  const int kty = (int)(m.kt >> 16), ktx = (int)(m.kt & 0xffffu);
  return ChunkInfo{((m.flag >> wave) & 1u) != 0, ((m.flag >> (8 + wave)) & 1u) == 0, ks.window == 1,
                   (m.flag & kTileInside) != 0, kChunk, kty, ktx, kty * kKeyH, ktx * kKeyW};
}

// Barrier of the chunk walk.  Direct-to-LDS copies are vector-memory loads
// that write LDS: the compiler orders them only against the same wavefront's
// later LDS reads, and the barrier's fence need not wait for them, so a
// wavefront could pass the barrier with its last copy still landing while the
// others start reading that stage.  Each wavefront therefore first waits for
// all of its own copies (vmcnt(0)); after the barrier every wavefront's copies
// of the stage are complete.
__device__ __forceinline__ void stage_barrier() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// The chunk walk of the attention kernels.  Two LDS stages: after the
// barrier of iteration j, chunk j is in its stage (the copies were issued in
// iteration j - 1, and stage_barrier has every wavefront wait for its own),
// and every wavefront is done with chunk j - 1, so the copies of chunk j + 1
// go to the other stage while chunk j is computed.  The descriptor of chunk j + 2 is
// fetched in iteration j, so its scalar load is complete when needed.
//   stage(st, meta, dense) issues the copies of a chunk into stage st;
//   compute(info, st) computes the chunk held in st.
// The dense chunks come first (text keys, or all of a text workgroup's
// chunks; the one after the last may be a key tile).  Each kind of chunk has
// a loop of its own that carries only its own state and tests, and the key
// tiles go two per trip so that the stages and the two descriptors in flight
// keep fixed roles: in tile_step, mc describes chunk jj (in cur), mn chunk
// jj + 1 (copied to nxt), and mc then receives chunk jj + 2.  The dense loop
// also goes two chunks per trip; its odd last chunk swaps the roles.
template <class Stage, class Compute>
__device__ __forceinline__ void walk_chunks(const KeySource& ks, int n, int wave, char* st_cur, char* st_nxt,
                                            Stage&& stage, Compute&& compute) {
  if (n <= 0) return;
  ChunkMeta m_cur = chunk_meta(ks, 0);
  ChunkMeta m_nxt = chunk_meta(ks, n > 1 ? 1 : 0);
  stage(st_cur, m_cur, 0 < ks.n_dense);
  auto dense_step = [&](int jj, ChunkMeta& mc, const ChunkMeta& mn, const char* cur, char* nxt) {
    stage_barrier();
    if (jj + 1 < n) stage(nxt, mn, jj + 1 < ks.n_dense);
    const ChunkInfo c = dense_chunk_info(mc, ks);
    mc = chunk_meta(ks, jj + 2 < n ? jj + 2 : n - 1);
    compute(c, cur);
  };
  int j = 0;
  for (; j + 1 < ks.n_dense; j += 2) {
    dense_step(j, m_cur, m_nxt, st_cur, st_nxt);
    dense_step(j + 1, m_nxt, m_cur, st_nxt, st_cur);
  }
  for (; j < ks.n_dense; ++j) {
    dense_step(j, m_cur, m_nxt, st_cur, st_nxt);  // m_cur now describes chunk j + 2
    const ChunkMeta m = m_cur;
    m_cur = m_nxt;
    m_nxt = m;
    char* t = st_cur;
    st_cur = st_nxt;
    st_nxt = t;
  }
  auto tile_step = [&](int jj, ChunkMeta& mc, const ChunkMeta& mn, const char* cur, char* nxt) {
    stage_barrier();
    if (jj + 1 < n) stage(nxt, mn, false);
    const ChunkInfo c = tile_chunk_info(mc, ks, wave);
    mc = tile_chunk_meta(ks, jj + 2 < n ? jj + 2 : n - 1);
    compute(c, cur);
  };
  for (; j + 1 < n; j += 2) {
    tile_step(j, m_cur, m_nxt, st_cur, st_nxt);
    tile_step(j + 1, m_nxt, m_cur, st_nxt, st_cur);
  }
  if (j < n) tile_step(j, m_cur, m_nxt, st_cur, st_nxt);
}

// The lane-mask table of partly admitted chunks (built on the host next to
// the tile map): for a chunk tile at offset (dy, dx) = (4 iy, 8 ix) from the
// wavefront's sub-tile, word i has bit l set iff register i of lane l is
// admitted.  Read through the scalar cache; each word is a lane mask.
typedef __attribute__((address_space(4))) const uint64_t const_u64_t;

struct MaskTable {
  const_u64_t* tbl;  // null: no table (masks computed per element)
  int ky, kx;        // |iy| <= ky, |ix| <= kx
};

// Apply the sixteen lane masks at w (word i masks register i).
__device__ __forceinline__ void apply_lane_masks(f32x16_t& s, const_u64_t* w) {
  for (int i = 0; i < 16; ++i) s[i] = __builtin_amdgcn_inverse_ballot_w64(w[i]) ? s[i] : -__builtin_inff();
}

// Table row of a wavefront whose sub-tile starts at cell (sy0, sx0), a
// multiple of (4, 8): the words of key tile (kty, ktx) start at entry
// kty * (2 kx + 1) + ktx + table_base(mt, sy0, sx0).
__device__ __forceinline__ int table_base(const MaskTable& mt, int sy0, int sx0) {
  return (mt.ky - (sy0 >> 2)) * (2 * mt.kx + 1) + mt.kx - (sx0 >> 3);
}

// The window mask of one chunk, in place on 32x32 accumulator values s whose
// rows are the chunk's 32 positions (register i of lane group g is position
// acc_row(i, g)) and whose column is the lane's own cell (cy, cx).  A dense
// chunk masks positions >= tail; a key-tile chunk that is not wholly admitted
// masks by coordinates: position 8a + c is cell (ky0 + a, kx0 + c), admitted
// iff dx^2 <= lim[a], lim = r2 - dy^2 (circle) or lim = dy^2 <= r2 ? r2 : -1
// (square), with the chunk's cell on the grid.  The distance is symmetric, so
// the same code serves a query column against key rows and a key column
// against query rows.
__device__ __forceinline__ void mask_chunk(f32x16_t& s, const ChunkInfo& c, const KeySource& ks, int g,
                                           int cy, int cx, int r2) {
  if (c.tail < 32) {
    for (int i = 0; i < 16; ++i) s[i] = acc_row(i, g) >= c.tail ? -__builtin_inff() : s[i];
  } else if (c.coord) {
    int lim[4], dxx[4];
    const int dy0 = cy - c.ky0, dx0 = cx - c.kx0 - 4 * g;
    if (c.square) {
      for (int a = 0; a < 4; ++a) lim[a] = __mul24(dy0 - a, dy0 - a) <= r2 ? r2 : -1;
    } else {
      for (int a = 0; a < 4; ++a) lim[a] = r2 - __mul24(dy0 - a, dy0 - a);
    }
    for (int b = 0; b < 4; ++b) dxx[b] = __mul24(dx0 - b, dx0 - b);
    if (!c.inside) {
      for (int a = 0; a < 4; ++a)
        if (c.ky0 + a >= ks.gh) lim[a] = -1;
      for (int b = 0; b < 4; ++b)
        if (c.kx0 + 4 * g + b >= ks.gw) dxx[b] = 0x7fffffff;
    }
    for (int i = 0; i < 16; ++i) s[i] = dxx[i & 3] > lim[i >> 2] ? -__builtin_inff() : s[i];
  }
}

}  // namespace
}  // namespace clear
