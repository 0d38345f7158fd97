// attn_fwd.hip -- fused CLEAR attention forward for gfx950 (MI355X).
//
// What is computed: masked softmax attention with CLEAR's circular-window mask
// (pith.science review of arXiv 2412.16112, "Core claim"; 0-based,
// M_ij = [i < n_text] | [j < n_text] | [dy^2 + dx^2 <= r2]), logits
// scaled by 1/sqrt(d) (the review's Eq. 1 / Eq. 7), text queries attending to
// every key (the review's referee summary: text-token attention stays global).
//
// Work decomposition (one launch):
//  * image workgroups: 256 threads = 4 wavefronts own a 16 x 8 cell query tile,
//    each wavefront a 4 x 8 sub-tile (32 queries).  Keys stream through LDS in
//    chunks of 32: first the text keys, then the 4 x 8 cell key tiles the tile
//    map lists for the query tile.  A wavefront skips key tiles its sub-tile does
//    not touch and applies the per-element circular mask only to key tiles it
//    does not fully admit: the mask (0 or -inf per element, from a small table
//    of lane masks indexed by the tile's offset from the sub-tile) is the Q.K
//    product's initial accumulator;
//  * text workgroups: 128 text queries against a contiguous range of all keys
//    (the range is one of `splits` parts; partial results are merged exactly by
//    log-sum-exp in a second kernel when splits > 1).
//
// Matrix-core formulation (per wavefront, per chunk of 32 keys):
//    S^T[key][query] = K[key][:] . Q[query][:]          A = K (LDS), B = Q^T (VGPRs)
//    O^T[d][query]  += V^T[d][key] . P^T[key][query]    A = V^T (LDS), B = P^T (VGPRs)
// With the 32x32 accumulator layout, lane l holds 16 keys of query l % 32, so
// the softmax row statistics are per lane (plus an exchange with lane l ^ 32
// when the reference max moves) and the rescaling of O^T is per lane.  bf16 uses v_mfma_f32_32x32x16_bf16 with
// V^T read from row-major V by the LDS transpose load ds_read_b64_tr_b16; fp32
// uses v_mfma_f32_32x32x2_f32.
//
// Pipeline (walk_chunks): two LDS stages and one workgroup barrier per chunk.
// Each chunk goes from global memory straight into LDS (direct-to-LDS buffer
// loads issued by all four wavefronts) one iteration before it is consumed, so
// the copy of chunk j + 1 overlaps the computation on chunk j; each key tile's
// 16-byte tile-map descriptor arrives by one scalar load two chunks ahead.
// Three wavefronts per SIMD (bf16) hide the remaining latency.
//
// Online softmax in base 2 with a lazily updated reference max: p = 2^(s*c - M)
// with c = log2(e)/sqrt(d); M is raised only when a row max exceeds M + 8, so
// p <= 256 and O / L is unchanged (softmax is invariant to the reference).
#include "attn_common.h"

namespace clear {
namespace {

constexpr int kTextQ = kWaves * 32;  // text queries per workgroup
constexpr float kLazyTau = 8.0f;
constexpr float kMInit = -1.0e30f;

struct Params {
  const char* q;
  const char* k;
  const char* v;
  char* out;
  float* lse;
  float* ws_o;
  float* ws_ml;
  const uint32_t* tm_offsets;
  const uint32_t* tm_desc;
  const uint64_t* mask_tbl;  // lane masks of partly admitted chunks (null: computed)
  int mt_ky, mt_kx;
  int N, n_text, gh, gw, r2, window;
  int ntiles, ntx;
  int n_text_blocks, splits, chunks_per_split;
  int n_text_wg, n_text_wg_pad, n_img_wg, BH;
  // image rows computed: [row_begin, row_end), i.e. query-tile rows
  // band_ty0 .. band_ty0 + band_tiles / ntx - 1 (the whole grid unless a strip)
  int row_begin, row_end, band_ty0, band_tiles;
  // text rows: a strip's partial (text keys if strip_text_keys, then the image
  // keys of rows [row_begin, row_end)) instead of key-range splits
  int text_strip, strip_text_keys;
  int partial_out;  // text workgroups write unnormalised partials (O, M, L)
  float scale_log2;
};

// ---------------------------------------------------------------- engines

// bf16 inputs; K and V row-major in LDS (different row pitches: K is read
// row-per-lane by ds_read_b128, V by 16-lane transpose loads).
template <int D>
struct Bf16 {
  static constexpr int kElem = 2;
  static constexpr int kRowBytes = D * 2;       // global row
  static constexpr int kPPR = D / 8;            // 16-byte pieces per row
  static constexpr int kSlotsK = kPPR + 1;      // LDS row pitch in 16-byte slots (K)
  static constexpr int kSlotsV = kPPR + 4;      // (V: transpose reads need a wider pad)
  static constexpr int kKK = D / 16;
  static constexpr int kNB = D / 32;
  static constexpr int kWavesPerSimd = 3;
  static constexpr int kStages = 2;

  static constexpr int kRowK = kSlotsK * 16;
  static constexpr int kRowV = kSlotsV * 16;
  // 1 KB direct-to-LDS blocks per region, a multiple of the wavefront count
  static constexpr int kBlocksK = (kChunk * kSlotsK + 64 * kWaves - 1) / (64 * kWaves) * kWaves;
  static constexpr int kBlocksV = (kChunk * kSlotsV + 64 * kWaves - 1) / (64 * kWaves) * kWaves;
  static constexpr int kKOff = 0;
  static constexpr int kVOff = kBlocksK * 1024;
  static constexpr int kStage = kVOff + kBlocksV * 1024;

  bf16x8_t q[kKK];
  f32x16_t o[kNB];

  // qrow is always a valid row (invalid queries read row 0 and are zeroed), so
  // every lane issues the same loads.
  __device__ void load_q(const char* qrow, bool valid, int g) {
    for (int kk = 0; kk < kKK; ++kk) {
      const u32x4_t x = *(const u32x4_t*)(qrow + (16 * kk + 8 * g) * 2);
      q[kk] = __builtin_bit_cast(bf16x8_t, valid ? x : u32x4_t{0, 0, 0, 0});
    }
  }
  __device__ void zero_o() {
    for (int nb = 0; nb < kNB; ++nb) o[nb] = f32x16_t{};
  }
  __device__ void scale_o(float a) {
    for (int nb = 0; nb < kNB; ++nb)
      for (int i = 0; i < 16; ++i) o[nb][i] *= a;
  }
  // Waits for the Q loads here, once, so that no wait for them is left
  // inside the chunk loop (where it would also wait for the prefetches).
  __device__ void settle_q() {
    for (int kk = 0; kk < kKK; ++kk) asm volatile("" ::"v"(q[kk]));
  }
  __device__ void qk(const char* st, int lane, f32x16_t& s, const f32x16_t& init) const {
    const char* kb = st + kKOff + (lane & 31) * kRowK + (lane >> 5) * 16;
    s = init;
    for (int kk = 0; kk < kKK; ++kk) {
      bf16x8_t a = *(const bf16x8_t*)(kb + kk * 32);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q[kk], s, 0, 0, 0);
      // at most four operands in flight (register budget of three waves per SIMD)
      if (kk % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
  }
  // Probabilities as the B operand of P.V (bf16, registers 8t .. 8t+7 in
  // operand t) and their sum, taken over the rounded values P.V uses.
  struct Probs {
    bf16x8_t b[2];
  };
  __device__ static void probs(const f32x16_t& e, Probs& pr, float& l) {
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    for (int t = 0; t < 2; ++t)
      for (int j = 0; j < 4; ++j) {
        const bf16x2_t h = __builtin_convertvector(f32x2_t{e[8 * t + 2 * j], e[8 * t + 2 * j + 1]}, bf16x2_t);
        pr.b[t][2 * j] = h[0];
        pr.b[t][2 * j + 1] = h[1];
        l = __builtin_amdgcn_fdot2_f32_bf16(h, one, l, false);
      }
  }
  // O^T += V^T P^T.  The A operand (lane l: d = 32*nb + l % 32, eight keys of
  // lane group g = l / 32) comes from two transpose loads: in each 16-lane group,
  // lane i receives element i % 4 of the 8-byte rows addressed by lanes i/4,
  // i/4 + 4, i/4 + 8, i/4 + 12.  Lane s of a group therefore addresses key row
  // 16t + 8h + 4g + s/4 (h = 0, 1 for the two loads) at columns
  // 32nb + 16*((l/16) % 2) + 4*(s % 4): lane i then holds keys
  // 16t + 8h + 4g + e (e = 0..3) at d = 32nb + l % 32, which are the keys of
  // accumulator registers 8t + 4h + e (acc_row) whose probabilities the B
  // operand carries.
  __device__ void pv(const char* st, int lane, const Probs& pr) {
    const int g = lane >> 5;
    const int s = lane & 15;
    const int half = (lane >> 4) & 1;
    const char* vb = st + kVOff + (4 * g + (s >> 2)) * kRowV + (16 * half + 4 * (s & 3)) * 2;
    for (int t = 0; t < 2; ++t) {
      for (int nb = 0; nb < kNB; ++nb) {
        const char* a0 = vb + 16 * t * kRowV + nb * 64;
        s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds_char_t*)const_cast<char*>(a0));
        s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(lds_char_t*)const_cast<char*>(a0 + 8 * kRowV));
        s16x8_t w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), pr.b[t], o[nb], 0, 0, 0);
        if (nb % 2 == 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  __device__ static void store4(char* dst, float a, float b, float c, float d) {
    bf16x2_t h0 = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
    bf16x2_t h1 = __builtin_convertvector(f32x2_t{c, d}, bf16x2_t);
    uint2 w;
    w.x = __builtin_bit_cast(unsigned, h0);
    w.y = __builtin_bit_cast(unsigned, h1);
    *(uint2*)dst = w;
  }
};

// bf16 inputs at d = 128.  K and V sit in LDS in copy
// blocks: one direct-to-LDS copy of a wavefront (64 lanes x 16 bytes) fills one
// 1 KB block holding four whole 256-byte rows.  A row is four 64-byte granules
// (four 16-byte pieces each); within a block, granule c of row j sits at
// bytes 256 c + 64 j, so lane l of the copy reads granule l / 16 of row
// (l / 4) % 4, piece l % 4 of it: every four consecutive lanes read 64
// contiguous bytes of global memory.  Consecutive blocks start one 16-byte
// bank group further round the LDS (pitch 1040 bytes), so that
//  * the row-per-lane K reads (ds_read_b128, eight or sixteen consecutive
//    rows, one piece index) hit distinct bank groups: 4 j + v within a
//    block, plus the block's skew;
//  * the V transpose reads (ds_read_b64_tr_b16: per 16-lane group four rows of
//    a block, two pieces each) read 128 distinct bytes;
//  * a piece's offset from the row's first piece is the same on every lane
//    (256 bytes per granule, 16 per piece), so one lane address and
//    immediate offsets serve every product.
// No slot is padding: a chunk is 16 copies (4 per wavefront), 16 KB of LDS
// writes, where a row pitch of 17 or 20 slots takes 24.
struct Bf16G {
  static constexpr int D = 128;
  static constexpr int kElem = 2;
  static constexpr int kRowBytes = D * 2;          // global row
  static constexpr int kRowsPerBlock = 4;
  static constexpr int kBlocks = kChunk / kRowsPerBlock;  // copy blocks per region (K or V)
  static constexpr int kBlocksPerWave = kBlocks / kWaves;
  static constexpr int kPitch = 1024 + 16;         // block pitch: one bank group of skew
  static constexpr int kKK = D / 16;
  static constexpr int kNB = D / 32;
  static constexpr int kWavesPerSimd = 3;
  static constexpr int kStages = 2;
  static constexpr int kKOff = 0;
  static constexpr int kVOff = kBlocks * kPitch;
  static constexpr int kStage = 2 * kBlocks * kPitch;
  static_assert(kBlocks % kWaves == 0, "copy blocks split evenly over the wavefronts");

  // LDS byte offset, within a region, of element `col` of chunk row `row`
  __device__ static constexpr int lds_off(int row, int col) {
    return (row / 4) * kPitch + 256 * (col / 32) + 64 * (row % 4) + 16 * ((col / 8) % 4) + 2 * (col % 8);
  }

  bf16x8_t q[kKK];
  f32x16_t o[kNB];

  __device__ void load_q(const char* qrow, bool valid, int g) {
    for (int kk = 0; kk < kKK; ++kk) {
      const u32x4_t x = *(const u32x4_t*)(qrow + (16 * kk + 8 * g) * 2);
      q[kk] = __builtin_bit_cast(bf16x8_t, valid ? x : u32x4_t{0, 0, 0, 0});
    }
  }
  __device__ void zero_o() {
    for (int nb = 0; nb < kNB; ++nb) o[nb] = f32x16_t{};
  }
  __device__ void scale_o(float a) {
    for (int nb = 0; nb < kNB; ++nb)
      for (int i = 0; i < 16; ++i) o[nb][i] *= a;
  }
  __device__ void settle_q() {
    for (int kk = 0; kk < kKK; ++kk) asm volatile("" ::"v"(q[kk]));
  }
  // K rows: lane l reads row l % 32, piece 2 kk + l / 32 (d values
  // 16 kk + 8 (l / 32) .. + 7) for product kk: granule kk / 2, piece
  // 2 (kk % 2) + l / 32 within it.
  __device__ void qk(const char* st, int lane, f32x16_t& s, const f32x16_t& init) const {
    const char* kb = st + kKOff + lds_off(lane & 31, 8 * (lane >> 5));
    s = init;
    for (int kk = 0; kk < kKK; ++kk) {
      bf16x8_t a = *(const bf16x8_t*)(kb + 256 * (kk / 2) + 32 * (kk % 2));
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q[kk], s, 0, 0, 0);
      // at most four operands in flight (register budget of three waves per SIMD)
      if (kk % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
  }
  struct Probs {
    bf16x8_t b[2];
  };
  __device__ static void probs(const f32x16_t& e, Probs& pr, float& l) {
    const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
    for (int t = 0; t < 2; ++t)
      for (int j = 0; j < 4; ++j) {
        const bf16x2_t h = __builtin_convertvector(f32x2_t{e[8 * t + 2 * j], e[8 * t + 2 * j + 1]}, bf16x2_t);
        pr.b[t][2 * j] = h[0];
        pr.b[t][2 * j + 1] = h[1];
        l = __builtin_amdgcn_fdot2_f32_bf16(h, one, l, false);
      }
  }
  // O^T += V^T P^T, the A operand from transpose loads as in the padded
  // engine: lane s of a 16-lane group addresses key row 16t + 8h + 4g + s/4 at
  // columns 32nb + 16 ((l/16) % 2) + 4 (s % 4).  Rows 16t + 8h further are
  // 4t + 2h blocks further, columns 32nb further one granule (256 bytes)
  // further, so the lane address of (t, h, nb) = (0, 0, 0) serves all.
  __device__ void pv(const char* st, int lane, const Probs& pr) {
    const int g = lane >> 5;
    const int s = lane & 15;
    const int half = (lane >> 4) & 1;
    const char* vb = st + kVOff + lds_off(4 * g + (s >> 2), 16 * half + 4 * (s & 3));
    for (int t = 0; t < 2; ++t) {
      for (int nb = 0; nb < kNB; ++nb) {
        const char* a0 = vb + 4 * t * kPitch + 256 * nb;
        s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds_char_t*)const_cast<char*>(a0));
        s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(lds_char_t*)const_cast<char*>(a0 + 2 * kPitch));
        s16x8_t w = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, w), pr.b[t], o[nb], 0, 0, 0);
        if (nb % 2 == 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  __device__ static void store4(char* dst, float a, float b, float c, float d) {
    bf16x2_t h0 = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
    bf16x2_t h1 = __builtin_convertvector(f32x2_t{c, d}, bf16x2_t);
    uint2 w;
    w.x = __builtin_bit_cast(unsigned, h0);
    w.y = __builtin_bit_cast(unsigned, h1);
    *(uint2*)dst = w;
  }
};

// fp32 inputs; K and V row-major in LDS.
template <int D>
struct F32 {
  static constexpr int kElem = 4;
  static constexpr int kRowBytes = D * 4;
  static constexpr int kPPR = D / 4;
  static constexpr int kSlotsK = kPPR + 1;
  static constexpr int kSlotsV = kPPR + 1;
  static constexpr int kHalf = D / 2;   // d values per lane group in Q.K
  static constexpr int kNB = D / 32;
  static constexpr int kWavesPerSimd = 1;
  static constexpr int kStages = 2;

  static constexpr int kRowK = kSlotsK * 16;
  static constexpr int kRowV = kSlotsV * 16;
  static constexpr int kBlocksK = (kChunk * kSlotsK + 64 * kWaves - 1) / (64 * kWaves) * kWaves;
  static constexpr int kBlocksV = (kChunk * kSlotsV + 64 * kWaves - 1) / (64 * kWaves) * kWaves;
  static constexpr int kKOff = 0;
  static constexpr int kVOff = kBlocksK * 1024;
  static constexpr int kStage = kVOff + kBlocksV * 1024;

  float q[kHalf];
  f32x16_t o[kNB];

  __device__ void load_q(const char* qrow, bool valid, int g) {
    for (int s4 = 0; s4 < kHalf / 4; ++s4) {
      const f32x4_t x = *(const f32x4_t*)(qrow + (kHalf * g + 4 * s4) * 4);
      for (int e = 0; e < 4; ++e) q[4 * s4 + e] = valid ? x[e] : 0.0f;
    }
  }
  __device__ void zero_o() {
    for (int nb = 0; nb < kNB; ++nb) o[nb] = f32x16_t{};
  }
  __device__ void scale_o(float a) {
    for (int nb = 0; nb < kNB; ++nb)
      for (int i = 0; i < 16; ++i) o[nb][i] *= a;
  }
  __device__ void settle_q() {
    for (int i = 0; i < kHalf; ++i) asm volatile("" ::"v"(q[i]));
  }
  __device__ void qk(const char* st, int lane, f32x16_t& s, const f32x16_t& init) const {
    const char* kb = st + kKOff + (lane & 31) * kRowK + (lane >> 5) * kHalf * 4;
    s = init;
    for (int s4 = 0; s4 < kHalf / 4; ++s4) {
      f32x4_t a = *(const f32x4_t*)(kb + s4 * 16);
      for (int e = 0; e < 4; ++e)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], q[4 * s4 + e], s, 0, 0, 0);
    }
  }
  struct Probs {
    f32x16_t p;
  };
  __device__ static void probs(const f32x16_t& e, Probs& pr, float& l) {
    for (int i = 0; i < 16; ++i) l += e[i];
    pr.p = e;
  }
  __device__ void pv(const char* st, int lane, const Probs& pr) {
    const f32x16_t& p = pr.p;
    const int g = lane >> 5;
    for (int u = 0; u < 16; ++u) {
      const float* vr = (const float*)(st + kVOff + acc_row(u, g) * kRowV) + (lane & 31);
      for (int nb = 0; nb < kNB; ++nb)
        o[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[32 * nb], p[u], o[nb], 0, 0, 0);
    }
  }
  __device__ static void store4(char* dst, float a, float b, float c, float d) {
    *(f32x4_t*)dst = f32x4_t{a, b, c, d};
  }
};

// Staging a chunk into LDS with direct-to-LDS buffer loads.  One load
// instruction of a wavefront fills one 1 KB block (lane l writes 16-byte slot
// 64 * block + l); the K region holds key rows at a pitch of kSlotsK slots, the
// V region at kSlotsV, so a slot is either piece p of row r or row padding.
// Block b of a region goes to wavefront b % 4 (regions are padded to a
// multiple of four blocks, so every wavefront issues the same loads).  Each
// lane keeps, per block it fills, the byte offset of its piece from the
// chunk's first key: one for a dense token range and one for a key tile (rows
// 8 apart on the grid).
// Padding slots get an offset past any buffer bound and load zeros.
template <class E>
struct DmaPlan {
  static constexpr int kPerWaveK = E::kBlocksK / kWaves;
  static constexpr int kPerWaveV = E::kBlocksV / kWaves;
  uint32_t dense_k[kPerWaveK], tile_k[kPerWaveK];
  uint32_t dense_v[kPerWaveV], tile_v[kPerWaveV];
};


template <class E>
__device__ __forceinline__ void slot_offsets(int slot, int slots_per_row, int gw, uint32_t& dense,
                                             uint32_t& tile) {
  const int r = slot / slots_per_row, pc = slot - r * slots_per_row;
  if (r >= kChunk || pc >= E::kPPR) {
    dense = tile = kNoPiece;
  } else {
    dense = (uint32_t)(r * E::kRowBytes + pc * 16);
    tile = (uint32_t)((((r >> 3) * gw) + (r & 7)) * E::kRowBytes + pc * 16);
  }
}

template <class E>
__device__ __forceinline__ DmaPlan<E> make_plan(int wave, int lane, int gw) {
  DmaPlan<E> pl;
  for (int i = 0; i < DmaPlan<E>::kPerWaveK; ++i)
    slot_offsets<E>(64 * (wave + kWaves * i) + lane, E::kSlotsK, gw, pl.dense_k[i], pl.tile_k[i]);
  for (int i = 0; i < DmaPlan<E>::kPerWaveV; ++i)
    slot_offsets<E>(64 * (wave + kWaves * i) + lane, E::kSlotsV, gw, pl.dense_v[i], pl.tile_v[i]);
  return pl;
}


template <class E>
__device__ __forceinline__ void dma_blocks(char* st, int wave, __amdgpu_buffer_rsrc_t rk,
                                           __amdgpu_buffer_rsrc_t rv, const uint32_t* ok,
                                           const uint32_t* ov) {
  char* sk = st + E::kKOff + 1024 * wave;
  char* sv = st + E::kVOff + 1024 * wave;
  for (int i = 0; i < DmaPlan<E>::kPerWaveK; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void_t*)(sk + 1024 * kWaves * i), 16, (int)ok[i], 0, 0, 0);
  for (int i = 0; i < DmaPlan<E>::kPerWaveV; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void_t*)(sv + 1024 * kWaves * i), 16, (int)ov[i], 0, 0, 0);
}

// Start the copy of a chunk into LDS stage st.  The buffer resources start at
// the chunk's first key and end with the head, so pieces past the head read
// zeros; pieces past the grid's right edge read the next row's keys, pieces
// past a dense range's limit the following tokens: all finite and masked.
template <class E>
__device__ __forceinline__ void stage_chunk(char* st, const ChunkMeta& m, bool dense, int wave,
                                            const KeySource& ks, const char* kbase, const char* vbase,
                                            const DmaPlan<E>& pl) {
  const size_t base = (size_t)m.tok0 * E::kRowBytes;
  constexpr int kMaxLeft = 0x7fffffff / E::kRowBytes;  // a resource covers < 2 GB
  const uint32_t bytes = (uint32_t)(m.left < kMaxLeft ? m.left : kMaxLeft) * E::kRowBytes;
  const __amdgpu_buffer_rsrc_t rk = byte_rsrc(kbase + base, bytes), rv = byte_rsrc(vbase + base, bytes);
  if (dense) {
    dma_blocks<E>(st, wave, rk, rv, pl.dense_k, pl.dense_v);
    asm volatile("; stage dense chunk");
  } else {
    dma_blocks<E>(st, wave, rk, rv, pl.tile_k, pl.tile_v);
    asm volatile("; stage key tile");
  }
}

// ------------------------------------------- copies of the bf16 block layout

// Copy plan of the granule layout (Bf16G): lane l of wavefront w fills slot l
// of blocks w + 4i (i < kBlocksPerWave) of both regions, i.e. piece
// 4 (l / 16) + l % 4 of chunk row 4 (w + 4i) + (l / 4) % 4.  Its byte offsets
// from the chunk's first key: for a dense token range (consecutive rows) and
// for a key tile (row 8a + c is cell (a, c), rows a grid row, gw tokens,
// apart).  K and V use the same offsets.
template <class E>
struct BlockPlan {
  uint32_t dense[E::kBlocksPerWave], tile[E::kBlocksPerWave];
};

template <class E>
__device__ __forceinline__ BlockPlan<E> make_block_plan(int wave, int lane, int gw) {
  BlockPlan<E> pl;
  for (int i = 0; i < E::kBlocksPerWave; ++i) {
    const int r = E::kRowsPerBlock * (wave + kWaves * i) + (lane >> 2) % E::kRowsPerBlock;
    const int pc = 4 * (lane >> 4) + (lane & 3);
    pl.dense[i] = (uint32_t)(r * E::kRowBytes + pc * 16);
    pl.tile[i] = (uint32_t)(((r >> 3) * gw + (r & 7)) * E::kRowBytes + pc * 16);
  }
  return pl;
}

// Start the copy of a chunk into stage st (kCopies copies per wavefront, the
// same on every path) in the granule layout.  The resources start at the chunk's first key and end
// with the head: pieces past the head read zeros, pieces past the grid's right
// edge or a dense range's limit read other real keys, all masked.
template <class E>
__device__ __forceinline__ void stage_blocks(char* st, const ChunkMeta& m, bool dense, int wave,
                                             const char* kbase, const char* vbase, const BlockPlan<E>& pl) {
  const size_t off = (size_t)m.tok0 * E::kRowBytes;
  constexpr int kMaxLeft = 0x7fffffff / E::kRowBytes;  // a resource covers < 2 GB
  const uint32_t bytes = (uint32_t)(m.left < kMaxLeft ? m.left : kMaxLeft) * E::kRowBytes;
  const u32x4_t rk = rsrc_words(kbase + off, bytes), rv = rsrc_words(vbase + off, bytes);
  const uint32_t sk = lds_addr(st) + E::kKOff + wave * E::kPitch;
  const uint32_t sv = lds_addr(st) + E::kVOff + wave * E::kPitch;
  if (dense) {
    for (int i = 0; i < E::kBlocksPerWave; ++i) lds_copy(sk + i * kWaves * E::kPitch, rk, pl.dense[i]);
    for (int i = 0; i < E::kBlocksPerWave; ++i) lds_copy(sv + i * kWaves * E::kPitch, rv, pl.dense[i]);
  } else {
    for (int i = 0; i < E::kBlocksPerWave; ++i) lds_copy(sk + i * kWaves * E::kPitch, rk, pl.tile[i]);
    for (int i = 0; i < E::kBlocksPerWave; ++i) lds_copy(sv + i * kWaves * E::kPitch, rv, pl.tile[i]);
  }
}

struct SoftmaxState {
  float M, L;
  float T;  // raw logit above which the reference max moves: (M + tau) / scale_log2
};

// Online-softmax step of one chunk's masked logits (base 2, lazy reference
// max): a rescale only when some lane's sixteen logits pass their row's
// threshold (then the row max over the lane pair moves the reference max),
// probabilities into pr and their sum into L.  Returns true (the same on
// every lane) when the reference max moved; alpha is then the factor O must
// be scaled by before this chunk's P.V.  O itself is not touched here, so the
// caller can skip this step for a chunk the wavefront does not touch.
template <class E>
__device__ __forceinline__ bool chunk_softmax(SoftmaxState& sm, f32x16_t& s, float scale_log2,
                                              float inv_scale_log2, typename E::Probs& pr, float& alpha) {
  float mx = s[0];
  for (int i = 1; i < 16; ++i) mx = __builtin_elementwise_maximum(mx, s[i]);
  bool moved = false;
  if (__ballot(mx > sm.T) != 0ull) {
    // both lanes of a row take this branch and agree on the new reference
    const float Mn = fmaxf(sm.M, max_xor32(mx) * scale_log2);
    alpha = __builtin_amdgcn_exp2f(sm.M - Mn);
    sm.L *= alpha;
    sm.M = Mn;
    sm.T = (Mn + kLazyTau) * inv_scale_log2;
    moved = true;
  }
  for (int i = 0; i < 16; ++i) s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], scale_log2, -sm.M));
  E::probs(s, pr, sm.L);
  return moved;
}

// Logits of one chunk.  A partly admitted chunk starts Q.K from its mask as
// the accumulator, 0 where the pair is admitted and -inf elsewhere, so the
// mask costs no pass over the logits and a whole chunk none at all.  A key
// tile wholly on the grid takes its lane masks from the table; tail chunks and
// tiles reaching past the grid compute theirs.  Each branch keeps its own
// products (the empty statements differ, so they are not merged): joined
// before the products, the branches would meet on the sixteen accumulator
// registers, and the whole chunk would pay for zeroing them.
template <class E>
__device__ __forceinline__ void chunk_logits(const E& eng, const char* st, int lane, f32x16_t& s,
                                             const ChunkInfo& c, const KeySource& ks, int qy, int qx, int r2,
                                             const MaskTable& mt, int mt_base) {
  if (c.coord || c.tail < kChunk) {
    f32x16_t bias{};
    if (c.coord && c.inside && mt.tbl != nullptr)
      apply_lane_masks(bias, mt.tbl + ((c.kty * (2 * mt.kx + 1) + c.ktx + mt_base) << 4));
    else mask_chunk(bias, c, ks, lane >> 5, qy, qx, r2);
    eng.qk(st, lane, s, bias);
    asm volatile("; masked chunk" : "+v"(s));
  } else {
    eng.qk(st, lane, s, f32x16_t{});
    asm volatile("; whole chunk" : "+v"(s));
  }
}

template <class E>
__global__ void __launch_bounds__(kThreads, E::kWavesPerSimd) clear_attn_fwd_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[E::kStages * E::kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int qi = lane & 31;
  const int bid = blockIdx.x;

  const bool text_wg = bid < p.n_text_wg_pad;
  if (text_wg && bid >= p.n_text_wg) return;  // padding workgroup (keeps image ids XCD-aligned)

  int bh, qtok, qy = 0, qx = 0;
  int sy0 = 0, sx0 = 0;  // origin of the wavefront's sub-tile (image workgroups)
  bool qvalid;
  KeySource ks;
  ks.n_text = p.n_text;
  ks.gh = p.gh;
  ks.gw = p.gw;
  ks.desc = (const_u32x4_t*)p.tm_desc;
  ks.e0 = 0;
  ks.n_tok = p.N;
  ks.window = p.window;
  int n_chunks;
  int split = 0, tq = 0;
  if (text_wg) {
    split = bid % p.splits;
    const int rest = bid / p.splits;
    const int tb = rest % p.n_text_blocks;
    bh = rest / p.n_text_blocks;
    tq = tb * kTextQ + wave * 32 + qi;
    qvalid = tq < p.n_text;
    qtok = tq;
    if (p.text_strip) {
      ks.dense_base = 0;
      ks.dense_limit = p.n_text;
      ks.n_dense1 = p.strip_text_keys ? (p.n_text + kChunk - 1) / kChunk : 0;
      ks.dense2_base = p.n_text + p.row_begin * p.gw;
      ks.dense2_limit = p.n_text + p.row_end * p.gw;
      ks.n_dense = ks.n_dense1 + (ks.dense2_limit - ks.dense2_base + kChunk - 1) / kChunk;
    } else {
      const int c0 = split * p.chunks_per_split;
      const int nall = (p.N + kChunk - 1) / kChunk;
      const int c1 = c0 + p.chunks_per_split < nall ? c0 + p.chunks_per_split : nall;
      ks.dense_base = c0 * kChunk;
      ks.dense_limit = p.N;
      ks.n_dense1 = ks.n_dense = c1 - c0;
    }
    n_chunks = ks.n_dense;
  } else {
    // XCD-aware order: hardware places workgroup i on XCD i % 8.  Give each XCD
    // one contiguous range of (head, tile) so the K/V rows its tiles share stay
    // in that XCD's L2.
    const int ib = bid - p.n_text_wg_pad;
    const int per = p.n_img_wg / 8, rem = p.n_img_wg % 8;
    const int xcd = ib % 8, slot = ib / 8;
    const int logical = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    bh = logical / p.band_tiles;
    const int local = logical - bh * p.band_tiles;
    const int ty = p.band_ty0 + local / p.ntx, tx = local - (local / p.ntx) * p.ntx;
    const int tile = ty * p.ntx + tx;
    sy0 = ty * kTileH + wave * kSubH;
    sx0 = tx * kTileW;
    qy = sy0 + (qi >> 3);
    qx = sx0 + (qi & 7);
    qvalid = qy >= p.row_begin && qy < p.row_end && qx < p.gw;
    qtok = p.n_text + qy * p.gw + qx;
    ks.dense_base = 0;
    ks.dense_limit = p.n_text;
    ks.n_dense1 = ks.n_dense = (p.n_text + kChunk - 1) / kChunk;
    const const_u32_t* offs = (const const_u32_t*)p.tm_offsets;
    const uint32_t e0 = offs[tile];
    ks.e0 = (int)e0;
    n_chunks = ks.n_dense + (int)(offs[tile + 1] - e0);
  }

  const size_t head_off = (size_t)bh * p.N * E::kRowBytes;
  const char* kbase = p.k + head_off;
  const char* vbase = p.v + head_off;

  const MaskTable mt{(const_u64_t*)p.mask_tbl, p.mt_ky, p.mt_kx};
  const int mt_base = table_base(mt, sy0, sx0);

  E eng;
  eng.load_q(p.q + head_off + (size_t)(qvalid ? qtok : 0) * E::kRowBytes, qvalid, g);
  eng.zero_o();
  const float inv_scale_log2 = 1.0f / p.scale_log2;
  SoftmaxState sm{kMInit, 0.0f, (kMInit + kLazyTau) * inv_scale_log2};

  // ---- chunk walk.  A chunk the wavefront's sub-tile does not touch
  // contributes nothing to its rows: the wavefront skips its products and
  // softmax and only takes part in the copies and barriers.
  eng.settle_q();
  auto compute = [&](const ChunkInfo& c, const char* st) {
    if (!c.active) return;
    typename E::Probs pr;
    float alpha = 1.0f;
    f32x16_t sc;
    chunk_logits(eng, st, lane, sc, c, ks, qy, qx, p.r2, mt, mt_base);
    if (chunk_softmax<E>(sm, sc, p.scale_log2, inv_scale_log2, pr, alpha)) eng.scale_o(alpha);
    eng.pv(st, lane, pr);
  };
  if constexpr (__is_same(E, Bf16G)) {
    const BlockPlan<E> plan = make_block_plan<E>(wave, lane, p.gw);
    walk_chunks(
        ks, n_chunks, wave, smem, smem + E::kStage,
        [&](char* st, const ChunkMeta& m, bool dense) { stage_blocks<E>(st, m, dense, wave, kbase, vbase, plan); },
        compute);
  } else {
    const DmaPlan<E> plan = make_plan<E>(wave, lane, p.gw);
    walk_chunks(
        ks, n_chunks, wave, smem, smem + E::kStage,
        [&](char* st, const ChunkMeta& m, bool dense) { stage_chunk<E>(st, m, dense, wave, ks, kbase, vbase, plan); },
        compute);
  }

  // ---- epilogue
  const float Lt = sum_xor32(sm.L);
  if (!qvalid) return;
  const int row = text_wg ? tq : qtok;
  if (text_wg && p.partial_out) {
    // unnormalised partial for the log-sum-exp merge
    float* wo = p.ws_o + (((size_t)split * p.BH + bh) * p.n_text + tq) * (E::kNB * 32);
    for (int nb = 0; nb < E::kNB; ++nb)
      for (int a = 0; a < 4; ++a) {
        const int d0 = 32 * nb + 8 * a + 4 * g;
        *(f32x4_t*)(wo + d0) = f32x4_t{eng.o[nb][4 * a], eng.o[nb][4 * a + 1], eng.o[nb][4 * a + 2],
                                       eng.o[nb][4 * a + 3]};
      }
    if (g == 0) {
      float* wm = p.ws_ml + (((size_t)split * p.BH + bh) * p.n_text + tq) * 2;
      wm[0] = sm.M;
      wm[1] = Lt;
    }
    return;
  }
  const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
  char* orow = p.out + head_off + (size_t)row * E::kRowBytes;
  for (int nb = 0; nb < E::kNB; ++nb)
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * nb + 8 * a + 4 * g;
      E::store4(orow + d0 * E::kElem, eng.o[nb][4 * a] * inv, eng.o[nb][4 * a + 1] * inv,
                eng.o[nb][4 * a + 2] * inv, eng.o[nb][4 * a + 3] * inv);
    }
  if (p.lse && g == 0) p.lse[(size_t)bh * p.N + row] = (sm.M + __log2f(Lt)) * 0.69314718055994531f;
}

// Text rows from partials (O_s, M_s, L_s) laid out [part][B*H][n_text][d] and
// [part][B*H][n_text][2] (M in log2 units).
//  * exact (log-sum-exp): M = max_s M_s, w_s = 2^(M_s - M),
//    O = sum_s w_s O_s / sum_s w_s L_s -- softmax over the union of the parts'
//    key sets when they partition the keys;
//  * patch average (the patch-wise approximation of the text rows, Eq. 7 as
//    quoted in the pith.science review of CLEAR, "What carries the argument"):
//    O = (1/P) sum_s O_s / L_s.
struct MergeArgs {
  const float* po;
  const float* pml;
  int nparts, BH, n_text, N, mode;
  void* out;
  float* lse;
};

template <int D, bool BF16>
__global__ void __launch_bounds__(D) clear_text_merge_kernel(MergeArgs m) {
  const int r = blockIdx.x;  // (bh, text row)
  const int bh = r / m.n_text, tq = r - bh * m.n_text;
  const int d = threadIdx.x;
  float o;
  if (m.mode == CLEAR_MERGE_EXACT) {
    float M = kMInit;
    for (int s = 0; s < m.nparts; ++s)
      M = fmaxf(M, m.pml[(((size_t)s * m.BH + bh) * m.n_text + tq) * 2]);
    float L = 0.0f, acc = 0.0f;
    for (int s = 0; s < m.nparts; ++s) {
      const size_t base = ((size_t)s * m.BH + bh) * m.n_text + tq;
      const float w = __builtin_amdgcn_exp2f(m.pml[base * 2] - M);
      L += w * m.pml[base * 2 + 1];
      acc += w * m.po[base * D + d];
    }
    o = L > 0.0f ? acc / L : 0.0f;
    if (m.lse && d == 0) m.lse[(size_t)bh * m.N + tq] = (M + __log2f(L)) * 0.69314718055994531f;
  } else {
    float acc = 0.0f;
    for (int s = 0; s < m.nparts; ++s) {
      const size_t base = ((size_t)s * m.BH + bh) * m.n_text + tq;
      const float L = m.pml[base * 2 + 1];
      acc += L > 0.0f ? m.po[base * D + d] / L : 0.0f;
    }
    o = acc / (float)m.nparts;
  }
  const size_t oi = ((size_t)bh * m.N + tq) * D + d;
  if constexpr (BF16) {
    ((__bf16*)m.out)[oi] = (__bf16)o;
  } else {
    ((float*)m.out)[oi] = o;
  }
}

int launch_merge(const MergeArgs& m, int d, int dtype, hipStream_t s) {
  const int rows = m.BH * m.n_text;
  if (rows == 0) return CLEAR_OK;
  if (dtype == CLEAR_BF16) {
    if (d == 128) hipLaunchKernelGGL((clear_text_merge_kernel<128, true>), dim3(rows), dim3(128), 0, s, m);
    else hipLaunchKernelGGL((clear_text_merge_kernel<64, true>), dim3(rows), dim3(64), 0, s, m);
  } else {
    if (d == 128) hipLaunchKernelGGL((clear_text_merge_kernel<128, false>), dim3(rows), dim3(128), 0, s, m);
    else hipLaunchKernelGGL((clear_text_merge_kernel<64, false>), dim3(rows), dim3(64), 0, s, m);
  }
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(CLEAR_EHIP, "merge kernel launch: %s", hipGetErrorString(e));
  return CLEAR_OK;
}

template <class E>
int launch_main(const Params& p, hipStream_t s, int grid) {
  hipLaunchKernelGGL(clear_attn_fwd_kernel<E>, dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError() == hipSuccess ? CLEAR_OK : CLEAR_EHIP;
}

}  // namespace

int text_merge_launch(const float* part_o, const float* part_ml, int nparts, int mode, void* out,
                      float* lse, int BH, int n_text, int N, int d, int dtype, void* stream) {
  MergeArgs m{part_o, part_ml, nparts, BH, n_text, N, mode, out, lse};
  return launch_merge(m, d, dtype, (hipStream_t)stream);
}

int attn_launch(const AttnLaunch& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  Params p;
  p.q = (const char*)a.q;
  p.k = (const char*)a.k;
  p.v = (const char*)a.v;
  p.out = (char*)a.out;
  p.lse = a.lse;
  p.ws_o = a.ws_o;
  p.ws_ml = a.ws_ml;
  p.tm_offsets = a.tm_offsets;
  p.tm_desc = a.tm_desc;
  p.mask_tbl = a.mask_tbl;
  p.mt_ky = a.mt_ky;
  p.mt_kx = a.mt_kx;
  p.N = a.n_text + a.gh * a.gw;
  p.n_text = a.n_text;
  p.gh = a.gh;
  p.gw = a.gw;
  p.r2 = a.r2;
  p.window = a.window;
  p.ntx = (a.gw + kTileW - 1) / kTileW;
  p.ntiles = ((a.gh + kTileH - 1) / kTileH) * p.ntx;
  p.BH = a.B * a.H;
  p.n_text_blocks = (a.n_text + kTextQ - 1) / kTextQ;
  const int nall = (p.N + kChunk - 1) / kChunk;
  int splits = a.text_splits < 1 ? 1 : a.text_splits;
  if (splits > nall || a.strip) splits = a.strip ? 1 : nall;
  p.chunks_per_split = (nall + splits - 1) / splits;
  p.splits = (nall + p.chunks_per_split - 1) / p.chunks_per_split;  // no empty split
  p.text_strip = a.strip;
  p.strip_text_keys = a.strip_text_keys;
  p.partial_out = a.strip || p.splits > 1;
  p.n_text_wg = p.BH * p.n_text_blocks * p.splits;
  p.n_text_wg_pad = (p.n_text_wg + 7) / 8 * 8;
  p.row_begin = a.row_begin;
  p.row_end = a.row_end;
  p.band_ty0 = a.row_begin / kTileH;
  p.band_tiles = ((a.row_end + kTileH - 1) / kTileH - p.band_ty0) * p.ntx;
  p.n_img_wg = p.BH * p.band_tiles;
  p.scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)a.d));
  if (p.partial_out && p.n_text > 0 && (!a.ws_o || !a.ws_ml))
    return set_error(CLEAR_EINVAL, "text partials need a workspace");
  const long long grid = (long long)p.n_text_wg_pad + p.n_img_wg;
  if (grid > 0x7fffffffLL) return set_error(CLEAR_EINVAL, "too many workgroups");

  int rc;
  if (a.dtype == CLEAR_BF16) {
    rc = a.d == 128 ? launch_main<Bf16G>(p, s, (int)grid) : launch_main<Bf16<64>>(p, s, (int)grid);
  } else {
    rc = a.d == 128 ? launch_main<F32<128>>(p, s, (int)grid) : launch_main<F32<64>>(p, s, (int)grid);
  }
  if (rc) return set_error(CLEAR_EHIP, "attention kernel launch: %s", hipGetErrorString(hipGetLastError()));
  if (!a.strip && p.splits > 1 && p.n_text > 0) {
    MergeArgs m{p.ws_o, p.ws_ml, p.splits, p.BH, p.n_text, p.N, CLEAR_MERGE_EXACT, p.out, p.lse};
    rc = launch_merge(m, a.d, a.dtype, s);
    if (rc) return rc;
  }
  return CLEAR_OK;
}

}  // namespace clear
