// attn_bwd.hip -- gradients of CLEAR attention for gfx950 (MI355X).
//
// What is computed: dQ, dK, dV of O = softmax over admitted keys of
// Q K^T / sqrt(d), times V (the forward of attn_fwd.hip: CLEAR's mask from the
// pith.science review of arXiv 2412.16112, "Core claim"), for an upstream
// gradient dO.  The backward is the step that follows the forward in the
// paper's attention-only distillation fine-tuning ("What carries the
// argument": only the attention layers are trained).  By the chain rule, with
// c = log2(e)/sqrt(d) and lse2 = lse * log2(e) from the forward:
//    P_ij  = 2^(c s_ij - lse2_i) on admitted pairs, 0 elsewhere
//    dV_j  = sum_i P_ij dO_i          dP_ij = dO_i . v_j
//    D_i   = dO_i . O_i  (= sum_j P_ij dP_ij)
//    dS_ij = P_ij (dP_ij - D_i)
//    dQ_i  = sum_j dS_ij k_j / sqrt(d),   dK_j = sum_i dS_ij q_i / sqrt(d)
//
// Launches (one stream):
//  1. prep: per row, (lse2, -D) from the forward's LSE, O and dO;
//  2. dK/dV, key-centred.  Image workgroups own a 16 x 8 cell key tile, each
//     wavefront a 4 x 8 key sub-tile (32 keys) with its K rows in registers
//     and its V rows in registers (fp32) or in an LDS region of its own (bf16,
//     for the register budget of two wavefronts per SIMD).  Queries stream
//     through LDS in chunks of 32: the text queries, then the 4 x 8 query
//     tiles the tile map lists for the tile.  The window is
//     symmetric and query and key tiles have the same shapes, so the map built
//     for query tiles (key tiles per tile, touched/full flags per sub-tile)
//     reads unchanged for key tiles.  Text-key workgroups take 128 text keys
//     against one range of all queries (every query admits a text key) and
//     write fp32 partials;
//  3. dQ, query-centred, the forward's walk: image workgroups own a query tile
//     and stream the text keys and listed key tiles; text-query workgroups take
//     one range of all keys and write fp32 partials;
//  4. reduce: text rows of dQ, dK and dV from the partials of their ranges.
//
// Matrix-core formulation per wavefront and chunk (32 x 32 accumulators; the
// "own" tokens of the wavefront are the accumulator columns, one per lane):
//   dK/dV:  S  = Q . K^T,  dP = dO . V^T      A = Q, dO rows (LDS), B = K, V (own rows)
//           dV^T += dO^T . P,  dK^T += Q^T . dS   A = dO^T, Q^T (LDS transpose reads)
//   dQ:     S^T = K . Q^T, dP^T = V . dO^T    A = K, V rows (LDS), B = Q, dO (VGPRs)
//           dQ^T += K^T . dS^T                A = K^T (LDS transpose reads)
// so every row statistic (lse2, -D) of the key-centred kernel is per register
// and of the query-centred kernel per lane.
#include "attn_common.h"

namespace clear {
namespace {

constexpr int kStages = 2;
constexpr int kTextRows = kWaves * 32;  // text keys (or queries) per text workgroup

struct BwdParams {
  const char* q;
  const char* k;
  const char* v;
  const char* dout;
  const float* stats;  // [B*H][N][2]: (lse2, -D)
  char* dq;
  char* dk;
  char* dv;
  float* ws_dq;  // text partials [splits][B*H][n_text][d]
  float* ws_dk;
  float* ws_dv;
  const uint32_t* tm_offsets;
  const uint32_t* tm_desc;
  const uint64_t* mask_tbl;  // lane masks of partly admitted chunks (null: computed)
  int mt_ky, mt_kx;
  int N, n_text, gh, gw, r2, window;
  int ntiles, ntx;
  int n_text_blocks, splits, chunks_per_split;
  int n_text_wg, n_text_wg_pad, n_img_wg, BH;
  float scale_log2, scale;
};

// ---------------------------------------------------------------- engines
//
// An engine fixes the element type and how 32-row chunks sit in LDS, and
// provides the two matrix-core patterns:
//   row_mma: acc[m][n] = init[m][n] + sum_k A[m][k] B[k][n], A = the chunk's
//            rows m (LDS), B = the lane's own row n (VGPRs), k over d;
//   tr_mma:  acc[nb][d][n] += sum_m A[m][d] W[m][n], A = the chunk's rows read
//            transposed (LDS), W = 32x32 accumulator values of this chunk
//            (probabilities or dS) converted to an operand.

// bf16: a chunk region holds 32 rows of 16-byte pieces, piece p of row r at
// position p ^ swz(r) of the row.  The swizzle keeps both read patterns free
// of LDS bank conflicts: a row read (16 lanes, rows 0..15, one piece each) and
// a transpose read (4 consecutive rows x 4 consecutive pieces) each touch 16
// distinct 16-byte bank groups.
template <int D>
struct BwdBf16 {
  static constexpr int kElem = 2;
  static constexpr int kRowBytes = D * 2;
  static constexpr int kPPR = D / 8;
  static constexpr int kRegion = kChunk * kRowBytes;  // bytes of one 32-row region
  static constexpr int kBlocks = kRegion / 1024;      // 1 KB direct-to-LDS blocks
  static constexpr int kBlockPitch = 1024;            // copy block pitch
  static constexpr int kKK = D / 16;
  static constexpr int kNB = D / 32;
  static constexpr int kWavesPerSimd = 2;
  // the key-centred kernel keeps each wavefront's V rows in LDS (register budget)
  static constexpr bool kOwnInLds = true;
  static_assert(kBlocks % kWaves == 0, "regions split evenly over the wavefronts");

  __device__ static int swz(int r) {
    if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  // piece p of row r -> byte offset in the region
  __device__ static int piece_at(int r, int p) { return r * kRowBytes + ((p ^ swz(r)) << 4); }
  // slot (16-byte position) of a region -> (row, piece); every slot holds a piece
  __device__ static bool slot_piece(int slot, int& r, int& p) {
    r = slot / kPPR;
    p = (slot - r * kPPR) ^ swz(r);
    return true;
  }

  struct Rows {
    bf16x8_t x[kKK];
  };
  struct Operand {
    bf16x8_t b[2];
  };
  // the lane's own row (d = 16 kk + 8 g .. + 7 in x[kk]); zeros when !valid
  __device__ static void load_rows(const char* row, bool valid, int g, Rows& r) {
    for (int kk = 0; kk < kKK; ++kk) {
      const u32x4_t x = *(const u32x4_t*)(row + (16 * kk + 8 * g) * 2);
      r.x[kk] = __builtin_bit_cast(bf16x8_t, valid ? x : u32x4_t{0, 0, 0, 0});
    }
  }
  __device__ static void row_mma(const char* region, int lane, const Rows& b, const f32x16_t& init,
                                  f32x16_t& acc) {
    const int r = lane & 31, g = lane >> 5;
    acc = init;
    for (int kk = 0; kk < kKK; ++kk) {
      const bf16x8_t a = *(const bf16x8_t*)(region + piece_at(r, 2 * kk + g));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b.x[kk], acc, 0, 0, 0);
      if (kk % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
  }
  // as row_mma, with B read from the wavefront's own rows in LDS
  __device__ static void row_mma_own(const char* region, const char* own, int lane, const f32x16_t& init,
                                      f32x16_t& acc) {
    const int r = lane & 31, g = lane >> 5;
    acc = init;
    for (int kk = 0; kk < kKK; ++kk) {
      const bf16x8_t a = *(const bf16x8_t*)(region + piece_at(r, 2 * kk + g));
      const bf16x8_t b = *(const bf16x8_t*)(own + piece_at(r, 2 * kk + g));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
      if (kk % 4 == 3) __builtin_amdgcn_sched_barrier(0);
    }
  }
  __device__ static void to_operand(const f32x16_t& e, Operand& w) {
    for (int t = 0; t < 2; ++t)
      for (int j = 0; j < 4; ++j) {
        const bf16x2_t h = __builtin_convertvector(f32x2_t{e[8 * t + 2 * j], e[8 * t + 2 * j + 1]}, bf16x2_t);
        w.b[t][2 * j] = h[0];
        w.b[t][2 * j + 1] = h[1];
      }
  }
  // Transpose loads: in each 16-lane group, lane i receives element i % 4 of
  // the 8-byte pieces addressed by lanes i/4, i/4 + 4, i/4 + 8, i/4 + 12.  Lane
  // s of a group addresses row 16t + 8h + 4g + s/4 at columns
  // 32nb + 16*((l/16) % 2) + 4*(s % 4), so lane l ends up holding rows
  // 16t + 8h + 4g + e (e = 0..3) at d = 32nb + l % 32: the rows of accumulator
  // registers 8t + 4h + e whose values operand b[t] carries.
  __device__ static void tr_mma(const char* region, int lane, const Operand& w, f32x16_t* acc) {
    const int g = lane >> 5, s = lane & 15, half = (lane >> 4) & 1;
    for (int t = 0; t < 2; ++t) {
      for (int nb = 0; nb < kNB; ++nb) {
        s16x4_t part[2];
        for (int h = 0; h < 2; ++h) {
          const int r = 16 * t + 8 * h + 4 * g + (s >> 2);
          const int e = 32 * nb + 16 * half + 4 * (s & 3);
          const char* a = region + piece_at(r, e >> 3) + (e & 7) * 2;
          part[h] = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds_char_t*)const_cast<char*>(a));
        }
        const s16x8_t x = __builtin_shufflevector(part[0], part[1], 0, 1, 2, 3, 4, 5, 6, 7);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, x), w.b[t], acc[nb], 0, 0, 0);
        if (nb % 2 == 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  __device__ static void store4(char* dst, float a, float b, float c, float d) {
    bf16x2_t h0 = __builtin_convertvector(f32x2_t{a, b}, bf16x2_t);
    bf16x2_t h1 = __builtin_convertvector(f32x2_t{c, d}, bf16x2_t);
    uint2 u;
    u.x = __builtin_bit_cast(unsigned, h0);
    u.y = __builtin_bit_cast(unsigned, h1);
    *(uint2*)dst = u;
  }
};

// bf16, d = 128: the forward's granule layout.  A region is 8 blocks of 4
// rows at a pitch of 1040 bytes (1 KB plus one 16-byte bank group of skew);
// within a block, 32-column granule c of row j sits at bytes 256 c + 64 j, so
// one copy instruction fills one block with coalesced 64-byte quads (lane l:
// row (l / 4) % 4, piece 4 (l / 16) + l % 4) and no slot is padding.  Both
// read patterns are conflict-free, and a piece's offset from the lane's first
// piece is the same on every lane, so one lane address and immediate offsets
// serve each product:
//   row reads:       lane l, row l % 32, piece 2 kk + l / 32 -> granule kk / 2,
//                    piece 2 (kk % 2) + l / 32 of it;
//   transpose reads: rows 16 t + 8 h + 4 g + s / 4 sit 4 t + 2 h + g blocks in,
//                    columns 32 nb + ... one granule (256 bytes) per nb.
// Operand types, row loads and stores are those of BwdBf16<128>.
struct BwdBf16G : BwdBf16<128> {
  static constexpr int kBlockPitch = 1024 + 16;
  static constexpr int kPitch = kBlockPitch;
  static constexpr int kBlocks = kChunk / 4;
  static constexpr int kRegion = kBlocks * kPitch;
  static_assert(kBlocks % kWaves == 0, "regions split evenly over the wavefronts");

  // LDS byte offset, within a region, of element `col` of chunk row `row`
  __device__ static constexpr int lds_off(int row, int col) {
    return (row / 4) * kPitch + 256 * (col / 32) + 64 * (row % 4) + 16 * ((col / 8) % 4) + 2 * (col % 8);
  }
  __device__ static bool slot_piece(int slot, int& r, int& p) {
    const int b = slot >> 6, l = slot & 63;
    r = 4 * b + ((l >> 2) & 3);
    p = 4 * (l >> 4) + (l & 3);
    return true;
  }
  __device__ static void row_mma(const char* region, int lane, const Rows& b, const f32x16_t& init,
                                  f32x16_t& acc) {
    const char* a0 = region + lds_off(lane & 31, 8 * (lane >> 5));
    acc = init;
    for (int kk = 0; kk < kKK; ++kk) {
      const bf16x8_t a = *(const bf16x8_t*)(a0 + 256 * (kk / 2) + 32 * (kk % 2));
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b.x[kk], acc, 0, 0, 0);
    }
  }
  __device__ static void row_mma_own(const char* region, const char* own, int lane, const f32x16_t& init,
                                      f32x16_t& acc) {
    const int o = lds_off(lane & 31, 8 * (lane >> 5));
    acc = init;
    for (int kk = 0; kk < kKK; ++kk) {
      const int e = o + 256 * (kk / 2) + 32 * (kk % 2);
      const bf16x8_t a = *(const bf16x8_t*)(region + e);
      const bf16x8_t b = *(const bf16x8_t*)(own + e);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc, 0, 0, 0);
    }
  }
  __device__ static void tr_mma(const char* region, int lane, const Operand& w, f32x16_t* acc) {
    const int g = lane >> 5, s = lane & 15, half = (lane >> 4) & 1;
    const char* a00 = region + lds_off(4 * g + (s >> 2), 16 * half + 4 * (s & 3));
    for (int t = 0; t < 2; ++t) {
      for (int nb = 0; nb < kNB; ++nb) {
        const char* a0 = a00 + 4 * t * kPitch + 256 * nb;
        const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(lds_char_t*)const_cast<char*>(a0));
        const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_s16x4_t*)(lds_char_t*)const_cast<char*>(a0 + 2 * kPitch));
        const s16x8_t x = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, x), w.b[t], acc[nb], 0, 0, 0);
        if (nb % 2 == 1) __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
};

// fp32: rows at a pitch of kPPR + 1 slots, no swizzle; v_mfma_f32_32x32x2_f32.
template <int D>
struct BwdF32 {
  static constexpr int kElem = 4;
  static constexpr int kRowBytes = D * 4;
  static constexpr int kPPR = D / 4;
  static constexpr int kSlots = kPPR + 1;
  static constexpr int kPitch = kSlots * 16;
  static constexpr int kBlocks = (kChunk * kSlots + 64 * kWaves - 1) / (64 * kWaves) * kWaves;
  static constexpr int kBlockPitch = 1024;
  static constexpr int kRegion = kBlocks * kBlockPitch;
  static constexpr int kHalf = D / 2;
  static constexpr int kNB = D / 32;
  static constexpr int kWavesPerSimd = 1;
  static constexpr bool kOwnInLds = false;

  __device__ static bool slot_piece(int slot, int& r, int& p) {
    r = slot / kSlots;
    p = slot - r * kSlots;
    return r < kChunk && p < kPPR;
  }

  struct Rows {
    float x[kHalf];
  };
  struct Operand {
    f32x16_t p;
  };
  __device__ static void load_rows(const char* row, bool valid, int g, Rows& r) {
    for (int s4 = 0; s4 < kHalf / 4; ++s4) {
      const f32x4_t x = *(const f32x4_t*)(row + (kHalf * g + 4 * s4) * 4);
      for (int e = 0; e < 4; ++e) r.x[4 * s4 + e] = valid ? x[e] : 0.0f;
    }
  }
  __device__ static void row_mma(const char* region, int lane, const Rows& b, const f32x16_t& init,
                                  f32x16_t& acc) {
    const char* rb = region + (lane & 31) * kPitch + (lane >> 5) * kHalf * 4;
    acc = init;
    for (int s4 = 0; s4 < kHalf / 4; ++s4) {
      const f32x4_t a = *(const f32x4_t*)(rb + s4 * 16);
      for (int e = 0; e < 4; ++e) acc = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], b.x[4 * s4 + e], acc, 0, 0, 0);
    }
  }
  __device__ static void row_mma_own(const char*, const char*, int, const f32x16_t&, f32x16_t&) {}
  __device__ static void to_operand(const f32x16_t& e, Operand& w) { w.p = e; }
  __device__ static void tr_mma(const char* region, int lane, const Operand& w, f32x16_t* acc) {
    const int g = lane >> 5;
    for (int u = 0; u < 16; ++u) {
      const float* rr = (const float*)(region + acc_row(u, g) * kPitch) + (lane & 31);
      for (int nb = 0; nb < kNB; ++nb)
        acc[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(rr[32 * nb], w.p[u], acc[nb], 0, 0, 0);
    }
  }
  __device__ static void store4(char* dst, float a, float b, float c, float d) {
    *(f32x4_t*)dst = f32x4_t{a, b, c, d};
  }
};

// ---------------------------------------------------------------- staging
//
// Both gradient kernels stage two 32-row regions per chunk (dK/dV: Q and dO;
// dQ: K and V) with direct-to-LDS buffer loads issued in assembly (lds_copy),
// as the forward does: one load instruction of a wavefront fills one 1 KB
// block, lane l writing the 16-byte slot 64 * block + l (blocks
// E::kBlockPitch apart), and block b of a region is filled by wavefront b % 4.
// Each lane keeps the byte offset of its slot's piece from the chunk's first
// token, for a dense token range and for a 4 x 8 cell tile (rows gw apart).
// The key-centred kernel also stages the chunk's (lse2, -D) pairs: one 4-byte
// load per lane, lane l fetching component l / 32 of row l % 32; every
// wavefront keeps its own copy.

template <class E>
struct BwdPlan {
  static constexpr int kPerWave = E::kBlocks / kWaves;
  uint32_t dense[kPerWave], tile[kPerWave];
  uint32_t st_dense, st_tile;
};

template <class E>
__device__ __forceinline__ BwdPlan<E> make_bwd_plan(int wave, int lane, int gw) {
  BwdPlan<E> pl;
  for (int i = 0; i < BwdPlan<E>::kPerWave; ++i) {
    int r, pc;
    if (E::slot_piece(64 * (wave + kWaves * i) + lane, r, pc)) {
      pl.dense[i] = (uint32_t)(r * E::kRowBytes + pc * 16);
      pl.tile[i] = (uint32_t)((((r >> 3) * gw) + (r & 7)) * E::kRowBytes + pc * 16);
    } else {
      pl.dense[i] = pl.tile[i] = kNoPiece;
    }
  }
  const int r = lane & 31, comp = lane >> 5;
  pl.st_dense = (uint32_t)(r * 8 + comp * 4);
  pl.st_tile = (uint32_t)((((r >> 3) * gw) + (r & 7)) * 8 + comp * 4);
  return pl;
}

template <class E>
struct BwdLayout {
  static constexpr int kA = 0;                  // Q (dK/dV) or K (dQ)
  static constexpr int kB = E::kRegion;         // dO (dK/dV) or V (dQ)
  static constexpr int kStats = 2 * E::kRegion;  // kWaves copies of [2][32] floats
  static constexpr int kStageAB = 2 * E::kRegion;
  static constexpr int kStageABS = 2 * E::kRegion + kWaves * 256;
  // key-centred kernel: the wavefronts' own V rows, one region each, after the stages
  static constexpr int kOwn = kStages * kStageABS;
  static constexpr int kSmemKV = kOwn + (E::kOwnInLds ? kWaves * E::kRegion : 0);
};

// Bytes from token `tok` to the end of a head of n_tok tokens (0 past the
// end), capped to a buffer resource's 31-bit range.
template <class E>
__device__ __forceinline__ uint32_t bytes_left(int n_tok, int tok) {
  if (tok >= n_tok) return 0u;
  const size_t left = (size_t)(n_tok - tok) * E::kRowBytes;
  return left < 0x7fffffffu ? (uint32_t)left : 0x7fffffffu;
}

// Copy a wavefront's own 32 rows (a dense token range or a 4 x 8 cell tile
// starting at `first`, which may lie past the head for a wavefront whose
// tokens are all invalid) into its LDS region, direct to LDS.  Rows past the
// head read zeros; the caller's barrier waits for the copy.
template <class E>
__device__ __forceinline__ void stage_own(char* region, const char* head, int first, int n_tok, bool dense,
                                          int lane, int gw) {
  const int base = first < n_tok ? first : n_tok;
  const u32x4_t rs = rsrc_words(head + (size_t)base * E::kRowBytes, bytes_left<E>(n_tok, first));
  const uint32_t lds = lds_addr(region);
  for (int b = 0; b < E::kBlocks; ++b) {
    int r, pc;
    uint32_t off = kNoPiece;
    if (E::slot_piece(64 * b + lane, r, pc))
      off = (uint32_t)((dense ? r : ((r >> 3) * gw + (r & 7))) * E::kRowBytes + pc * 16);
    lds_copy(lds + E::kBlockPitch * b, rs, off);
  }
}

template <class E, bool STATS>
__device__ __forceinline__ void stage_bwd(char* st, const ChunkMeta& m, bool dense, int wave,
                                          const char* abase, const char* bbase, const float* sbase,
                                          const BwdPlan<E>& pl) {
  const size_t base = (size_t)m.tok0 * E::kRowBytes;
  constexpr int kMaxLeft = 0x7fffffff / E::kRowBytes;  // a resource covers < 2 GB
  const uint32_t bytes = (uint32_t)(m.left < kMaxLeft ? m.left : kMaxLeft) * E::kRowBytes;
  const u32x4_t ra = rsrc_words(abase + base, bytes), rb = rsrc_words(bbase + base, bytes);
  const uint32_t sa = lds_addr(st) + BwdLayout<E>::kA + E::kBlockPitch * wave;
  const uint32_t sb = lds_addr(st) + BwdLayout<E>::kB + E::kBlockPitch * wave;
  const uint32_t* off = dense ? pl.dense : pl.tile;
  for (int i = 0; i < BwdPlan<E>::kPerWave; ++i) lds_copy(sa + E::kBlockPitch * kWaves * i, ra, off[i]);
  for (int i = 0; i < BwdPlan<E>::kPerWave; ++i) lds_copy(sb + E::kBlockPitch * kWaves * i, rb, off[i]);
  if constexpr (STATS) {
    const u32x4_t rs = rsrc_words((const char*)(sbase + (size_t)m.tok0 * 2),
                                  (uint32_t)(m.left < 0x0fffffff ? m.left : 0x0fffffff) * 8);
    lds_copy_dword(lds_addr(st) + BwdLayout<E>::kStats + 256 * wave, rs, dense ? pl.st_dense : pl.st_tile);
  }
  if (dense) asm volatile("; stage dense chunk");
  else asm volatile("; stage tile chunk");
}

// The workgroup's chunk walk, shared by both gradient kernels: text
// workgroups (text keys for dK/dV, text queries for dQ) take one range of all
// N tokens; image workgroups take the text tokens, then the tiles the tile
// map lists for their tile.  Returns the number of chunks.
struct WgSetup {
  int bh, tok, cy, cx, split, trow;
  int sy0, sx0;  // origin of the wavefront's own sub-tile (image workgroups)
  int first;  // the wavefront's first own token (uniform)
  bool valid, text;
};

__device__ __forceinline__ int setup_walk(const BwdParams& p, int bid, int wave, int lane, KeySource& ks,
                                          WgSetup& w) {
  const int li = lane & 31;
  ks.n_text = p.n_text;
  ks.gh = p.gh;
  ks.gw = p.gw;
  ks.desc = (const_u32x4_t*)p.tm_desc;
  ks.e0 = 0;
  ks.n_tok = p.N;
  ks.window = p.window;
  ks.dense2_base = ks.dense2_limit = 0;
  w.text = bid < p.n_text_wg_pad;
  w.cy = w.cx = 0;
  w.sy0 = w.sx0 = 0;
  w.split = 0;
  w.trow = 0;
  if (w.text) {
    w.split = bid % p.splits;
    const int rest = bid / p.splits;
    const int tb = rest % p.n_text_blocks;
    w.bh = rest / p.n_text_blocks;
    w.trow = tb * kTextRows + wave * 32 + li;
    w.valid = w.trow < p.n_text;
    w.tok = w.trow;
    w.first = tb * kTextRows + wave * 32;
    const int c0 = w.split * p.chunks_per_split;
    const int nall = (p.N + kChunk - 1) / kChunk;
    const int c1 = c0 + p.chunks_per_split < nall ? c0 + p.chunks_per_split : nall;
    ks.dense_base = c0 * kChunk;
    ks.dense_limit = p.N;
    ks.n_dense1 = ks.n_dense = c1 - c0;
    return ks.n_dense;
  }
  // XCD-aware order (workgroup i runs on XCD i % 8): each XCD takes one
  // contiguous range of (head, tile).
  const int ib = bid - p.n_text_wg_pad;
  const int per = p.n_img_wg / 8, rem = p.n_img_wg % 8;
  const int xcd = ib % 8, slot = ib / 8;
  const int logical = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
  w.bh = logical / p.ntiles;
  const int tile = logical - w.bh * p.ntiles;
  const int ty = tile / p.ntx, tx = tile - ty * p.ntx;
  w.sy0 = ty * kTileH + wave * kSubH;
  w.sx0 = tx * kTileW;
  w.cy = w.sy0 + (li >> 3);
  w.cx = w.sx0 + (li & 7);
  w.valid = w.cy < p.gh && w.cx < p.gw;
  w.tok = p.n_text + w.cy * p.gw + w.cx;
  w.first = p.n_text + (ty * kTileH + wave * kSubH) * p.gw + tx * kTileW;
  ks.dense_base = 0;
  ks.dense_limit = p.n_text;
  ks.n_dense1 = ks.n_dense = (p.n_text + kChunk - 1) / kChunk;
  const const_u32_t* offs = (const const_u32_t*)p.tm_offsets;
  const uint32_t e0 = offs[tile];
  ks.e0 = (int)e0;
  return ks.n_dense + (int)(offs[tile + 1] - e0);
}

// Accumulator values (lane l: d = 32 nb + acc_row(i, g) of its own token) to
// a row of the output (scaled), or to an fp32 partial.
template <class E>
__device__ __forceinline__ void store_row(char* row, const f32x16_t* acc, int g, float scale) {
  for (int nb = 0; nb < E::kNB; ++nb)
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * nb + 8 * a + 4 * g;
      E::store4(row + d0 * E::kElem, acc[nb][4 * a] * scale, acc[nb][4 * a + 1] * scale,
                acc[nb][4 * a + 2] * scale, acc[nb][4 * a + 3] * scale);
    }
}
template <class E>
__device__ __forceinline__ void store_partial(float* row, const f32x16_t* acc, int g, float scale) {
  for (int nb = 0; nb < E::kNB; ++nb)
    for (int a = 0; a < 4; ++a) {
      const int d0 = 32 * nb + 8 * a + 4 * g;
      *(f32x4_t*)(row + d0) = f32x4_t{acc[nb][4 * a] * scale, acc[nb][4 * a + 1] * scale,
                                      acc[nb][4 * a + 2] * scale, acc[nb][4 * a + 3] * scale};
    }
}

// ---------------------------------------------------------------- dK, dV

template <class E>
__global__ void __launch_bounds__(kThreads, E::kWavesPerSimd) clear_attn_bwd_dkdv_kernel(BwdParams p) {
  using L = BwdLayout<E>;
  __shared__ __attribute__((aligned(16))) char smem[L::kSmemKV];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int bid = blockIdx.x;
  if (bid < p.n_text_wg_pad && bid >= p.n_text_wg) return;  // padding (keeps image ids XCD-aligned)

  KeySource ks;
  WgSetup w;
  const int n = setup_walk(p, bid, wave, lane, ks, w);
  const size_t head_off = (size_t)w.bh * p.N * E::kRowBytes;
  const char* qbase = p.q + head_off;
  const char* obase = p.dout + head_off;
  const float* sbase = p.stats + (size_t)w.bh * p.N * 2;

  // the wavefront's own keys (zeros for lanes past the grid or the text);
  // V either in registers or in the wavefront's LDS region
  typename E::Rows kr, vr;
  const size_t own = (size_t)(w.valid ? w.tok : 0) * E::kRowBytes;
  E::load_rows(p.k + head_off + own, w.valid, g, kr);
  char* own_v = smem + L::kOwn + E::kRegion * wave;
  if constexpr (E::kOwnInLds) {
    stage_own<E>(own_v, p.v + head_off, w.first, p.N, w.text, lane, p.gw);
  } else {
    E::load_rows(p.v + head_off + own, w.valid, g, vr);
  }
  f32x16_t dk[E::kNB], dv[E::kNB];
  for (int nb = 0; nb < E::kNB; ++nb) dk[nb] = dv[nb] = f32x16_t{};

  const BwdPlan<E> plan = make_bwd_plan<E>(wave, lane, p.gw);
  const MaskTable mt{(const_u64_t*)p.mask_tbl, p.mt_ky, p.mt_kx};
  const int mt_base = table_base(mt, w.sy0, w.sx0);
  // two key tiles per trip (the stages and descriptors in flight keep fixed roles)
  walk_chunks(
      ks, n, wave, smem, smem + L::kStageABS,
      [&](char* st, const ChunkMeta& m, bool dense) {
        stage_bwd<E, true>(st, m, dense, wave, qbase, obase, sbase, plan);
      },
      [&](const ChunkInfo& c, const char* st) {
        if (!c.active) return;
        // dP - D: the product starts from -D of each query row (the staged
        // statistics hold -D), so dS = P (dP - D) is one multiply
        const float* sv = (const float*)(st + L::kStats + 256 * wave);
        f32x16_t s, dp, nd;
        for (int a = 0; a < 4; ++a) {
          const f32x4_t x = *(const f32x4_t*)(sv + 32 + 8 * a + 4 * g);
          for (int e = 0; e < 4; ++e) nd[4 * a + e] = x[e];
        }
        E::row_mma(st + L::kA, lane, kr, f32x16_t{}, s);
        if constexpr (E::kOwnInLds) E::row_mma_own(st + L::kB, own_v, lane, nd, dp);
        else E::row_mma(st + L::kB, lane, vr, nd, dp);
        if (c.coord && c.inside && mt.tbl != nullptr)
          apply_lane_masks(s, mt.tbl + ((c.kty * (2 * mt.kx + 1) + c.ktx + mt_base) << 4));
        else mask_chunk(s, c, ks, g, w.cy, w.cx, p.r2);
        for (int a = 0; a < 4; ++a) {
          const f32x4_t l2 = *(const f32x4_t*)(sv + 8 * a + 4 * g);
          for (int e = 0; e < 4; ++e) {
            const int i = 4 * a + e;
            s[i] = __builtin_amdgcn_exp2f(fmaf(s[i], p.scale_log2, -l2[e]));
            dp[i] = s[i] * dp[i];
          }
        }
        typename E::Operand op;
        E::to_operand(s, op);
        E::tr_mma(st + L::kB, lane, op, dv);
        E::to_operand(dp, op);
        E::tr_mma(st + L::kA, lane, op, dk);
      });

  if (!w.valid) return;
  if (w.text) {
    const size_t prow = (((size_t)w.split * p.BH + w.bh) * p.n_text + w.trow) * (E::kNB * 32);
    store_partial<E>(p.ws_dk + prow, dk, g, p.scale);
    store_partial<E>(p.ws_dv + prow, dv, g, 1.0f);
    return;
  }
  const size_t orow = head_off + (size_t)w.tok * E::kRowBytes;
  store_row<E>(p.dk + orow, dk, g, p.scale);
  store_row<E>(p.dv + orow, dv, g, 1.0f);
}

// ---------------------------------------------------------------- dQ

template <class E>
__global__ void __launch_bounds__(kThreads, E::kWavesPerSimd) clear_attn_bwd_dq_kernel(BwdParams p) {
  using L = BwdLayout<E>;
  __shared__ __attribute__((aligned(16))) char smem[kStages * L::kStageAB];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int bid = blockIdx.x;
  if (bid < p.n_text_wg_pad && bid >= p.n_text_wg) return;

  KeySource ks;
  WgSetup w;
  const int n = setup_walk(p, bid, wave, lane, ks, w);
  const size_t head_off = (size_t)w.bh * p.N * E::kRowBytes;
  const char* kbase = p.k + head_off;
  const char* vbase = p.v + head_off;

  typename E::Rows qr, dor;
  const int own_tok = w.valid ? w.tok : 0;
  const size_t own = (size_t)own_tok * E::kRowBytes;
  E::load_rows(p.q + head_off + own, w.valid, g, qr);
  E::load_rows(p.dout + head_off + own, w.valid, g, dor);
  const float2 stq = *(const float2*)(p.stats + ((size_t)w.bh * p.N + own_tok) * 2);  // (lse2, -D)
  f32x16_t nd;
  for (int i = 0; i < 16; ++i) nd[i] = stq.y;
  f32x16_t dq[E::kNB];
  for (int nb = 0; nb < E::kNB; ++nb) dq[nb] = f32x16_t{};

  const BwdPlan<E> plan = make_bwd_plan<E>(wave, lane, p.gw);
  const MaskTable mt{(const_u64_t*)p.mask_tbl, p.mt_ky, p.mt_kx};
  const int mt_base = table_base(mt, w.sy0, w.sx0);
  walk_chunks(
      ks, n, wave, smem, smem + L::kStageAB,
      [&](char* st, const ChunkMeta& m, bool dense) {
        stage_bwd<E, false>(st, m, dense, wave, kbase, vbase, nullptr, plan);
      },
      [&](const ChunkInfo& c, const char* st) {
        if (!c.active) return;
        f32x16_t s, dp;
        E::row_mma(st + L::kA, lane, qr, f32x16_t{}, s);
        E::row_mma(st + L::kB, lane, dor, nd, dp);  // dP - D of the lane's query
        if (c.coord && c.inside && mt.tbl != nullptr)
          apply_lane_masks(s, mt.tbl + ((c.kty * (2 * mt.kx + 1) + c.ktx + mt_base) << 4));
        else mask_chunk(s, c, ks, g, w.cy, w.cx, p.r2);
        for (int i = 0; i < 16; ++i) {
          const float pr = __builtin_amdgcn_exp2f(fmaf(s[i], p.scale_log2, -stq.x));
          dp[i] = pr * dp[i];
        }
        typename E::Operand op;
        E::to_operand(dp, op);
        E::tr_mma(st + L::kA, lane, op, dq);
      });

  if (!w.valid) return;
  if (w.text) {
    const size_t prow = (((size_t)w.split * p.BH + w.bh) * p.n_text + w.trow) * (E::kNB * 32);
    store_partial<E>(p.ws_dq + prow, dq, g, p.scale);
    return;
  }
  store_row<E>(p.dq + head_off + (size_t)w.tok * E::kRowBytes, dq, g, p.scale);
}

// ---------------------------------------------------------------- prep, reduce

struct PrepArgs {
  const char* out;
  const char* dout;
  const float* lse;
  float* stats;
  long long rows;  // B*H*N
};

// 16 threads per row, 16 rows per 256-thread workgroup: lse2_i = lse_i *
// log2(e) and -D_i = -(dO_i . O_i) in fp32 (the gradient kernels start the dP
// products from -D).
template <int D, bool BF16>
__global__ void __launch_bounds__(256) clear_attn_bwd_prep_kernel(PrepArgs a) {
  constexpr int kPer = D / 16;  // elements per thread
  const long long row = (long long)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int sub = threadIdx.x & 15;
  float acc = 0.0f;
  if (row < a.rows) {
    const size_t base = (size_t)row * D + sub * kPer;
    if constexpr (BF16) {
      const __bf16* o = (const __bf16*)a.out + base;
      const __bf16* g = (const __bf16*)a.dout + base;
      for (int e = 0; e < kPer; ++e) acc = fmaf((float)o[e], (float)g[e], acc);
    } else {
      const float* o = (const float*)a.out + base;
      const float* g = (const float*)a.dout + base;
      for (int e = 0; e < kPer; ++e) acc = fmaf(o[e], g[e], acc);
    }
  }
  for (int m = 8; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 16);
  if (row < a.rows && sub == 0) {
    a.stats[2 * row] = a.lse[row] * 1.4426950408889634f;
    a.stats[2 * row + 1] = -acc;
  }
}

struct ReduceArgs {
  const float* ws[3];  // dq, dk, dv partials [splits][B*H][n_text][d]
  char* out[3];
  int splits, BH, n_text, N;
};

// Text rows of dQ, dK, dV: the sum of their range partials (already scaled).
template <int D, bool BF16>
__global__ void __launch_bounds__(D) clear_attn_bwd_reduce_kernel(ReduceArgs a) {
  const int r = blockIdx.x;  // (bh, text row)
  const int t = blockIdx.y;  // 0 dq, 1 dk, 2 dv
  const int bh = r / a.n_text, row = r - bh * a.n_text;
  const int d = threadIdx.x;
  float acc = 0.0f;
  for (int s = 0; s < a.splits; ++s) acc += a.ws[t][(((size_t)s * a.BH + bh) * a.n_text + row) * D + d];
  const size_t oi = ((size_t)bh * a.N + row) * D + d;
  if constexpr (BF16) ((__bf16*)a.out[t])[oi] = (__bf16)acc;
  else ((float*)a.out[t])[oi] = acc;
}

template <class E>
int launch_grads(const BwdParams& p, hipStream_t s, int grid) {
  hipLaunchKernelGGL(clear_attn_bwd_dkdv_kernel<E>, dim3(grid), dim3(kThreads), 0, s, p);
  if (hipGetLastError() != hipSuccess) return CLEAR_EHIP;
  hipLaunchKernelGGL(clear_attn_bwd_dq_kernel<E>, dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError() == hipSuccess ? CLEAR_OK : CLEAR_EHIP;
}

template <int D, bool BF16>
void launch_prep_reduce(const PrepArgs& pa, const ReduceArgs* ra, hipStream_t s, bool reduce) {
  if (!reduce) {
    const long long blocks = (pa.rows + 15) / 16;
    hipLaunchKernelGGL((clear_attn_bwd_prep_kernel<D, BF16>), dim3((unsigned)blocks), dim3(256), 0, s, pa);
  } else {
    hipLaunchKernelGGL((clear_attn_bwd_reduce_kernel<D, BF16>), dim3(ra->BH * ra->n_text, 3), dim3(D), 0, s, *ra);
  }
}

void prep_or_reduce(int d, int dtype, const PrepArgs& pa, const ReduceArgs* ra, hipStream_t s, bool reduce) {
  if (dtype == CLEAR_BF16) {
    if (d == 128) launch_prep_reduce<128, true>(pa, ra, s, reduce);
    else launch_prep_reduce<64, true>(pa, ra, s, reduce);
  } else {
    if (d == 128) launch_prep_reduce<128, false>(pa, ra, s, reduce);
    else launch_prep_reduce<64, false>(pa, ra, s, reduce);
  }
}

}  // namespace

int attn_bwd_launch(const BwdLaunch& a, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  BwdParams p;
  p.q = (const char*)a.q;
  p.k = (const char*)a.k;
  p.v = (const char*)a.v;
  p.dout = (const char*)a.dout;
  p.stats = a.ws_stats;
  p.dq = (char*)a.dq;
  p.dk = (char*)a.dk;
  p.dv = (char*)a.dv;
  p.ws_dq = a.ws_dq;
  p.ws_dk = a.ws_dk;
  p.ws_dv = a.ws_dv;
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
  p.n_text_blocks = (a.n_text + kTextRows - 1) / kTextRows;
  const int nall = (p.N + kChunk - 1) / kChunk;
  int splits = a.text_splits < 1 ? 1 : a.text_splits;
  if (splits > nall) splits = nall;
  p.chunks_per_split = (nall + splits - 1) / splits;
  p.splits = (nall + p.chunks_per_split - 1) / p.chunks_per_split;  // no empty range
  p.n_text_wg = p.BH * p.n_text_blocks * p.splits;
  p.n_text_wg_pad = (p.n_text_wg + 7) / 8 * 8;
  p.n_img_wg = p.BH * p.ntiles;
  p.scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)a.d));
  p.scale = (float)(1.0 / __builtin_sqrt((double)a.d));
  const long long grid = (long long)p.n_text_wg_pad + p.n_img_wg;
  if (grid > 0x7fffffffLL) return set_error(CLEAR_EINVAL, "too many workgroups");
  if (p.n_text > 0 && (!a.ws_dq || !a.ws_dk || !a.ws_dv))
    return set_error(CLEAR_EINVAL, "text partials need a workspace");

  PrepArgs pa{(const char*)a.out, (const char*)a.dout, a.lse, a.ws_stats, (long long)p.BH * p.N};
  prep_or_reduce(a.d, a.dtype, pa, nullptr, s, false);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return set_error(CLEAR_EHIP, "backward prep launch: %s", hipGetErrorString(e));

  int rc;
  if (a.dtype == CLEAR_BF16) {
    rc = a.d == 128 ? launch_grads<BwdBf16G>(p, s, (int)grid) : launch_grads<BwdBf16<64>>(p, s, (int)grid);
  } else {
    rc = a.d == 128 ? launch_grads<BwdF32<128>>(p, s, (int)grid) : launch_grads<BwdF32<64>>(p, s, (int)grid);
  }
  if (rc) return set_error(CLEAR_EHIP, "backward kernel launch: %s", hipGetErrorString(hipGetLastError()));

  if (p.n_text > 0) {
    ReduceArgs ra{{p.ws_dq, p.ws_dk, p.ws_dv}, {p.dq, p.dk, p.dv}, p.splits, p.BH, p.n_text, p.N};
    prep_or_reduce(a.d, a.dtype, pa, &ra, s, true);
    e = hipGetLastError();
    if (e != hipSuccess) return set_error(CLEAR_EHIP, "backward reduce launch: %s", hipGetErrorString(e));
  }
  return CLEAR_OK;
}

}  // namespace clear
