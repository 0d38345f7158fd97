// attn_fwd.hip -- fused CLEAR attention forward for gfx950 (MI355X).
//
// What is computed: masked softmax attention with CLEAR's circular-window mask
// (pith.science review of arXiv 2412.16112, "Core claim": a pair is admitted
// when either token is text or the two image tokens are within radius r), logits
// scaled by 1/sqrt(d) (the review's Eq. 1 / Eq. 7), text queries attending to
// every key (the review's referee summary: text-token attention stays global).
//
// Work decomposition (one launch):
//  * image workgroups: 256 threads = 4 wavefronts own a 16 x 8 cell query tile,
//    each wavefront a 4 x 8 sub-tile (32 queries).  Keys stream through LDS in
//    chunks of 32: first the text keys, then the tile's key list (one run of
//    columns per key row, from the tile map).  A wavefront skips chunks its
//    sub-tile does not touch and applies the per-element circular mask only on
//    chunks it does not fully admit;
//  * text workgroups: 128 text queries against a contiguous range of all keys
//    (the range is one of `splits` parts; partial results are merged exactly by
//    log-sum-exp in a second kernel when splits > 1).
//
// Matrix-core formulation (per wavefront, per chunk of 32 keys):
//    S^T[key][query] = K[key][:] . Q[query][:]          A = K (LDS), B = Q^T (VGPRs)
//    O^T[d][query]  += V^T[d][key] . P^T[key][query]    A = V^T (LDS), B = P^T (VGPRs)
// With the 32x32 accumulator layout, lane l holds 16 keys of query l % 32, so
// the softmax row statistics are per lane (plus one exchange with lane l ^ 32)
// and the rescaling of O^T is per lane.  bf16 uses v_mfma_f32_32x32x16_bf16,
// fp32 uses v_mfma_f32_32x32x2_f32.
//
// Online softmax in base 2 with a lazily updated reference max: p = 2^(s*c - M)
// with c = log2(e)/sqrt(d); M is raised only when a row max exceeds M + 8, so
// p <= 256 and O / L is unchanged (softmax is invariant to the reference).
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
typedef __attribute__((ext_vector_type(2))) short s16x2_t;

constexpr int kThreads = 256;
constexpr int kWaves = 4;
constexpr int kTileH = CLEAR_TILE_H;
constexpr int kTileW = CLEAR_TILE_W;
constexpr int kSubH = CLEAR_SUB_H;
constexpr int kChunk = CLEAR_CHUNK;
constexpr int kTextQ = kWaves * 32;  // text queries per workgroup
constexpr float kLazyTau = 8.0f;
constexpr float kMInit = -1.0e30f;
constexpr short kCoordFar = -16384;  // key y of padding positions: never admitted

static_assert(kTileH == kWaves * kSubH && kTileW == CLEAR_SUB_W && kTileW * kSubH == 32,
              "one 32-query sub-tile per wavefront");
static_assert(kChunk == 32, "chunk = one 32-row MFMA block");

struct Params {
  const char* q;
  const char* k;
  const char* v;
  char* out;
  float* lse;
  float* ws_o;
  float* ws_ml;
  const uint32_t* run_off;
  const uint32_t* runs;
  const uint32_t* chunk_off;
  const uint16_t* flags;
  int N, n_text, gh, gw, r2;
  int ntiles, ntx;
  int n_text_blocks, splits, chunks_per_split;
  int n_text_wg, n_text_wg_pad, n_img_wg, BH;
  float scale_log2;
};

// Key position m (0..31) of accumulator register i in lane group g: the row
// index of the 32x32 accumulator layout.
__device__ __forceinline__ int acc_row(int i, int g) { return 8 * (i >> 2) + 4 * g + (i & 3); }

// ---------------------------------------------------------------- engines

// bf16 inputs; K row-major and V transposed ([d][key]) in LDS.
template <int D>
struct Bf16 {
  using T = unsigned short;
  static constexpr int kElem = 2;
  static constexpr int kPPR = D / 8;             // 16-byte pieces per row
  static constexpr int kKRow = D * 2 + 16;       // LDS bytes per K row
  static constexpr int kVtRow = kChunk * 2 + 16; // LDS bytes per V^T row (one d)
  static constexpr int kKOff = 0;
  static constexpr int kVOff = kChunk * kKRow;
  static constexpr int kCOff = kVOff + D * kVtRow;
  static constexpr int kStage = kCOff + kChunk * 4;
  static constexpr int kKIters = kChunk * kPPR / kThreads;
  static constexpr int kVUnits = (kChunk / 2) * kPPR;   // (key pair, piece) units
  static constexpr int kKK = D / 16;
  static constexpr int kNB = D / 32;
  static_assert(kChunk * kPPR % kThreads == 0, "K pieces must split evenly");

  bf16x8_t q[kKK];
  f32x16_t o[kNB];
  u32x4_t kreg[kKIters];
  u32x4_t vreg[2];

  __device__ static int kpos(int r) { return (threadIdx.x + r * kThreads) / kPPR; }
  __device__ static int kcol(int r) { return (threadIdx.x + r * kThreads) % kPPR; }
  __device__ static bool vact() { return threadIdx.x < kVUnits; }
  __device__ static int vpair() { return threadIdx.x % (kChunk / 2); }
  __device__ static int vcol() { return threadIdx.x / (kChunk / 2); }
  // V^T column of key position p: swaps bits 2 and 3 so that the 8 keys one
  // lane group feeds to a P.V step are 16 contiguous bytes.
  __device__ static int vt_col(int p) { return (p & ~15) | ((p & 4) << 1) | ((p & 8) >> 1) | (p & 3); }

  __device__ void load_q(const char* qrow, bool valid, int g) {
    for (int kk = 0; kk < kKK; ++kk) {
      u32x4_t x = valid ? *(const u32x4_t*)(qrow + (16 * kk + 8 * g) * 2) : u32x4_t{0, 0, 0, 0};
      q[kk] = __builtin_bit_cast(bf16x8_t, x);
    }
  }
  __device__ void zero_o() {
    for (int nb = 0; nb < kNB; ++nb) o[nb] = f32x16_t{};
  }
  // Global -> registers.  tok_k[r]: token of K piece r; tok_v[0..1]: tokens of the V pair.
  __device__ void gload(const char* kbase, const char* vbase, const int* tok_k, const int* tok_v) {
    for (int r = 0; r < kKIters; ++r)
      kreg[r] = *(const u32x4_t*)(kbase + (size_t)tok_k[r] * (D * 2) + kcol(r) * 16);
    if (vact()) {
      vreg[0] = *(const u32x4_t*)(vbase + (size_t)tok_v[0] * (D * 2) + vcol() * 16);
      vreg[1] = *(const u32x4_t*)(vbase + (size_t)tok_v[1] * (D * 2) + vcol() * 16);
    }
  }
  // Registers -> LDS stage.
  __device__ void lstore(char* st) {
    for (int r = 0; r < kKIters; ++r)
      *(u32x4_t*)(st + kKOff + kpos(r) * kKRow + kcol(r) * 16) = kreg[r];
    if (vact()) {
      char* vt = st + kVOff + vt_col(2 * vpair()) * 2;
      int d0 = vcol() * 8;
      for (int e = 0; e < 8; ++e) {
        unsigned a = vreg[0][e >> 1], b = vreg[1][e >> 1];
        unsigned w = (e & 1) ? __builtin_amdgcn_perm(b, a, 0x07060302u)
                             : __builtin_amdgcn_perm(b, a, 0x05040100u);
        *(unsigned*)(vt + (d0 + e) * kVtRow) = w;
      }
    }
  }
  __device__ void qk(const char* st, int lane, f32x16_t& s) const {
    const char* kb = st + kKOff + (lane & 31) * kKRow + (lane >> 5) * 16;
    s = f32x16_t{};
    for (int kk = 0; kk < kKK; ++kk) {
      bf16x8_t a = *(const bf16x8_t*)(kb + kk * 32);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, q[kk], s, 0, 0, 0);
    }
  }
  __device__ void pv(const char* st, int lane, const f32x16_t& p) {
    const int g = lane >> 5;
    for (int t = 0; t < 2; ++t) {
      bf16x8_t b;
      for (int j = 0; j < 4; ++j) {
        bf16x2_t h = __builtin_convertvector(f32x2_t{p[8 * t + 2 * j], p[8 * t + 2 * j + 1]}, bf16x2_t);
        b[2 * j] = h[0];
        b[2 * j + 1] = h[1];
      }
      const char* vb = st + kVOff + (lane & 31) * kVtRow + (16 * t + 8 * g) * 2;
      for (int nb = 0; nb < kNB; ++nb) {
        bf16x8_t a = *(const bf16x8_t*)(vb + nb * 32 * kVtRow);
        o[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o[nb], 0, 0, 0);
      }
    }
  }
  // Store 4 consecutive output values (d0 .. d0+3) of one row.
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
  using T = float;
  static constexpr int kElem = 4;
  static constexpr int kPPR = D / 4;
  static constexpr int kRow = D * 4 + 16;
  static constexpr int kKOff = 0;
  static constexpr int kVOff = kChunk * kRow;
  static constexpr int kCOff = 2 * kChunk * kRow;
  static constexpr int kStage = kCOff + kChunk * 4;
  static constexpr int kKIters = kChunk * kPPR / kThreads;
  static constexpr int kHalf = D / 2;   // d values per lane group in Q.K
  static constexpr int kNB = D / 32;
  static_assert(kChunk * kPPR % kThreads == 0, "pieces must split evenly");

  float q[kHalf];
  f32x16_t o[kNB];
  u32x4_t kreg[kKIters];
  u32x4_t vreg[kKIters];

  __device__ static int kpos(int r) { return (threadIdx.x + r * kThreads) / kPPR; }
  __device__ static int kcol(int r) { return (threadIdx.x + r * kThreads) % kPPR; }

  __device__ void load_q(const char* qrow, bool valid, int g) {
    for (int s4 = 0; s4 < kHalf / 4; ++s4) {
      f32x4_t x = valid ? *(const f32x4_t*)(qrow + (kHalf * g + 4 * s4) * 4) : f32x4_t{0, 0, 0, 0};
      for (int e = 0; e < 4; ++e) q[4 * s4 + e] = x[e];
    }
  }
  __device__ void zero_o() {
    for (int nb = 0; nb < kNB; ++nb) o[nb] = f32x16_t{};
  }
  __device__ void gload(const char* kbase, const char* vbase, const int* tok_k, const int* tok_v) {
    for (int r = 0; r < kKIters; ++r) {
      kreg[r] = *(const u32x4_t*)(kbase + (size_t)tok_k[r] * (D * 4) + kcol(r) * 16);
      vreg[r] = *(const u32x4_t*)(vbase + (size_t)tok_v[r] * (D * 4) + kcol(r) * 16);
    }
  }
  __device__ void lstore(char* st) {
    for (int r = 0; r < kKIters; ++r) {
      *(u32x4_t*)(st + kKOff + kpos(r) * kRow + kcol(r) * 16) = kreg[r];
      *(u32x4_t*)(st + kVOff + kpos(r) * kRow + kcol(r) * 16) = vreg[r];
    }
  }
  __device__ void qk(const char* st, int lane, f32x16_t& s) const {
    const char* kb = st + kKOff + (lane & 31) * kRow + (lane >> 5) * kHalf * 4;
    s = f32x16_t{};
    for (int s4 = 0; s4 < kHalf / 4; ++s4) {
      f32x4_t a = *(const f32x4_t*)(kb + s4 * 16);
      for (int e = 0; e < 4; ++e)
        s = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], q[4 * s4 + e], s, 0, 0, 0);
    }
  }
  __device__ void pv(const char* st, int lane, const f32x16_t& p) {
    const int g = lane >> 5;
    for (int u = 0; u < 16; ++u) {
      const float* vr = (const float*)(st + kVOff + acc_row(u, g) * kRow) + (lane & 31);
      for (int nb = 0; nb < kNB; ++nb)
        o[nb] = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[32 * nb], p[u], o[nb], 0, 0, 0);
    }
  }
  __device__ static void store4(char* dst, float a, float b, float c, float d) {
    *(f32x4_t*)dst = f32x4_t{a, b, c, d};
  }
};

// ---------------------------------------------------------------- key sources

// Token and validity of key position p of chunk j for the current workgroup.
struct KeySource {
  // dense range: tokens base .. limit-1 (text chunks, text rows)
  int dense_base;   // token of chunk 0 position 0
  int dense_limit;  // first invalid token
  int n_dense;      // number of dense chunks
  // image runs of the tile
  const uint32_t* runs;
  int r_begin, r_end;   // absolute run indices
  uint32_t total;       // keys in the tile's list
  int n_text;
  int gw;
  // cursor: run containing the first position of the next image chunk to load
  int cur_i;
  uint32_t cur_base;

  __device__ uint32_t rlen(int i) const { return runs[2 * i + 1]; }
  __device__ uint32_t rstart(int i) const { return runs[2 * i]; }

  // Token for position p of chunk j (j < n_dense: dense, else image chunk j - n_dense).
  // Out-of-range positions return a clamped, in-bounds token and valid = false.
  __device__ int token(int j, int p, bool& valid, int& ky, int& kx) const {
    if (j < n_dense) {
      int t = dense_base + j * kChunk + p;
      valid = t < dense_limit;
      ky = 0; kx = 0;
      return valid ? t : dense_limit - 1;
    }
    uint32_t f = (uint32_t)(j - n_dense) * kChunk + p;
    valid = f < total;
    if (!valid) f = total - 1;
    int i = cur_i;
    uint32_t b = cur_base;
    while (i + 1 < r_end && f >= b + rlen(i)) {
      b += rlen(i);
      ++i;
    }
    uint32_t s = rstart(i) + (f - b);
    ky = (int)(rstart(i) / (uint32_t)gw);
    kx = (int)(s - (uint32_t)ky * (uint32_t)gw);
    return n_text + (int)s;
  }
  // Move the cursor to the first position of image chunk (j + 1 - n_dense).
  __device__ void advance_past(int j) {
    if (j < n_dense - 1) return;
    uint32_t f = (uint32_t)(j + 1 - n_dense) * kChunk;
    while (cur_i + 1 < r_end && cur_base + rlen(cur_i) <= f) {
      cur_base += rlen(cur_i);
      ++cur_i;
    }
  }
};

// ---------------------------------------------------------------- kernel

template <class E>
__device__ __forceinline__ void gather_chunk(E& eng, const KeySource& ks, int j, const char* kbase,
                                             const char* vbase, unsigned& creg) {
  int tok_k[E::kKIters > 2 ? E::kKIters : 2];
  int tok_v[E::kKIters > 2 ? E::kKIters : 2];
  bool valid;
  int ky, kx;
  for (int r = 0; r < E::kKIters; ++r) tok_k[r] = ks.token(j, E::kpos(r), valid, ky, kx);
  if constexpr (sizeof(typename E::T) == 2) {
    tok_v[0] = ks.token(j, 2 * E::vpair(), valid, ky, kx);
    tok_v[1] = ks.token(j, 2 * E::vpair() + 1, valid, ky, kx);
  } else {
    for (int r = 0; r < E::kKIters; ++r) tok_v[r] = tok_k[r];
  }
  eng.gload(kbase, vbase, tok_k, tok_v);
  if (threadIdx.x < kChunk) {
    ks.token(j, threadIdx.x, valid, ky, kx);
    short cy = valid ? (short)ky : kCoordFar;
    short cx = valid ? (short)kx : (short)0;
    creg = (unsigned)(unsigned short)cx | ((unsigned)(unsigned short)cy << 16);
  }
}

template <class E>
__global__ void __launch_bounds__(kThreads) clear_attn_fwd_kernel(Params p) {
  __shared__ __attribute__((aligned(16))) char smem[2 * E::kStage];
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;
  const int qi = lane & 31;
  const int bid = blockIdx.x;

  const bool text_wg = bid < p.n_text_wg_pad;
  if (text_wg && bid >= p.n_text_wg) return;  // padding workgroup (keeps image ids XCD-aligned)

  int bh, qtok, qy = 0, qx = 0;
  bool qvalid;
  KeySource ks;
  ks.runs = p.runs;
  ks.n_text = p.n_text;
  ks.gw = p.gw;
  ks.cur_i = 0;
  ks.cur_base = 0;
  ks.r_begin = ks.r_end = 0;
  ks.total = 0;
  int n_chunks;
  int split = 0, tq = 0;
  int tile = 0, co = 0;
  if (text_wg) {
    split = bid % p.splits;
    int rest = bid / p.splits;
    int tb = rest % p.n_text_blocks;
    bh = rest / p.n_text_blocks;
    tq = tb * kTextQ + wave * 32 + qi;
    qvalid = tq < p.n_text;
    qtok = tq;
    int c0 = split * p.chunks_per_split;
    int nall = (p.N + kChunk - 1) / kChunk;
    int c1 = c0 + p.chunks_per_split < nall ? c0 + p.chunks_per_split : nall;
    ks.dense_base = c0 * kChunk;
    ks.dense_limit = p.N;
    ks.n_dense = c1 - c0;
    n_chunks = c1 - c0;
  } else {
    // XCD-aware order: hardware places workgroup i on XCD i % 8.  Give each XCD
    // one contiguous range of (head, tile) so the K/V rows its tiles share stay
    // in that XCD's L2.
    const int ib = bid - p.n_text_wg_pad;
    const int per = p.n_img_wg / 8, rem = p.n_img_wg % 8;
    const int xcd = ib % 8, slot = ib / 8;
    const int logical = xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
    bh = logical / p.ntiles;
    tile = logical - bh * p.ntiles;
    const int ty = tile / p.ntx, tx = tile - (tile / p.ntx) * p.ntx;
    qy = ty * kTileH + wave * kSubH + (qi >> 3);
    qx = tx * kTileW + (qi & 7);
    qvalid = qy < p.gh && qx < p.gw;
    qtok = p.n_text + qy * p.gw + qx;
    ks.dense_base = 0;
    ks.dense_limit = p.n_text;
    ks.n_dense = (p.n_text + kChunk - 1) / kChunk;
    ks.r_begin = (int)p.run_off[tile];
    ks.r_end = (int)p.run_off[tile + 1];
    uint32_t tot = 0;
    for (int i = ks.r_begin; i < ks.r_end; ++i) tot += p.runs[2 * i + 1];
    ks.total = tot;
    ks.cur_i = ks.r_begin;
    co = (int)p.chunk_off[tile];
    n_chunks = ks.n_dense + (int)(p.chunk_off[tile + 1] - p.chunk_off[tile]);
  }

  const size_t head_off = (size_t)bh * p.N * (E::kPPR * 16);
  const char* kbase = p.k + head_off;
  const char* vbase = p.v + head_off;

  E eng;
  eng.load_q(p.q + head_off + (size_t)(qvalid ? qtok : 0) * (E::kPPR * 16), qvalid, g);
  eng.zero_o();
  const bool wave_active = __ballot(qvalid) != 0ull;
  const s16x2_t qc = {(short)qx, (short)qy};

  float M = kMInit, L = 0.0f;
  unsigned creg = 0;

  if (n_chunks > 0) {
    gather_chunk(eng, ks, 0, kbase, vbase, creg);
    ks.advance_past(0);
  }
  for (int j = 0; j < n_chunks; ++j) {
    char* st = smem + (j & 1) * E::kStage;
    eng.lstore(st);
    if (tid < kChunk) *(unsigned*)(st + E::kCOff + tid * 4) = creg;
    if (j + 1 < n_chunks) {
      gather_chunk(eng, ks, j + 1, kbase, vbase, creg);
      ks.advance_past(j + 1);
    }
    __syncthreads();

    if (!wave_active) continue;
    // What this wavefront does with chunk j.
    bool dense = j < ks.n_dense;
    int tail = 32;  // dense chunk: positions >= tail are masked
    bool coord_mask = false;
    if (dense) {
      int rem_keys = ks.dense_limit - (ks.dense_base + j * kChunk);
      tail = rem_keys < 32 ? rem_keys : 32;
    } else {
      unsigned f = p.flags[co + (j - ks.n_dense)];
      if (!((f >> wave) & 1u)) continue;
      coord_mask = !((f >> (8 + wave)) & 1u);
    }

    f32x16_t s;
    eng.qk(st, lane, s);

    if (tail < 32) {
      for (int i = 0; i < 16; ++i)
        if (acc_row(i, g) >= tail) s[i] = -__builtin_inff();
    } else if (coord_mask) {
      const u32x4_t* cp = (const u32x4_t*)(st + E::kCOff);
      for (int a = 0; a < 4; ++a) {
        u32x4_t c4 = cp[2 * a + g];  // positions 8a + 4g .. 8a + 4g + 3
        for (int b = 0; b < 4; ++b) {
          // (built from shifts: a bit_cast of the vector element itself was
          // compiled as element 0 for every b)
          const unsigned cv = c4[b];
          const s16x2_t kc = {(short)(cv & 0xffffu), (short)(cv >> 16)};
          s16x2_t dd = qc - kc;
          int d2 = __builtin_amdgcn_sdot2(dd, dd, 0, false);
          if (d2 > p.r2) s[4 * a + b] = -__builtin_inff();
        }
      }
    }

    // online softmax (base 2, lazy reference max)
    float mx = s[0];
    for (int i = 1; i < 16; ++i) mx = fmaxf(mx, s[i]);
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mxs = mx * p.scale_log2;
    if (__ballot(mxs > M + kLazyTau) != 0ull) {
      float Mn = fmaxf(M, mxs);
      float alpha = __builtin_amdgcn_exp2f(M - Mn);
      L *= alpha;
      for (int nb = 0; nb < E::kNB; ++nb)
        for (int i = 0; i < 16; ++i) eng.o[nb][i] *= alpha;
      M = Mn;
    }
    for (int i = 0; i < 16; ++i) {
      float e = __builtin_amdgcn_exp2f(fmaf(s[i], p.scale_log2, -M));
      s[i] = e;
      L += e;
    }
    eng.pv(st, lane, s);
  }

  // ---- epilogue
  const float Lt = L + __shfl_xor(L, 32);
  if (!qvalid) return;
  const int row = text_wg ? tq : qtok;
  if (text_wg && p.splits > 1) {
    // unnormalised partial for the log-sum-exp merge
    float* wo = p.ws_o + (((size_t)split * p.BH + bh) * p.n_text + tq) * (E::kNB * 32);
    for (int nb = 0; nb < E::kNB; ++nb)
      for (int a = 0; a < 4; ++a) {
        int d0 = 32 * nb + 8 * a + 4 * g;
        *(f32x4_t*)(wo + d0) = f32x4_t{eng.o[nb][4 * a], eng.o[nb][4 * a + 1], eng.o[nb][4 * a + 2],
                                       eng.o[nb][4 * a + 3]};
      }
    if (g == 0) {
      float* wm = p.ws_ml + (((size_t)split * p.BH + bh) * p.n_text + tq) * 2;
      wm[0] = M;
      wm[1] = Lt;
    }
    return;
  }
  const float inv = Lt > 0.0f ? 1.0f / Lt : 0.0f;
  char* orow = p.out + head_off + (size_t)row * (E::kPPR * 16);
  for (int nb = 0; nb < E::kNB; ++nb)
    for (int a = 0; a < 4; ++a) {
      int d0 = 32 * nb + 8 * a + 4 * g;
      E::store4(orow + d0 * E::kElem, eng.o[nb][4 * a] * inv, eng.o[nb][4 * a + 1] * inv,
                eng.o[nb][4 * a + 2] * inv, eng.o[nb][4 * a + 3] * inv);
    }
  if (p.lse && g == 0) p.lse[(size_t)bh * p.N + row] = (M + __log2f(Lt)) * 0.69314718055994531f;
}

// Exact merge of the text-row partials: M = max_s M_s, w_s = 2^(M_s - M),
// O = sum_s w_s O_s / sum_s w_s L_s.
template <int D, bool BF16>
__global__ void __launch_bounds__(D) clear_text_merge_kernel(Params p) {
  const int r = blockIdx.x;  // (bh, text row)
  const int bh = r / p.n_text, tq = r - bh * p.n_text;
  const int d = threadIdx.x;
  float M = kMInit;
  for (int s = 0; s < p.splits; ++s)
    M = fmaxf(M, p.ws_ml[(((size_t)s * p.BH + bh) * p.n_text + tq) * 2]);
  float L = 0.0f, acc = 0.0f;
  for (int s = 0; s < p.splits; ++s) {
    size_t base = ((size_t)s * p.BH + bh) * p.n_text + tq;
    float w = __builtin_amdgcn_exp2f(p.ws_ml[base * 2] - M);
    L += w * p.ws_ml[base * 2 + 1];
    acc += w * p.ws_o[base * D + d];
  }
  float o = L > 0.0f ? acc / L : 0.0f;
  size_t oi = ((size_t)bh * p.N + tq) * D + d;
  if constexpr (BF16) {
    __bf16 h = (__bf16)o;
    ((__bf16*)p.out)[oi] = h;
  } else {
    ((float*)p.out)[oi] = o;
  }
  if (p.lse && d == 0) p.lse[(size_t)bh * p.N + tq] = (M + __log2f(L)) * 0.69314718055994531f;
}

template <class E>
int launch_main(const Params& p, hipStream_t s, int grid) {
  hipLaunchKernelGGL(clear_attn_fwd_kernel<E>, dim3(grid), dim3(kThreads), 0, s, p);
  return hipGetLastError() == hipSuccess ? CLEAR_OK : CLEAR_EHIP;
}

}  // namespace

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
  p.run_off = a.run_off;
  p.runs = a.runs;
  p.chunk_off = a.chunk_off;
  p.flags = a.flags;
  p.N = a.n_text + a.gh * a.gw;
  p.n_text = a.n_text;
  p.gh = a.gh;
  p.gw = a.gw;
  p.r2 = a.r2;
  p.ntx = (a.gw + kTileW - 1) / kTileW;
  p.ntiles = ((a.gh + kTileH - 1) / kTileH) * p.ntx;
  p.BH = a.B * a.H;
  p.n_text_blocks = (a.n_text + kTextQ - 1) / kTextQ;
  const int nall = (p.N + kChunk - 1) / kChunk;
  int splits = a.text_splits < 1 ? 1 : a.text_splits;
  if (splits > nall) splits = nall;
  p.chunks_per_split = (nall + splits - 1) / splits;
  p.splits = (nall + p.chunks_per_split - 1) / p.chunks_per_split;  // no empty split
  p.n_text_wg = p.BH * p.n_text_blocks * p.splits;
  p.n_text_wg_pad = (p.n_text_wg + 7) / 8 * 8;
  p.n_img_wg = p.BH * p.ntiles;
  p.scale_log2 = (float)(1.4426950408889634 / __builtin_sqrt((double)a.d));
  if (p.splits > 1 && (!a.ws_o || !a.ws_ml))
    return set_error(CLEAR_EINVAL, "text splits > 1 need a workspace");
  const long long grid = (long long)p.n_text_wg_pad + p.n_img_wg;
  if (grid > 0x7fffffffLL) return set_error(CLEAR_EINVAL, "too many workgroups");

  int rc;
  if (a.dtype == CLEAR_BF16) {
    rc = a.d == 128 ? launch_main<Bf16<128>>(p, s, (int)grid) : launch_main<Bf16<64>>(p, s, (int)grid);
  } else {
    rc = a.d == 128 ? launch_main<F32<128>>(p, s, (int)grid) : launch_main<F32<64>>(p, s, (int)grid);
  }
  if (rc) return set_error(CLEAR_EHIP, "attention kernel launch: %s", hipGetErrorString(hipGetLastError()));
  if (p.splits > 1 && p.n_text > 0) {
    const int rows = p.BH * p.n_text;
    if (a.dtype == CLEAR_BF16) {
      if (a.d == 128) hipLaunchKernelGGL((clear_text_merge_kernel<128, true>), dim3(rows), dim3(128), 0, s, p);
      else hipLaunchKernelGGL((clear_text_merge_kernel<64, true>), dim3(rows), dim3(64), 0, s, p);
    } else {
      if (a.d == 128) hipLaunchKernelGGL((clear_text_merge_kernel<128, false>), dim3(rows), dim3(128), 0, s, p);
      else hipLaunchKernelGGL((clear_text_merge_kernel<64, false>), dim3(rows), dim3(64), 0, s, p);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return set_error(CLEAR_EHIP, "merge kernel launch: %s", hipGetErrorString(e));
  }
  return CLEAR_OK;
}

}  // namespace clear
