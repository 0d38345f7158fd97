/*
 * clear_attn.h -- C ABI of libclear_attn.so: the forward pass of CLEAR
 * circular-window attention on AMD Instinct MI355X (gfx950), and its gradients.
 *
 * The operation (CLEAR, arXiv 2412.16112; mask as written in the pith.science
 * review of the paper, section "Core claim"; softmax attention with 1/sqrt(c)
 * scaling, the review's Eq. 1 / Eq. 7; text-token attention kept global, the
 * review's referee summary):
 *
 *   tokens   : n_text text tokens first, then a grid_h x grid_w image grid
 *              flattened row-major (image cell (y, x) is token n_text + y*grid_w + x)
 *   mask     : M[i][j] = i < n_text  or  j < n_text  or  dy^2 + dx^2 <= r2
 *              (dy, dx = grid offsets between image tokens i and j; keys outside
 *              the grid do not exist)
 *   output   : O_i = sum_j M_ij exp(s_ij) v_j / sum_j M_ij exp(s_ij),
 *              s_ij = q_i . k_j / sqrt(d)
 *
 * r2 = radius^2 is the "<=" reading of the window; the review prints a strict
 * "< r^2", which on the integer lattice is r2 = radius^2 - 1 (pass it through
 * clear_attn_fwd_ex).  A negative r2 admits no image key.
 *
 * Square-window variant (CLEAR_WINDOW_SQUARE; not CLEAR's mask: the square the
 * circle is inscribed in, against which the review's "What carries the
 * argument" prices the circle at about pi/4): the image condition becomes
 * max(dy^2, dx^2) <= r2, i.e. max(|dy|, |dx|) <= isqrt(r2).
 *
 * Conventions shared by every entry point
 *   - Return value: CLEAR_OK (0) or a negative error code below.  On error
 *     nothing has been launched or written, and clear_last_error() describes
 *     the problem.  Argument checks run before any HIP call.
 *   - Device pointers are plain addresses in the current HIP device's memory.
 *     `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued on that stream; the library never synchronises it.
 *     Exceptions: clear_release_cache (synchronises every device it used);
 *     the clean-up after a failed HIP call while a tile map is being built
 *     (synchronises the stream before freeing); and CLEAR_DEBUG=1 in the
 *     environment, which synchronises after each launch and maps failures to
 *     CLEAR_EHIP.  The library's workspace grows in stream order: the old
 *     buffer is released with hipFreeAsync and the new one taken with
 *     hipMallocAsync on the caller's stream, after that stream has waited for
 *     the buffer's previous user, so growth never blocks the host.
 *   - Faults inside kernels surface at the caller's next synchronisation.
 *   - Thread safety: every entry point may be called from several host
 *     threads; the library's caches are guarded by a mutex.  Calls that use
 *     the library's workspace (the text-row partials of clear_attn_fwd* and
 *     the statistics and partials of clear_attn_bwd) share one buffer per
 *     device.  Calls on one stream are ordered by the stream; a call on
 *     another stream than the previous user of the buffer first makes its
 *     stream wait (on the device, by an event) for that user's kernels, so
 *     such calls take turns with the buffer instead of overlapping.
 */
#ifndef CLEAR_ATTN_H
#define CLEAR_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CLEAR_OK 0
#define CLEAR_EINVAL (-22)  /* invalid argument                          */
#define CLEAR_ENOMEM (-12)  /* caller buffer too small / allocation fail */
#define CLEAR_EHIP (-5)     /* a HIP runtime call failed                 */
#define CLEAR_ENOTSUP (-95) /* valid but unsupported combination         */

#define CLEAR_BF16 0
#define CLEAR_FP32 1

#define CLEAR_WINDOW_CIRCLE 0  /* dy^2 + dx^2 <= r2 (CLEAR)      */
#define CLEAR_WINDOW_SQUARE 1  /* max(dy^2, dx^2) <= r2 (variant) */

#define CLEAR_MERGE_EXACT 0          /* log-sum-exp merge of text-row partials      */
#define CLEAR_MERGE_PATCH_AVERAGE 1  /* mean of normalised partials (Eq. 7 reading) */

/* Tiling of the attention kernels: a workgroup owns a 16 x 8 cell query tile;
 * each of its four wavefronts owns a 4 x 8 sub-tile; image keys stream in 4 x 8
 * cell key tiles (32 keys), text keys in chunks of 32.  clear_tile_map_build*
 * accept other tilings (for testing). */
#define CLEAR_TILE_H 16
#define CLEAR_TILE_W 8
#define CLEAR_SUB_H 4
#define CLEAR_SUB_W 8
#define CLEAR_KEY_H 4
#define CLEAR_KEY_W 8
#define CLEAR_CHUNK 32

/* Largest grid side the kernels accept (grid coordinates travel as 16-bit). */
#define CLEAR_MAX_GRID 8192

typedef struct clear_opts {
  int dtype;        /* CLEAR_BF16 or CLEAR_FP32 (element type of q, k, v, out) */
  int r2_max;       /* admit image pairs with dy^2 + dx^2 <= r2_max; >= -1     */
  float* lse_out;   /* optional device [B, H, N] float32: natural-log
                       log-sum-exp of each row's admitted logits; NULL = skip  */
  int text_splits;  /* text rows: number of key-range splits merged exactly by
                       log-sum-exp; 0 = chosen by the library; 1..64          */
  int window;       /* CLEAR_WINDOW_CIRCLE (0) or CLEAR_WINDOW_SQUARE (1)
                       (added in version 1.1; zero-initialise the struct)     */
} clear_opts;

/*
 * clear_attn_fwd -- one CLEAR attention layer, bfloat16, r2 = radius^2.
 *
 *   q, k, v : device, [B, H, N, d] contiguous bfloat16, N = n_text + grid_h*grid_w,
 *             16-byte aligned.  Caller-owned, read only.
 *   out     : device, [B, H, N, d] contiguous bfloat16; caller-owned; must not
 *             overlap q, k or v.  Every element is written.
 *   B, H    : >= 1.  d: 64 or 128.  n_text >= 0; N at most 2^31 - 4097.
 *   grid_h, grid_w : 1 .. CLEAR_MAX_GRID.  radius >= 0.
 *   n_text == 0 with an empty window cannot happen here (radius >= 0 admits
 *   the query itself).
 * Arithmetic: bf16 inputs, fp32 accumulation of q.k and of p.v, softmax in
 * fp32 (exp2 form), probabilities rounded to bf16 for the p.v product, output
 * rounded to bf16.
 * The library builds (on the stream, once per (grid_h, grid_w, r2)) and caches
 * the tile map, and owns the text-row workspace; see clear_release_cache.
 * Returns CLEAR_ENOTSUP, launching nothing, when that tile map would list more
 * than 2^31 - 1 key tiles (the kernels' 32-bit signed entry index): only huge
 * grids at large radii: from r = 197 on an 8192 x 8192 grid.  Every entry
 * point that attends (forward, strips, backward) shares this limit.
 */
int clear_attn_fwd(const void* q, const void* k, const void* v, void* out,
                   int B, int H, int d, int n_text, int grid_h, int grid_w,
                   int radius, void* stream);

/*
 * clear_attn_fwd_ex -- as clear_attn_fwd with options: element type (bf16 or
 * fp32; fp32 runs fp32 matrix-core products and keeps probabilities in fp32),
 * explicit r2_max (-1 .. any; n_text == 0 with r2_max < 0 leaves every row
 * empty and returns CLEAR_EINVAL), optional LSE output, the text-row split
 * count and the window.  opts == NULL means {CLEAR_BF16, 0, NULL, 0,
 * CLEAR_WINDOW_CIRCLE}.
 */
int clear_attn_fwd_ex(const void* q, const void* k, const void* v, void* out,
                      int B, int H, int d, int n_text, int grid_h, int grid_w,
                      const clear_opts* opts, void* stream);

/*
 * clear_attn_fwd_strip -- one horizontal strip of a patch-parallel layer: the
 * share of one device when the image grid is split into row strips (the pages'
 * patch-parallel inference; pith.science review, "What carries the argument").
 *
 *   q, k, v, out, B, H, d, n_text, grid_h, grid_w, opts: as clear_attn_fwd_ex
 *     (opts->text_splits must be 0; opts->lse_out, if set, receives the LSE of
 *     the strip's image rows only).
 *   row_begin, row_end : the strip, image rows [row_begin, row_end), 0 <= row_begin
 *     < row_end <= grid_h.  Exactly those image rows of out are written (text
 *     rows and other image rows are left untouched).  Their keys are the text
 *     tokens and the image rows within isqrt(r2_max) of the strip: the strip plus
 *     halos of O(r x grid_w) keys, as on a device holding only that slab.
 *   with_text_keys : nonzero = the text-row partial also covers the text keys.
 *   text_part_o  : device, [B*H, n_text, d] float32 -- unnormalised partial
 *                  O_s = sum_j 2^(c s_j - M_s) v_j over the strip's keys for the text
 *                  rows (c = log2(e)/sqrt(d), s_j = q.k_j);
 *   text_part_ml : device, [B*H, n_text, 2] float32 -- (M_s, L_s), M_s the reference
 *                  max in log2 units, L_s = sum_j 2^(c s_j - M_s).
 *                  The partial's keys: text keys if with_text_keys, then the image
 *                  tokens of rows [row_begin, row_end).  Both buffers caller-owned,
 *                  4-byte aligned; NULL allowed when n_text == 0.
 * Merging the partials of strips that cover all rows, exactly one of them with
 * text keys, with CLEAR_MERGE_EXACT reproduces the text rows of clear_attn_fwd_ex.
 */
int clear_attn_fwd_strip(const void* q, const void* k, const void* v, void* out,
                         int B, int H, int d, int n_text, int grid_h, int grid_w,
                         const clear_opts* opts, int row_begin, int row_end,
                         int with_text_keys, float* text_part_o, float* text_part_ml,
                         void* stream);

/*
 * clear_text_merge -- text rows of out from nparts text-row partials stacked as
 * [nparts][B*H][n_text][d] and [nparts][B*H][n_text][2] (the layout written by
 * clear_attn_fwd_strip; consecutive strips' buffers).
 *   mode CLEAR_MERGE_EXACT: M = max_s M_s, w_s = 2^(M_s - M),
 *        O = sum_s w_s O_s / sum_s w_s L_s (softmax over the union of the parts'
 *        keys; exact when they partition the keys); lse_out (optional, device
 *        [B, H, N] float32) receives the natural-log LSE of the text rows.
 *   mode CLEAR_MERGE_PATCH_AVERAGE: O = (1/nparts) sum_s O_s / L_s, the
 *        patch-wise text-row approximation (Eq. 7 as quoted in the pith.science
 *        review, "What carries the argument"), with each part the softmax over its
 *        device's keys; lse_out must be NULL.
 *   out: device [B, H, N, d] (N = n_text + grid_h*grid_w) of dtype; only rows
 *        0 .. n_text-1 are written.
 */
int clear_text_merge(const float* part_o, const float* part_ml, int nparts, int mode,
                     void* out, float* lse_out, int B, int H, int d, int n_text,
                     int grid_h, int grid_w, int dtype, void* stream);

/*
 * clear_attn_bwd -- gradients of one CLEAR attention layer (added in 1.3).
 * The backward is the step that follows the forward in the paper's
 * attention-only distillation fine-tuning (pith.science review of arXiv
 * 2412.16112, "What carries the argument").  For the forward
 * O = softmax_M(Q K^T / sqrt(d)) V and an upstream gradient dO = dL/dO:
 *
 *   P_ij  = M_ij exp(s_ij - lse_i),  s_ij = q_i . k_j / sqrt(d)
 *   dV_j  = sum_i P_ij dO_i
 *   dS_ij = P_ij (dO_i . v_j - dO_i . O_i)
 *   dQ_i  = sum_j dS_ij k_j / sqrt(d),   dK_j = sum_i dS_ij q_i / sqrt(d)
 *
 *   q, k, v   : device, [B, H, N, d] contiguous, the forward's inputs.
 *   out       : device, [B, H, N, d], the forward's output O (same call options).
 *   dout      : device, [B, H, N, d], the upstream gradient dO.
 *   lse       : device, [B, H, N] float32, the forward's lse_out (natural log).
 *   dq, dk, dv: device, [B, H, N, d] contiguous outputs, every element written;
 *               must not overlap each other or any input.
 *   All of q .. dv are caller-owned, of opts->dtype, 16-byte aligned (lse:
 *   4-byte aligned).  Shapes, dtype, r2_max, window and their checks as
 *   clear_attn_fwd_ex; opts->lse_out must be NULL; opts->text_splits sets how
 *   many query (key) ranges the text keys' (text queries') gradient rows are
 *   split into (0 = chosen by the library), summed in a final step.
 * Arithmetic (bf16): bf16 inputs, fp32 accumulation, P and dS rounded to bf16
 * for the matrix-core products, D = dO . O in fp32, outputs rounded to bf16.
 * The library owns a workspace of B*H*N*8 bytes of row statistics plus
 * 3 * splits * B*H*n_text*d*4 bytes of text-row partials (see the thread
 * safety note above).
 */
int clear_attn_bwd(const void* q, const void* k, const void* v, const void* out,
                   const void* dout, const float* lse, void* dq, void* dk, void* dv,
                   int B, int H, int d, int n_text, int grid_h, int grid_w,
                   const clear_opts* opts, void* stream);

/*
 * clear_tile_map_size -- number of entries of the tile map (host, closed form).
 * The tile map lists, for each query tile, the key tiles that at least one of
 * its sub-tiles touches under the mask (the review's "Core claim", image pairs
 * only), with per-sub-tile flags.
 * Constraints: grid sides 1..CLEAR_MAX_GRID; r2_max >= -1; tile_h, tile_w,
 * sub_h, sub_w >= 1 with sub_h | tile_h, sub_w | tile_w, tile sides <= 1024 and
 * at most 8 sub-tiles per tile; key_h, key_w in 1..1024.
 */
int clear_tile_map_size(int grid_h, int grid_w, int r2_max, int tile_h, int tile_w,
                        int sub_h, int sub_w, int key_h, int key_w, size_t* n_entries);

/*
 * clear_tile_map_build -- build the tile map on the host.
 *
 * Query tiles are numbered row-major (t = ty * ceil(grid_w/tile_w) + tx); tile
 * t covers grid rows [ty*tile_h, ty*tile_h + tile_h) and columns
 * [tx*tile_w, tx*tile_w + tile_w), clipped to the grid; its sub-tiles are
 * numbered row-major within it.  Key tiles are numbered row-major the same way
 * with key_h x key_w cells (id = kty * ceil(grid_w/key_w) + ktx).  Outputs
 * (host memory, caller-owned):
 *   offsets   [ntiles + 1] : entries of query tile t are offsets[t] .. offsets[t+1]-1
 *   key_tiles [n_entries]  : key-tile ids, ascending within a query tile
 *   flags     [n_entries]  : bit s = sub-tile s admits some pair (query cell of the
 *                            sub-tile on the grid, key cell of the key tile on the
 *                            grid); bit 8+s = in addition the key tile lies wholly on
 *                            the grid and sub-tile s admits every such pair.  A key
 *                            tile is listed iff some bit 0..7 is set.
 * cap is the capacity of key_tiles / flags.  If it is too small, returns
 * CLEAR_ENOMEM with *n_entries set and nothing written (cap 0 queries the size).
 * A map of more than 2^32 - 1 entries does not fit the 32-bit offsets: then
 * CLEAR_ENOTSUP, with *n_entries set and nothing written.
 */
int clear_tile_map_build(int grid_h, int grid_w, int r2_max, int tile_h, int tile_w,
                         int sub_h, int sub_w, int key_h, int key_w, uint32_t* offsets,
                         uint32_t* key_tiles, uint16_t* flags, size_t cap,
                         size_t* n_entries);

/*
 * clear_tile_map_build_device -- the same tile map, built by kernels on `stream`
 * into device buffers (same layout and contents, bit for bit, as the host
 * builder).  The size is computed on the host first; if cap is too small it
 * returns CLEAR_ENOMEM with *n_entries (a host pointer) set and launches nothing
 * (CLEAR_ENOTSUP likewise above 2^32 - 1 entries).
 */
int clear_tile_map_build_device(int grid_h, int grid_w, int r2_max, int tile_h,
                                int tile_w, int sub_h, int sub_w, int key_h, int key_w,
                                uint32_t* offsets, uint32_t* key_tiles, uint16_t* flags,
                                size_t cap, size_t* n_entries, void* stream);

/*
 * clear_tile_map_size_ex / clear_tile_map_build_ex / clear_tile_map_build_device_ex
 * -- the same three operations for either window (first argument
 * CLEAR_WINDOW_CIRCLE or CLEAR_WINDOW_SQUARE; any other value returns
 * CLEAR_EINVAL).  The functions without _ex build the circular window.  For the
 * square window a sub-tile touches a key tile iff some pair has
 * max(dy^2, dx^2) <= r2_max, and admits it fully iff every pair does.
 */
int clear_tile_map_size_ex(int window, int grid_h, int grid_w, int r2_max, int tile_h,
                           int tile_w, int sub_h, int sub_w, int key_h, int key_w,
                           size_t* n_entries);
int clear_tile_map_build_ex(int window, int grid_h, int grid_w, int r2_max, int tile_h,
                            int tile_w, int sub_h, int sub_w, int key_h, int key_w,
                            uint32_t* offsets, uint32_t* key_tiles, uint16_t* flags,
                            size_t cap, size_t* n_entries);
int clear_tile_map_build_device_ex(int window, int grid_h, int grid_w, int r2_max,
                                   int tile_h, int tile_w, int sub_h, int sub_w, int key_h,
                                   int key_w, uint32_t* offsets, uint32_t* key_tiles,
                                   uint16_t* flags, size_t cap, size_t* n_entries,
                                   void* stream);

/*
 * clear_tile_map_descriptors -- the tile map at the attention kernels' own tiling
 * (CLEAR_TILE_H x CLEAR_TILE_W query tiles, CLEAR_SUB_H x CLEAR_SUB_W sub-tiles,
 * CLEAR_KEY_H x CLEAR_KEY_W key tiles), built on `stream` by the same kernels and
 * launch that build the layer entry points' cached copy, together with each
 * entry's descriptor, which the attention kernels read in place of the list.
 * Exposed so that the descriptors can be checked against the list they are
 * derived from (added in 1.4).
 *   window, grid_h, grid_w, r2_max, offsets, key_tiles, flags, cap, n_entries:
 *     as clear_tile_map_build_device_ex at that tiling (offsets, key_tiles and
 *     flags device buffers; n_entries a host pointer).
 *   desc : device, [cap][4] uint32, caller-owned.  For entry e with key tile
 *          (ky, kx) = divmod(key_tiles[e], ceil(grid_w / CLEAR_KEY_W)):
 *            desc[e][0] = ky*CLEAR_KEY_H*grid_w + kx*CLEAR_KEY_W, the token
 *                         offset of the key tile's first cell from the first
 *                         image token;
 *            desc[e][1] = flags[e] | (1 << 16) when the key tile lies wholly on
 *                         the grid, else flags[e];
 *            desc[e][2] = (ky << 16) | kx;
 *            desc[e][3] = grid_h*grid_w - desc[e][0], the image tokens from the
 *                         first cell to the end of the grid.
 * Errors as clear_tile_map_build_device_ex (CLEAR_ENOMEM with *n_entries set
 * when cap is too small; nothing launched); desc must not be NULL when the map
 * has entries.
 */
int clear_tile_map_descriptors(int window, int grid_h, int grid_w, int r2_max,
                               uint32_t* offsets, uint32_t* key_tiles, uint16_t* flags,
                               uint32_t* desc, size_t cap, size_t* n_entries, void* stream);

/* Size of the fixed device scratch of clear_attn_fwd_noalloc (64 MiB per GPU). */
#define CLEAR_NOALLOC_SCRATCH_BYTES (64u << 20)

/*
 * clear_attn_fwd_noalloc -- clear_attn_fwd_ex without any allocation, for callers
 * that cannot allocate device memory: code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc (added in 1.5).
 *
 * Same arguments, checks, result and errors as clear_attn_fwd_ex (the caller
 * still passes q, k, v, out and the optional lse_out).  Instead of the
 * library's cached tile map and workspace, it uses one fixed device array of
 * CLEAR_NOALLOC_SCRATCH_BYTES per GPU, which the device holds from this
 * entry point's first call on it (when its address is looked up, with that
 * device current) until the process ends.  Every call rebuilds the tile map
 * there on `stream` (three small kernels) and keeps the text-row partials
 * there; it computes the window mask per element (no lane-mask table).  It
 * calls no hipMalloc, hipFree, hipMallocAsync or other allocating routine, and
 * creates no events.
 * Limits: the tile map must fit the scratch, else CLEAR_ENOMEM and nothing is
 * launched (the 512 x 512 grid at radius 32 takes 6.9 MB); the text rows use
 * the library's split count, lowered until the partials fit beside the map
 * (one split needs none); an explicit opts->text_splits whose partials do not
 * fit returns CLEAR_ENOMEM.
 * All calls on one GPU share its scratch, which keeps the last call's
 * contents: calls that overlap on one GPU (other streams, other host threads
 * without ordering) race on it and must be serialised by the caller.
 */
int clear_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out,
                           int B, int H, int d, int n_text, int grid_h, int grid_w,
                           const clear_opts* opts, void* stream);

/* Message of the last error raised on the calling thread ("" if none). */
const char* clear_last_error(void);

/* Synchronises every device the library has used, then frees the cached tile
 * maps and the text-row workspaces.  Safe to call at any time from the host. */
void clear_release_cache(void);

/* Library version, major*10000 + minor*100 + patch. */
int clear_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CLEAR_ATTN_H */
