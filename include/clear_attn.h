/*
 * clear_attn.h -- C ABI of libclear_attn.so: the forward pass of CLEAR
 * circular-window attention on AMD Instinct MI355X (gfx950).
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
 * Conventions shared by every entry point
 *   - Return value: CLEAR_OK (0) or a negative error code below.  On error
 *     nothing has been launched or written, and clear_last_error() describes
 *     the problem.  Argument checks run before any HIP call.
 *   - Device pointers are plain addresses in the current HIP device's memory.
 *     `stream` is a hipStream_t passed as void* (NULL = the null stream).  All
 *     work is enqueued on that stream; the library never synchronises it
 *     (except where stated, and when the environment variable CLEAR_DEBUG=1
 *     is set, which synchronises after each launch and maps failures to
 *     CLEAR_EHIP).
 *   - Faults inside kernels surface at the caller's next synchronisation.
 *   - Thread safety: every entry point may be called from several host
 *     threads; the library's caches are guarded by a mutex.
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

/* Query tiling of the attention kernels: a workgroup owns a 16 x 8 cell query
 * tile; each of its four wavefronts owns a 4 x 8 sub-tile; keys stream in
 * chunks of 32.  clear_tile_map_build* accept other values (for testing). */
#define CLEAR_TILE_H 16
#define CLEAR_TILE_W 8
#define CLEAR_SUB_H 4
#define CLEAR_SUB_W 8
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
} clear_opts;

/*
 * clear_attn_fwd -- one CLEAR attention layer, bfloat16, r2 = radius^2.
 *
 *   q, k, v : device, [B, H, N, d] contiguous bfloat16, N = n_text + grid_h*grid_w,
 *             16-byte aligned.  Caller-owned, read only.
 *   out     : device, [B, H, N, d] contiguous bfloat16; caller-owned; must not
 *             overlap q, k or v.  Every element is written.
 *   B, H    : >= 1.  d: 64 or 128.  n_text >= 0.
 *   grid_h, grid_w : 1 .. CLEAR_MAX_GRID.  radius >= 0.
 *   n_text == 0 with an empty window cannot happen here (radius >= 0 admits
 *   the query itself).
 * Arithmetic: bf16 inputs, fp32 accumulation of q.k and of p.v, softmax in
 * fp32 (exp2 form), probabilities rounded to bf16 for the p.v product, output
 * rounded to bf16.
 * The library builds (on the stream, once per (grid_h, grid_w, r2)) and caches
 * the tile map, and owns the text-row workspace; see clear_release_cache.
 */
int clear_attn_fwd(const void* q, const void* k, const void* v, void* out,
                   int B, int H, int d, int n_text, int grid_h, int grid_w,
                   int radius, void* stream);

/*
 * clear_attn_fwd_ex -- as clear_attn_fwd with options: element type (bf16 or
 * fp32; fp32 runs fp32 matrix-core products and keeps probabilities in fp32),
 * explicit r2_max (-1 .. any; n_text == 0 with r2_max < 0 leaves every row
 * empty and returns CLEAR_EINVAL), optional LSE output and the text-row split
 * count.  opts == NULL means {CLEAR_BF16, 0, NULL, 0}.
 */
int clear_attn_fwd_ex(const void* q, const void* k, const void* v, void* out,
                      int B, int H, int d, int n_text, int grid_h, int grid_w,
                      const clear_opts* opts, void* stream);

/*
 * clear_tile_map_size -- sizes of the tile map (host, closed form).
 * The tile map lists, for each query tile, the image keys that any of its
 * queries admits (the union of their windows: the mask of the review's
 * "Core claim" restricted to image pairs), as one run of consecutive columns
 * per key row, and cuts that key list into chunks of `chunk` keys.
 *   *n_runs, *n_chunks : totals over all tiles.
 * Constraints: grid sides 1..CLEAR_MAX_GRID; r2_max >= -1; tile_h, tile_w,
 * sub_h, sub_w >= 1 with sub_h | tile_h, sub_w | tile_w and at most 8
 * sub-tiles per tile; 1 <= chunk <= 4096.
 */
int clear_tile_map_size(int grid_h, int grid_w, int r2_max, int tile_h, int tile_w,
                        int sub_h, int sub_w, int chunk, size_t* n_runs,
                        size_t* n_chunks);

/*
 * clear_tile_map_build -- build the tile map on the host.
 *
 * Tiles are numbered row-major (t = ty * ceil(grid_w/tile_w) + tx); tile t
 * covers grid rows [ty*tile_h, ty*tile_h + tile_h) and columns
 * [tx*tile_w, tx*tile_w + tile_w), clipped to the grid.  Outputs (host memory,
 * caller-owned):
 *   run_offsets   [ntiles + 1] : runs of tile t are run_offsets[t] .. run_offsets[t+1]-1
 *   runs          [2 * n_runs] : (start, length) pairs; start = ky*grid_w + kx0 is the
 *                                image-token index (text not counted) of the run's first
 *                                key; runs ascend by key row
 *   chunk_offsets [ntiles + 1] : chunks of tile t, in the concatenated key list
 *   flags         [n_chunks]   : bit s = sub-tile s (row-major within the tile) admits
 *                                some pair (query on the grid, key in the chunk); bit 8+s
 *                                = the chunk holds `chunk` keys, sub-tile s has a query
 *                                on the grid and admits every such pair
 * runs_cap / flags_cap are the capacities (in runs / in chunks).  If either is
 * too small, returns CLEAR_ENOMEM with *n_runs / *n_chunks set and nothing
 * written; call with caps 0 to query the sizes.
 */
int clear_tile_map_build(int grid_h, int grid_w, int r2_max, int tile_h, int tile_w,
                         int sub_h, int sub_w, int chunk, uint32_t* run_offsets,
                         uint32_t* runs, size_t runs_cap, uint32_t* chunk_offsets,
                         uint16_t* flags, size_t flags_cap, size_t* n_runs,
                         size_t* n_chunks);

/*
 * clear_tile_map_build_device -- same tile map, built by kernels on `stream`
 * into device buffers (same layout and contents, bit for bit, as the host
 * builder).  The sizes are computed on the host first (as clear_tile_map_size);
 * if a capacity is too small it returns CLEAR_ENOMEM with the sizes set and
 * launches nothing.  *n_runs / *n_chunks are host pointers.  Temporary device
 * memory is allocated with stream-ordered allocation and released on the
 * stream.
 */
int clear_tile_map_build_device(int grid_h, int grid_w, int r2_max, int tile_h,
                                int tile_w, int sub_h, int sub_w, int chunk,
                                uint32_t* run_offsets, uint32_t* runs,
                                size_t runs_cap, uint32_t* chunk_offsets,
                                uint16_t* flags, size_t flags_cap, size_t* n_runs,
                                size_t* n_chunks, void* stream);

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
