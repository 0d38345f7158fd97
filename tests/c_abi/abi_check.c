/* A plain C99 caller of libclear_attn.so: the header compiles as C, the
 * entry points link, and calls that need no GPU behave as documented
 * (version, tile-map size query, argument errors reported before any HIP
 * call).  Prints one line per check; exits non-zero on the first failure. */
#include <stdio.h>
#include <string.h>

#include "clear_attn.h"

#define CHECK(cond, ...)                  \
  do {                                    \
    if (!(cond)) {                        \
      printf("FAIL: " __VA_ARGS__);       \
      printf("\n");                       \
      return 1;                           \
    }                                     \
  } while (0)

int main(void) {
  int v = clear_version();
  CHECK(v >= 10000, "clear_version() = %d", v);
  printf("version %d\n", v);

  /* 8 x 8 grid, r2 = 4, the kernels' tiling: one 16 x 8 query tile (clipped),
     key tiles of 4 x 8 cells: both key-tile rows are touched */
  size_t n = 0;
  int rc = clear_tile_map_size(8, 8, 4, CLEAR_TILE_H, CLEAR_TILE_W, CLEAR_SUB_H, CLEAR_SUB_W, CLEAR_KEY_H,
                               CLEAR_KEY_W, &n);
  CHECK(rc == CLEAR_OK && n == 2, "clear_tile_map_size rc %d n %zu", rc, n);
  printf("tile map entries %zu\n", n);

  /* d = 32 is not supported: CLEAR_EINVAL with a message, nothing launched */
  rc = clear_attn_fwd((const void*)16, (const void*)16, (const void*)16, (void*)4096, 1, 1, 32, 0, 4, 4, 1,
                      NULL);
  CHECK(rc == CLEAR_EINVAL, "clear_attn_fwd(d = 32) rc %d", rc);
  const char* msg = clear_last_error();
  CHECK(msg != NULL && strlen(msg) > 0, "no error message");
  printf("rejected: %s\n", msg);

  /* options: an unknown window is rejected */
  clear_opts o;
  memset(&o, 0, sizeof o);
  o.dtype = CLEAR_FP32;
  o.r2_max = 4;
  o.window = 5;
  rc = clear_attn_fwd_ex((const void*)16, (const void*)16, (const void*)16, (void*)4096, 1, 1, 64, 0, 4, 4,
                         &o, NULL);
  CHECK(rc == CLEAR_EINVAL, "clear_attn_fwd_ex(window = 5) rc %d", rc);
  printf("rejected: %s\n", clear_last_error());
  printf("ok\n");
  return 0;
}
