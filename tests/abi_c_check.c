/* A C99 caller of the library: includes the public headers, links
 * libcompressor.so and calls the host-only paths (workspace sizes, shape and
 * argument checks, status strings) through the declared prototypes, so the
 * headers and the library agree as a C compiler sees them.  Nothing here
 * touches a GPU.  Prints one line per failed check and exits non-zero if
 * any failed. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "compressor.h"
#include "nsa_compress.h"

static int failures = 0;

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      printf("FAIL line %d: %s\n", __LINE__, #cond);                  \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

static compressor_shape shape(int32_t ratio, int32_t d, int32_t h, int32_t rotate, int32_t bs,
                              int32_t nblocks, int32_t stride) {
  compressor_shape s;
  s.ratio = ratio;
  s.head_dim = d;
  s.hidden = h;
  s.rope_head_dim = 64;
  s.rotate = rotate;
  s.block_size = bs;
  s.num_blocks = nblocks;
  s.table_stride = stride;
  return s;
}

int main(void) {
  /* the 128K C4A prefill: pooled rows and staging, no projection buffer */
  compressor_shape c4a = shape(4, 512, 7168, 1, 128, 1, 1);
  size_t bytes = 0;
  CHECK(compressor_prefill_workspace_size(&c4a, 131072, 1, 32768, &bytes) == CMP_OK);
  CHECK(bytes >= (size_t)32768 * 512 * 4 && bytes < (size_t)131072 * 2048 * 4);
  /* decode workspaces fit the allocation-free entry point's scratch */
  bytes = 0;
  CHECK(compressor_decode_workspace_size(&c4a, 32, 32, &bytes) == CMP_OK);
  CHECK(bytes > 0 && bytes <= CMP_DECODE_SCRATCH_BYTES);
  compressor_shape c128a = shape(128, 512, 10240, 0, 64, 128, 2);
  bytes = 0;
  CHECK(compressor_decode_workspace_size(&c128a, 64, 64, &bytes) == CMP_OK);
  CHECK(bytes > 0 && bytes <= CMP_DECODE_SCRATCH_BYTES);
  CHECK(compressor_decode_workspace_size(&c4a, 65, 65, &bytes) == CMP_ERR_UNSUPPORTED);

  /* shape checks */
  compressor_shape bad = c4a;
  bad.ratio = 3;
  CHECK(compressor_prefill_workspace_size(&bad, 64, 1, 16, &bytes) == CMP_ERR_UNSUPPORTED);
  bad = c4a;
  bad.head_dim = 256;
  CHECK(compressor_prefill_workspace_size(&bad, 64, 1, 16, &bytes) == CMP_ERR_UNSUPPORTED);
  bad = c4a;
  bad.hidden = 7000;
  CHECK(compressor_prefill_workspace_size(&bad, 64, 1, 16, &bytes) == CMP_ERR_INVALID);
  bad = c4a;
  bad.block_size = 4; /* two 4-row blocks needed for the 8-slot ring, stride 1 */
  CHECK(compressor_prefill_workspace_size(&bad, 64, 1, 16, &bytes) == CMP_ERR_INVALID);

  /* argument checks before any launch */
  compressor_args a;
  memset(&a, 0, sizeof a);
  a.batch = 1;
  a.T = 4;
  CHECK(compressor_prefill(&c4a, NULL, NULL) == CMP_ERR_NULLPTR);
  CHECK(compressor_decode(&c4a, NULL, NULL) == CMP_ERR_NULLPTR);
  CHECK(compressor_prefill(&c4a, &a, NULL) == CMP_ERR_NULLPTR);
  CHECK(compressor_decode(&c4a, &a, NULL) == CMP_ERR_NULLPTR);
  CHECK(compressor_decode_noalloc(&c4a, &a, NULL, NULL) == CMP_ERR_NULLPTR);
  CHECK(compressor_pack_weights(&c4a, NULL, NULL, NULL, NULL) == CMP_ERR_NULLPTR);
  CHECK(compressor_state_init(&c4a, NULL, NULL, NULL) == CMP_ERR_NULLPTR);
  CHECK(compressor_state_reset(&c4a, NULL, NULL, NULL, NULL, NULL, 0, 0, NULL, NULL) == CMP_OK);
  CHECK(compressor_state_reset(&c4a, NULL, NULL, NULL, NULL, NULL, -1, 4, NULL, NULL) ==
        CMP_ERR_INVALID);
  CHECK(compressor_state_reset(&c4a, NULL, NULL, NULL, NULL, NULL, 2, 4, NULL, NULL) ==
        CMP_ERR_NULLPTR);
  int32_t code = 0;
  CHECK(compressor_last_device_error(NULL, NULL, &code) == CMP_ERR_NULLPTR);
  CHECK(compressor_epilog(NULL, 0, 512, NULL, NULL, NULL, 0, NULL, NULL) == CMP_OK);
  CHECK(compressor_epilog(NULL, 4, 100, NULL, NULL, NULL, 8, NULL, NULL) == CMP_ERR_INVALID);
  CHECK(compressor_set_prefill_tile_rows(64) == CMP_ERR_INVALID);
  CHECK(compressor_set_prefill_tile_rows(0) == CMP_OK);
  int32_t launches = -1;
  double ms = -1.0;
  CHECK(compressor_timing_query("gemm", &launches, &ms) == CMP_OK && launches == 0);
  CHECK(compressor_timing_enable(3) == CMP_ERR_INVALID);

  /* NSA shape checks */
  nsa_shape ns;
  ns.head_num = 32;
  ns.head_dim = 128;
  ns.compress_block_size = 32;
  ns.compress_stride = 16;
  ns.page_block_size = 128;
  ns.dtype = NSA_BF16;
  ns.layout = NSA_LAYOUT_PAGED;
  nsa_args na;
  memset(&na, 0, sizeof na);
  CHECK(nsa_compress_with_cache(&ns, &na, NULL) == CMP_ERR_NULLPTR);
  ns.compress_stride = 24;
  CHECK(nsa_compress_with_cache(&ns, &na, NULL) == CMP_ERR_UNSUPPORTED);

  /* status strings */
  CHECK(strcmp(compressor_status_str(CMP_OK), "ok") == 0);
  CHECK(strstr(compressor_status_str(CMP_ERR_WORKSPACE), "workspace") != NULL);
  CHECK(strcmp(compressor_status_str(99), "unknown status") == 0);

  printf("abi_c_check: %d failures\n", failures);
  return failures != 0;
}
