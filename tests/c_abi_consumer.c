/* A plain C99 consumer of the C ABI: includes only include/paged_attn.h,
 * links libpagedattn, and exercises the host-side paths (size queries,
 * status strings, argument errors) that return before any GPU work. */
#include <stdio.h>
#include <string.h>
#include "paged_attn.h"

static int failures = 0;
#define CHECK(c)                                               \
  do {                                                         \
    if (!(c)) {                                                \
      fprintf(stderr, "check failed line %d: %s\n", __LINE__, #c); \
      ++failures;                                              \
    }                                                          \
  } while (0)

int main(void) {
  pkv_geometry_t g;
  memset(&g, 0, sizeof g);
  g.num_blocks = 1024;
  g.block_size = 16;
  g.num_heads = 32;
  g.num_kv_heads = 8;
  g.head_dim = 128;
  g.kv_dtype = PKV_BF16;

  CHECK(pkv_version() >= 100);
  CHECK(strncmp(pkv_status_string(PKV_EINVAL), "PKV_EINVAL", 10) == 0);
  CHECK(paged_attn_decode_workspace_bytes(&g, 4, 1000, 0, 0, 0) > 0);
  CHECK(paged_attn_decode_workers(&g, 4, 1000, 0, 0) > 0);
  /* null outputs: rejected before anything is enqueued */
  CHECK(paged_attn_decode(&g, NULL, NULL, NULL, NULL, NULL, NULL, 8, NULL, 4, 100, 0, 0, 0.1f, 0, NULL, 0,
                          NULL) == PKV_EINVAL);
  CHECK(paged_attn_prefill(&g, NULL, NULL, NULL, NULL, NULL, NULL, NULL, 8, NULL, 4, 4, 100, 0, 0, 0.1f,
                           NULL) == PKV_EINVAL);
  /* 8-bit pools: their own entry points (prefill needs no workspace) */
  g.kv_dtype = PKV_I8;
  CHECK(paged_attn_decode_workspace_bytes(&g, 4, 1000, 0, 0, 0) > 0);
  CHECK(paged_attn_decode(&g, NULL, NULL, NULL, NULL, NULL, NULL, 8, NULL, 4, 100, 0, 0, 0.1f, 0, NULL, 0,
                          NULL) == PKV_EUNSUPPORTED);
  CHECK(paged_attn_prefill_quant(&g, NULL, NULL, NULL, PKV_BF16, NULL, NULL, NULL, NULL, NULL, NULL, 8, NULL, 4, 4,
                                 100, 0, 0, 0.1f, NULL) == PKV_EINVAL);
  /* an unsupported head size */
  g.head_dim = 96;
  CHECK(paged_attn_decode_workspace_bytes(&g, 4, 1000, 0, 0, 0) == 0);
  /* the no-alloc decode refuses 8-bit pools before anything else */
  g.head_dim = 128;
  CHECK(paged_attn_decode_noalloc(&g, NULL, NULL, NULL, NULL, NULL, NULL, 8, NULL, 4, 100, 0, 0, 0.1f, 0, NULL) ==
        PKV_EUNSUPPORTED);
  if (failures) return 1;
  printf("c abi consumer ok\n");
  return 0;
}
