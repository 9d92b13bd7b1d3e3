/* Calls the library's C ABI from plain C (no C++, no Python) on the host-only paths: the workspace size
 * functions, argument checks that reject a call before anything is enqueued, and the error message.
 * Prints "ok" and returns 0 when every check holds. */
#include <stdio.h>
#include <string.h>

#include "pagedkv.h"

#define CHECK(cond)                                                   \
  do {                                                                \
    if (!(cond)) {                                                    \
      printf("check failed at line %d: %s\n", __LINE__, #cond);       \
      return 1;                                                       \
    }                                                                 \
  } while (0)

int main(void) {
  /* the decode workspace grows with the batch; the generic float32 path needs none */
  size_t small = attn_decode_workspace_bytes(8, 16, 8, 128, 16, 256, PKV_BF16);
  size_t big = attn_decode_workspace_bytes(256, 16, 8, 128, 128, 256, PKV_BF16);
  CHECK(small > 0 && small <= big);
  CHECK(attn_decode_workspace_bytes(8, 4, 2, 16, 4, 4, PKV_F32) == 0);
  /* the prefill planner's workspace: bounded batch only */
  CHECK(attn_prefill_workspace_bytes(16, 5000, 512, 16, 8, 128, PKV_BF16) > 0);
  CHECK(attn_prefill_workspace_bytes(5000, 9000, 64, 16, 8, 128, PKV_BF16) == 0);

  /* kv_store with null rows is rejected on the host, with a message */
  int32_t slots[1] = {0};
  int rc = kv_store(NULL, 1024, NULL, 1024, NULL, NULL, 16, slots, 1, 8, 128, PKV_BF16, NULL);
  CHECK(rc == PKV_ERR_INVALID_ARG);
  CHECK(strlen(pkv_last_error()) > 0);
  /* zero tokens is a valid no-op */
  CHECK(kv_store(NULL, 1024, NULL, 1024, NULL, NULL, 16, NULL, 0, 8, 128, PKV_BF16, NULL) == PKV_OK);

  /* num_q_heads not a multiple of num_kv_heads */
  rc = attn_decode_paged(NULL, 0, NULL, NULL, 1, NULL, NULL, 1, 1, 16, 12, 8, 128, 0.1f, NULL, NULL, 0, PKV_BF16,
                         NULL);
  CHECK(rc == PKV_ERR_INVALID_ARG);
  printf("ok\n");
  return 0;
}
