/* Host-side argument checks of every entry point at extreme values (zero, negative, INT32/INT64 limits, NaN and
 * infinity, sizes whose products overflow 32 bits).  Every call here must be answered on the host: the pointers
 * are stand-ins that are never dereferenced, so each case names the code it must return before anything could
 * be enqueued.  Built plainly and with the host sanitizers (address, undefined behaviour), so an overflow, a
 * read past a buffer or a leak in the checks themselves fails the run.
 * Prints "ok" and returns 0 when every case holds; otherwise prints every failing case and returns 1. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "pagedkv.h"

static int failures = 0;

/* rc must equal want; a failure must leave a message, a success none. */
static void expect(int line, int rc, int want) {
  const char* msg = pkv_last_error();
  if (rc != want) {
    printf("line %d: returned %d, expected %d (%s)\n", line, rc, want, msg);
    ++failures;
  } else if (want != PKV_OK && strlen(msg) == 0) {
    printf("line %d: code %d without a message\n", line, rc);
    ++failures;
  } else if (want == PKV_OK && strlen(msg) != 0) {
    printf("line %d: success left a message (%s)\n", line, msg);
    ++failures;
  }
}
#define EXPECT(call, want) expect(__LINE__, (call), (want))
#define EXPECT_SIZE(cond)                                      \
  do {                                                         \
    if (!(cond)) {                                             \
      printf("line %d: size check failed: %s\n", __LINE__, #cond); \
      ++failures;                                              \
    }                                                          \
  } while (0)

int main(void) {
  /* Stand-ins for device buffers: 256-byte aligned, never dereferenced (every call below is refused). */
  void* const P = (void*)(uintptr_t)0x100000;
  const int32_t* const I = (const int32_t*)(uintptr_t)0x200000;
  int32_t* const O = (int32_t*)(uintptr_t)0x300000;
  const float nan = NAN, inf = INFINITY;
  const int32_t BIG = INT32_MAX, NEG = INT32_MIN;

  /* ---- kv_slot_mapping ---- */
  EXPECT(kv_slot_mapping(I, I, NULL, I, -1, 4, 16, 8, O, NULL), PKV_ERR_INVALID_ARG);
  EXPECT(kv_slot_mapping(I, I, NULL, I, 2, NEG, 16, 8, O, NULL), PKV_ERR_INVALID_ARG);
  EXPECT(kv_slot_mapping(I, I, NULL, I, 2, 4, 16, NEG, O, NULL), PKV_ERR_INVALID_ARG);
  EXPECT(kv_slot_mapping(I, I, NULL, I, 2, 4, 0, 8, O, NULL), PKV_ERR_INVALID_ARG);
  EXPECT(kv_slot_mapping(I, I, NULL, I, 2, 4, NEG, 8, O, NULL), PKV_ERR_INVALID_ARG);
  EXPECT(kv_slot_mapping(I, I, I, I, 2, 4, 16, 8, O, NULL), PKV_ERR_INVALID_ARG);     /* both modes */
  EXPECT(kv_slot_mapping(NULL, NULL, NULL, I, 2, 4, 16, 8, O, NULL), PKV_ERR_INVALID_ARG); /* neither */
  EXPECT(kv_slot_mapping(I, I, NULL, I, 2, 4, 16, 8, NULL, NULL), PKV_ERR_INVALID_ARG);
  EXPECT(kv_slot_mapping(I, I, NULL, NULL, 2, 4, 16, 8, O, NULL), PKV_ERR_INVALID_ARG);
  EXPECT(kv_slot_mapping(I, I, NULL, I, 2, BIG, BIG, 8, O, NULL), PKV_ERR_UNSUPPORTED);
  EXPECT(kv_slot_mapping(I, I, NULL, I, 2, 65536, 32768, 8, O, NULL), PKV_ERR_UNSUPPORTED); /* 2^31 positions */
  EXPECT(kv_slot_mapping(I, I, NULL, I, BIG, 4, 16, 0, NULL, NULL), PKV_OK);           /* no tokens */

  /* ---- kv_store ---- */
  EXPECT(kv_store(P, 1024, P, 1024, P, P, 16, I, 1, 8, 128, (pkv_dtype)7, NULL), PKV_ERR_INVALID_ARG);
  EXPECT(kv_store(P, 1024, P, 1024, P, P, 16, I, -1, 8, 128, PKV_BF16, NULL), PKV_ERR_INVALID_ARG);
  EXPECT(kv_store(P, 1024, P, 1024, P, P, INT64_MIN, I, 1, 8, 128, PKV_BF16, NULL), PKV_ERR_INVALID_ARG);
  EXPECT(kv_store(P, 1024, P, 1024, P, P, 16, I, 1, 0, 128, PKV_BF16, NULL), PKV_ERR_INVALID_ARG);
  EXPECT(kv_store(P, 1024, P, 1024, P, P, 16, I, 1, 8, NEG, PKV_BF16, NULL), PKV_ERR_INVALID_ARG);
  EXPECT(kv_store(P, INT64_MAX, P, INT64_MAX, P, P, 16, I, 1, BIG, BIG, PKV_BF16, NULL), PKV_ERR_UNSUPPORTED);
  EXPECT(kv_store(P, 1023, P, 1024, P, P, 16, I, 1, 8, 128, PKV_BF16, NULL), PKV_ERR_INVALID_ARG);
  EXPECT(kv_store(P, 1024, P, INT64_MIN, P, P, 16, I, 1, 8, 128, PKV_BF16, NULL), PKV_ERR_INVALID_ARG);
  EXPECT(kv_store(P, 1024, NULL, 1024, P, P, 16, I, 1, 8, 128, PKV_BF16, NULL), PKV_ERR_INVALID_ARG);
  EXPECT(kv_store(P, 1024, P, 1024, P, P, 16, NULL, 1, 8, 128, PKV_BF16, NULL), PKV_ERR_INVALID_ARG);
  /* 2^31 - 1 tokens of 2^24-element rows: more elements than one launch addresses */
  EXPECT(kv_store(P, 1 << 24, P, 1 << 24, P, P, 16, I, BIG, 1 << 10, 1 << 14, PKV_BF16, NULL),
         PKV_ERR_UNSUPPORTED);
  EXPECT(kv_store(NULL, 1024, NULL, 1024, NULL, NULL, INT64_MAX, NULL, 0, 8, 128, PKV_F32, NULL), PKV_OK);

  /* ---- kv_store_qk_norm_rope ---- */
#define QKR(qs, hq, hkv, hd, eps, theta, n) \
  kv_store_qk_norm_rope(P, qs, P, 1024, P, 1024, I, P, P, eps, theta, P, P, P, 16, I, n, hq, hkv, hd, PKV_BF16, NULL)
  EXPECT(QKR(2048, 16, 8, 48, 1e-6f, 1e4f, 1), PKV_ERR_UNSUPPORTED);   /* head_dim not a power of two */
  EXPECT(QKR(2048, 16, 8, 512, 1e-6f, 1e4f, 1), PKV_ERR_UNSUPPORTED);
  EXPECT(QKR(2048, 16, 8, 128, nan, 1e4f, 1), PKV_ERR_INVALID_ARG);
  EXPECT(QKR(2048, 16, 8, 128, -1.f, 1e4f, 1), PKV_ERR_INVALID_ARG);
  EXPECT(QKR(2048, 16, 8, 128, inf, 1e4f, 1), PKV_ERR_INVALID_ARG);
  EXPECT(QKR(2048, 16, 8, 128, 1e-6f, 0.f, 1), PKV_ERR_INVALID_ARG);
  EXPECT(QKR(2048, 16, 8, 128, 1e-6f, inf, 1), PKV_ERR_INVALID_ARG);
  EXPECT(QKR(2048, 16, 8, 128, 1e-6f, nan, 1), PKV_ERR_INVALID_ARG);
  EXPECT(QKR(2047, 16, 8, 128, 1e-6f, 1e4f, 1), PKV_ERR_INVALID_ARG);  /* q row short of 16 x 128 */
  EXPECT(QKR(INT64_MAX, BIG, 1, 128, 1e-6f, 1e4f, 1), PKV_ERR_UNSUPPORTED); /* more query heads than a grid */
  EXPECT(QKR(2048, 16, 6, 128, 1e-6f, 1e4f, 1), PKV_ERR_INVALID_ARG);  /* 16 heads over 6 kv heads */
  EXPECT(QKR(2048, NEG, 8, 128, 1e-6f, 1e4f, 1), PKV_ERR_INVALID_ARG);
  EXPECT(QKR(2048, 16, 8, 128, 1e-6f, 1e4f, -5), PKV_ERR_INVALID_ARG);
  EXPECT(kv_store_qk_norm_rope(P, 2048, P, 1024, P, 1024, NULL, P, P, 1e-6f, 1e4f, P, P, P, 16, I, 1, 16, 8, 128,
                               PKV_BF16, NULL),
         PKV_ERR_INVALID_ARG);                                           /* positions missing */
  EXPECT(QKR(2048, 16, 8, 128, 0.f, 1e4f, 0), PKV_OK);                  /* no tokens */

  /* ---- attn_prefill_varlen ---- */
#define PF(hq, hkv, hd, nq, nk, mq, mk, b, scale, causal, bt, mbps, bs) \
  attn_prefill_varlen(P, 4096, P, 1024, P, 1024, I, I, mq, mk, b, nq, nk, hq, hkv, hd, scale, causal, bt, mbps, bs, \
                      P, NULL, 0, PKV_BF16, NULL)
  EXPECT(PF(16, 8, 128, 64, 64, 64, 64, 1, 0.1f, 2, NULL, 0, 0), PKV_ERR_INVALID_ARG);   /* causal 2 */
  EXPECT(PF(16, 8, 128, 64, 64, 64, 64, 1, nan, 1, NULL, 0, 0), PKV_ERR_INVALID_ARG);
  EXPECT(PF(16, 8, 128, 64, 64, 64, 64, 1, -inf, 1, NULL, 0, 0), PKV_ERR_INVALID_ARG);
  EXPECT(PF(16, 8, 128, 64, INT64_MIN, 64, 64, 1, 0.1f, 1, NULL, 0, 0), PKV_ERR_INVALID_ARG);
  EXPECT(PF(16, 8, 128, NEG, 64, 64, 64, 1, 0.1f, 1, NULL, 0, 0), PKV_ERR_INVALID_ARG);
  EXPECT(PF(16, 8, 128, 64, 64, -1, 64, 1, 0.1f, 1, NULL, 0, 0), PKV_ERR_INVALID_ARG);
  EXPECT(PF(16, 8, 128, 64, 64, 64, NEG, 1, 0.1f, 1, NULL, 0, 0), PKV_ERR_INVALID_ARG);
  EXPECT(PF(16, 8, 128, 64, 64, 64, 64, 70000, 0.1f, 1, NULL, 0, 0), PKV_ERR_UNSUPPORTED); /* batch > grid */
  EXPECT(PF(16, 8, 512, 64, 64, 64, 64, 1, 0.1f, 1, NULL, 0, 0), PKV_ERR_UNSUPPORTED);     /* head_dim 512 */
  EXPECT(PF(16, 8, 0, 64, 64, 64, 64, 1, 0.1f, 1, NULL, 0, 0), PKV_ERR_INVALID_ARG);
  EXPECT(PF(NEG, 8, 128, 64, 64, 64, 64, 1, 0.1f, 1, NULL, 0, 0), PKV_ERR_INVALID_ARG);
  EXPECT(PF(16, 8, 256, 64, 64, 64, 64, 1, 0.1f, 1, NULL, 0, 0), PKV_ERR_INVALID_ARG);     /* k row 1024 < 8 x 256 */
  EXPECT(PF(32, 8, 256, 64, 64, 64, 64, 1, 0.1f, 1, NULL, 0, 0), PKV_ERR_INVALID_ARG);     /* q row 4096 < 32 x 256 */
  /* paged: slots not a whole number of blocks, too many blocks for int32, positions beyond 2^31 */
  EXPECT(PF(16, 8, 128, 64, 1000, 64, 64, 1, 0.1f, 1, I, 4, 256), PKV_ERR_INVALID_ARG);
  EXPECT(PF(16, 8, 128, 64, INT64_MAX - (INT64_MAX % 2), 64, 64, 1, 0.1f, 1, I, 4, 2), PKV_ERR_UNSUPPORTED);
  EXPECT(PF(16, 8, 128, 64, 1 << 20, 64, 64, 1, 0.1f, 1, I, BIG, 256), PKV_ERR_UNSUPPORTED);
  EXPECT(PF(16, 8, 128, 64, 1 << 20, 64, 64, 1, 0.1f, 1, I, 0, 256), PKV_ERR_INVALID_ARG);
  EXPECT(PF(16, 8, 128, 64, 1 << 20, 64, 64, 1, 0.1f, 1, I, 4, NEG), PKV_ERR_INVALID_ARG);
  /* contiguous: k/v rows shorter than 8 x 128 */
  EXPECT(attn_prefill_varlen(P, 2048, P, 1023, P, 1024, I, I, 64, 64, 1, 64, 64, 16, 8, 128, 0.1f, 1, NULL, 0, 0, P,
                             NULL, 0, PKV_BF16, NULL),
         PKV_ERR_INVALID_ARG);
  EXPECT(attn_prefill_varlen(P, 2048, P, 1024, P, 1024, I, NULL, 64, 64, 1, 64, 64, 16, 8, 128, 0.1f, 1, NULL, 0, 0,
                             P, NULL, 0, PKV_BF16, NULL),
         PKV_ERR_INVALID_ARG);                                            /* cu_seqlens_k missing */
  /* a workspace smaller than the planner needs */
  EXPECT(attn_prefill_varlen(P, 2048, P, 1024, P, 1024, I, I, 512, 4096, 16, 5000, 1 << 20, 16, 8, 128, 0.1f, 1, I,
                             16, 256, P, P, 8, PKV_BF16, NULL),
         PKV_ERR_WORKSPACE);
  EXPECT(PF(16, 8, 128, 0, 64, 64, 64, 1, 0.1f, 1, NULL, 0, 0), PKV_OK);   /* no query tokens */
  EXPECT(PF(16, 8, 128, 64, 64, 64, 64, 0, 0.1f, 1, NULL, 0, 0), PKV_OK);  /* empty batch */

  /* ---- workspace sizes: defined for every input, 0 where no workspace is used or the sizes are refused ---- */
  EXPECT_SIZE(attn_prefill_workspace_bytes(BIG, BIG, BIG, 16, 8, 128, PKV_BF16) == 0);
  EXPECT_SIZE(attn_prefill_workspace_bytes(NEG, BIG, BIG, 16, 8, 128, PKV_BF16) == 0);
  EXPECT_SIZE(attn_prefill_workspace_bytes(16, NEG, NEG, 16, 8, 128, PKV_BF16) == 0);
  EXPECT_SIZE(attn_prefill_workspace_bytes(16, BIG, BIG, BIG, 1, 128, PKV_BF16) == 0);
  EXPECT_SIZE(attn_prefill_workspace_bytes(16, 5000, 512, 16, 0, 128, PKV_BF16) == 0);
  EXPECT_SIZE(attn_prefill_workspace_bytes(16, 5000, 512, 16, 8, 128, PKV_F32) == 0);
  EXPECT_SIZE(attn_prefill_workspace_bytes(16, 5000, 512, 16, 8, 64, PKV_BF16) == 0);
  EXPECT_SIZE(attn_prefill_workspace_bytes(16, 5000, 512, 16, 8, 128, PKV_BF16) > 0);
  EXPECT_SIZE(attn_prefill_workspace_bytes(16, BIG, BIG, 16, 8, 128, PKV_BF16) > 0);  /* 64-bit unit count */
  EXPECT_SIZE(attn_decode_workspace_bytes(BIG, 16, 8, 128, 16, 256, PKV_BF16) == 0);
  EXPECT_SIZE(attn_decode_workspace_bytes(65536, 16, 8, 128, 16, 256, PKV_BF16) == 0);
  EXPECT_SIZE(attn_decode_workspace_bytes(65535, 16, 8, 128, 16, 256, PKV_BF16) > 0);
  EXPECT_SIZE(attn_decode_workspace_bytes(64, BIG, 1, 128, 16, 256, PKV_BF16) == 0);
  EXPECT_SIZE(attn_decode_workspace_bytes(64, 16, 8, 128, BIG, BIG, PKV_BF16) == 0);
  EXPECT_SIZE(attn_decode_workspace_bytes(64, 16, 8, 128, NEG, 256, PKV_BF16) == 0);
  EXPECT_SIZE(attn_decode_workspace_bytes(NEG, 16, 8, 128, 16, 256, PKV_BF16) == 0);
  EXPECT_SIZE(attn_decode_workspace_bytes(64, 16, 8, 128, 16, 256, (pkv_dtype)9) == 0);

  /* ---- attn_decode_paged ---- */
#define DEC(qs, nb, b, mbps, bs, hq, hkv, hd, scale, ws, wsb) \
  attn_decode_paged(P, qs, P, P, nb, I, I, b, mbps, bs, hq, hkv, hd, scale, P, ws, wsb, PKV_BF16, NULL)
  EXPECT(DEC(2048, 64, 70000, 16, 256, 16, 8, 128, 0.1f, P, 1 << 30), PKV_ERR_UNSUPPORTED);
  EXPECT(DEC(2048, 64, -1, 16, 256, 16, 8, 128, 0.1f, P, 1 << 30), PKV_ERR_INVALID_ARG);
  EXPECT(DEC(2048, NEG, 4, 16, 256, 16, 8, 128, 0.1f, P, 1 << 30), PKV_ERR_INVALID_ARG);
  EXPECT(DEC(2048, 64, 4, 16, 0, 16, 8, 128, 0.1f, P, 1 << 30), PKV_ERR_INVALID_ARG);
  EXPECT(DEC(2048, 64, 4, 0, 256, 16, 8, 128, 0.1f, P, 1 << 30), PKV_ERR_INVALID_ARG);
  EXPECT(DEC(2048, 64, 4, BIG, BIG, 16, 8, 128, 0.1f, P, 1 << 30), PKV_ERR_UNSUPPORTED);
  EXPECT(DEC(2048, 64, 4, 16, 256, 16, 8, 128, inf, P, 1 << 30), PKV_ERR_INVALID_ARG);
  EXPECT(DEC(2048, 64, 4, 16, 256, 16, 8, 128, nan, P, 1 << 30), PKV_ERR_INVALID_ARG);
  EXPECT(DEC(2047, 64, 4, 16, 256, 16, 8, 128, 0.1f, P, 1 << 30), PKV_ERR_INVALID_ARG);
  EXPECT(DEC(INT64_MIN, 64, 4, 16, 256, 16, 8, 128, 0.1f, P, 1 << 30), PKV_ERR_INVALID_ARG);
  EXPECT(DEC(2048, 0, 4, 16, 256, 16, 8, 128, 0.1f, P, 1 << 30), PKV_ERR_INVALID_ARG);   /* rows but no blocks */
  EXPECT(DEC(2048, 64, 4, 16, 256, 16, 8, 128, 0.1f, NULL, 0), PKV_ERR_WORKSPACE);       /* fast path, no ws */
  EXPECT(DEC(2048, 64, 4, 16, 256, 16, 8, 128, 0.1f, P, 256), PKV_ERR_WORKSPACE);
  EXPECT(DEC(2048, 64, 4, 16, 256, 16, 8, 300, 0.1f, P, 1 << 30), PKV_ERR_UNSUPPORTED);  /* head_dim 300 */
  EXPECT(attn_decode_paged(P, 2048, P, P, 64, NULL, I, 4, 16, 256, 16, 8, 128, 0.1f, P, P, 1 << 30, PKV_BF16, NULL),
         PKV_ERR_INVALID_ARG);                                                          /* context_lens missing */
  EXPECT(DEC(2048, 64, 0, 16, 256, 16, 8, 128, 0.1f, NULL, 0), PKV_OK);                 /* empty batch */

  /* ---- attn_decode_paged_store and its allocation-free form ---- */
#define DST(ks, vs, kn, nb, bs, b) \
  attn_decode_paged_store(P, 2048, kn, ks, P, vs, P, P, nb, I, I, b, 16, bs, 16, 8, 128, 0.1f, P, O, P, 1 << 30, \
                          PKV_BF16, NULL)
  EXPECT(DST(1023, 1024, P, 64, 256, 4), PKV_ERR_INVALID_ARG);
  EXPECT(DST(1024, INT64_MIN, P, 64, 256, 4), PKV_ERR_INVALID_ARG);
  EXPECT(DST(1024, 1024, NULL, 64, 256, 4), PKV_ERR_INVALID_ARG);
  EXPECT(DST(1024, 1024, P, BIG, 256, 4), PKV_ERR_UNSUPPORTED);   /* more slots than int32 slot_mapping holds */
  EXPECT(DST(1024, 1024, P, 8388608, 256, 4), PKV_ERR_UNSUPPORTED); /* exactly 2^31 slots */
  EXPECT(DST(1024, 1024, P, 64, 256, 0), PKV_OK);
  EXPECT(attn_decode_paged_store_noalloc(P, 2048, P, 1024, P, 1024, P, P, 64, I, I, 20000, 16, 256, 16, 8, 128, 0.1f,
                                         P, O, PKV_BF16, NULL),
         PKV_ERR_WORKSPACE);                                      /* workspace beyond the static 32 MiB */
  EXPECT(attn_decode_paged_store_noalloc(P, 2048, P, 1024, P, 1024, P, P, 64, I, I, BIG, 16, 256, 16, 8, 128, 0.1f,
                                         P, O, PKV_BF16, NULL),
         PKV_ERR_UNSUPPORTED);                                    /* batch beyond a grid dimension */
  EXPECT(attn_decode_paged_store_noalloc(P, 2048, P, 1024, P, 1024, P, P, 64, I, I, 4, 16, 256, 16, 8, 128, nan, P,
                                         O, PKV_BF16, NULL),
         PKV_ERR_INVALID_ARG);

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
