/*
 * pagedkv.h -- C ABI of the paged-KV attention hot path on AMD Instinct MI355X (gfx950).
 *
 * One attention layer of a GQA decoder step, as three operations on one GPU:
 *   kv_store             scatter each new token's K/V row into a paged cache by slot_mapping;
 *   kv_store_qk_norm_rope  the same store with QK-Norm and RoPE of q and k fused in front of it;
 *   attn_prefill_varlen  causal attention over sequences packed by cu_seqlens, reading K/V either from
 *                        this step's rows or, for prefix-cache / chunked prefill, from the paged cache;
 *   attn_decode_paged    one query per sequence against its whole history in the paged cache;
 *   attn_decode_paged_store  the decode step's store and attention fused in one call;
 * plus kv_slot_mapping, which builds slot_mapping from the block tables on the device.
 *
 * Sources (three web pages on the attention layer of nano-vLLM; cited by tag, title and section):
 *   [P1] "Nano-VLLM全代码解析笔记(5)-laynorm和attention", m.demingchina.com/news/18656
 *   [P2] nano-vllm lesson on the Qwen3 attention sub-layer, www.yeyulingfeng.com/a/738130.html
 *   [P3] "课程 04 · KV 到底写到了哪一格", diomchen.github.io/lessons/0004-attention-slot-mapping.html
 *
 * Conventions shared by every entry point
 *   Memory.   Every pointer is device memory owned by the caller.  The library allocates nothing, keeps
 *             no pointer after it returns, and writes only the arrays documented as outputs.
 *   Streams.  Work is enqueued on `stream` (NULL = the default stream) and the call returns without
 *             waiting.  Issuing kv_store and then an attention call on the same stream gives the
 *             store-before-attend order the method needs [P3 §4 note].
 *   Layout.   Token rows are [heads, head_dim] with head_dim contiguous; `*_stride` arguments are the
 *             distance between consecutive token rows, in elements (>= heads * head_dim), so rows sliced
 *             out of a merged qkv buffer can be passed as they are.  A paged cache is
 *             [num_blocks, block_size, num_kv_heads, head_dim], contiguous: slot s = block * block_size +
 *             cell holds elements [s*D, s*D + D) with D = num_kv_heads * head_dim [P2 §5.1; P3 §2].
 *   Metadata. int32 arrays, as on the pages [P3 §1 table]: cu_seqlens [batch+1] prefix sums,
 *             block_tables [batch, max_blocks_per_seq] row-major padded with -1, context_lens [batch].
 *   Heads.    Query head h reads kv head h / (num_q_heads / num_kv_heads): consecutive groups share a
 *             kv head [P2 §3].
 *   Types.    PKV_BF16 (raw bf16 storage, float32 accumulation, outputs rounded to nearest-even) or
 *             PKV_F32 (float32 throughout).
 *   Errors.   Arguments are checked on the host before anything is enqueued.  A nonzero return means
 *             nothing was launched (except PKV_ERR_HIP, reported by the launch itself); pkv_last_error()
 *             then describes the failure.  No call aborts the process.
 *   Device-side values (slot_mapping, block tables, cu_seqlens, context_lens) cannot be checked without
 *   a copy to the host; they are clamped so that no kernel ever reads or writes outside the buffers the
 *   sizes describe, but out-of-range values give unspecified (not faulting) results, noted per call.
 */
#ifndef PAGEDKV_H
#define PAGEDKV_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PKV_F32 = 0,
  PKV_BF16 = 1,
  /* Range markers, not dtypes: they give the type every int32 value, so whatever a C caller passes is a
   * value of the type (and is refused with PKV_ERR_INVALID_ARG unless it names a dtype above). */
  PKV_DTYPE_RANGE_MIN_ = -2147483647 - 1,
  PKV_DTYPE_RANGE_MAX_ = 2147483647
} pkv_dtype;

enum {
  PKV_OK = 0,
  PKV_ERR_INVALID_ARG = -1, /* a null pointer, a negative size, inconsistent shapes or strides */
  PKV_ERR_UNSUPPORTED = -2, /* a valid request the library does not implement (e.g. head_dim > 256) */
  PKV_ERR_WORKSPACE = -3,   /* a workspace smaller than its size function requires (or missing for decode) */
  PKV_ERR_HIP = -4          /* the HIP runtime reported an error at launch */
};

/* Thread-local, NUL-terminated description of the last nonzero return on this thread ("" if none). */
const char* pkv_last_error(void);

/*
 * kv_slot_mapping -- the cache slot of every token this step writes [P3 §2; §9 exercise C].
 *
 * Slot of position p of sequence b: block_tables[b][p / block_size] * block_size + p % block_size.
 * Prefill mode (context_lens == NULL): token rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) are the last
 *   Lq = cu_seqlens_q[b+1]-cu_seqlens_q[b] of Lk = cu_seqlens_k[b+1]-cu_seqlens_k[b] positions, i.e.
 *   positions Lk-Lq .. Lk-1 (cu_seqlens_k == NULL means Lk = Lq: nothing cached before this step).
 * Decode mode (context_lens != NULL, both cu_seqlens NULL): row b is position context_lens[b]-1.
 * Output slot_mapping [num_tokens]: rows past the last token (cu_seqlens_q[batch], or batch in decode
 *   mode) are -1, the padding marker kv_store skips [P2 §5.1].  A position below 0, a logical block past
 *   max_blocks_per_seq, a negative block-table entry, or a slot above INT32_MAX (formed in 64 bits, never
 *   wrapped) also gives -1.
 * Requires: block_size >= 1; batch >= 0; num_tokens >= 0; cu_seqlens_q nondecreasing from 0 (device).
 *   The device arrays hold cu_seqlens_q/k [batch+1], context_lens [batch] and block_tables
 *   [batch, max_blocks_per_seq] entries: their lengths are not visible through these pointers, so a shorter
 *   array is read past (the Python binding checks the lengths).
 */
int kv_slot_mapping(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const int32_t* context_lens,
                    const int32_t* block_tables, int32_t batch, int32_t max_blocks_per_seq,
                    int32_t block_size, int32_t num_tokens, int32_t* slot_mapping, hipStream_t stream);

/*
 * kv_store -- store_kvcache: copy token row i of key and of value to cache slot slot_mapping[i]
 * [P2 §5.1 (the three changes from the scatter skeleton); P3 §3; P1 attention.py walkthrough].
 *
 * key, value: [num_tokens, num_kv_heads, head_dim], token stride key_stride / value_stride (elements).
 * k_cache, v_cache: paged caches with num_slots = num_blocks * block_size slots of D elements (in/out).
 * slot_mapping: [num_tokens].  A slot < 0 (the pages use -1) or >= num_slots is skipped, and bytes of
 *   slots nobody writes are left as they were.  The copy is bit-exact.  Two tokens with the same slot
 *   race (the pages never produce that).
 */
int kv_store(const void* key, int64_t key_stride, const void* value, int64_t value_stride, void* k_cache,
             void* v_cache, int64_t num_slots, const int32_t* slot_mapping, int32_t num_tokens,
             int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype, hipStream_t stream);

/*
 * kv_store_qk_norm_rope -- the steps between the qkv split and the attention call, fused: QK-Norm,
 * RoPE, and the store of k and v [P2 §2 steps 4-6; §4; §5.1; P1 layernorm.py walkthrough].
 *
 * For token i (position positions[i]) and every head: q and k are divided by the root of their mean
 * square over head_dim plus eps and multiplied elementwise by q_norm_weight / k_norm_weight
 * ([head_dim] each, same dtype as q); then element e < head_dim/2 and element e + head_dim/2 of q and of k
 * are rotated by the angle positions[i] * rope_theta^(-2e/head_dim) (the rotate-half rotary embedding);
 * v is not changed.  The rotated k and the v row are written to cache slot slot_mapping[i] exactly as
 * kv_store does (slot < 0 or >= num_slots skips the cache); the normalised, rotated q is written to q_out.
 * q, k, v: [num_tokens, heads, head_dim] with token strides (rows of a merged qkv projection work as
 * they are).  q_out: [num_tokens, num_q_heads, head_dim], contiguous.  head_dim: 16, 32, 64, 128 or 256.
 * Arithmetic in float32 with one rounding to the storage type at the end; the angles are formed in
 * float64 and reduced modulo 2 pi before the float32 sine and cosine.
 */
int kv_store_qk_norm_rope(const void* q, int64_t q_stride, const void* k, int64_t k_stride, const void* v,
                          int64_t v_stride, const int32_t* positions, const void* q_norm_weight,
                          const void* k_norm_weight, float eps, float rope_theta, void* q_out, void* k_cache,
                          void* v_cache, int64_t num_slots, const int32_t* slot_mapping, int32_t num_tokens,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype,
                          hipStream_t stream);

/*
 * attn_prefill_varlen -- varlen attention for a prefill step [P2 §5.3; P3 §4; P1 Q6 §3].
 *
 * Sequence b has query rows [cu_seqlens_q[b], cu_seqlens_q[b+1]) of q (token stride q_stride) and
 * Lk = cu_seqlens_k[b+1]-cu_seqlens_k[b] keys.  Its Lq queries are its last Lq positions: with causal=1
 * query i sees keys 0 .. Lk-Lq+i (bottom-right alignment; a query with no visible key gets zeros); with
 * causal=0 it sees all Lk keys.  out[i] = softmax(softmax_scale * q_i K^T) V over the visible keys.
 *   Contiguous mode (block_tables == NULL): k, v are [num_k_rows, num_kv_heads, head_dim] with token
 *     strides k_stride / v_stride, and sequence b's keys are rows [cu_seqlens_k[b], cu_seqlens_k[b+1]).
 *   Paged mode (block_tables != NULL): k, v are the paged caches (num_k_rows = num_blocks * block_size
 *     slots; k_stride and v_stride are ignored) and key j of sequence b is read from slot
 *     block_tables[b][j / block_size] * block_size + j % block_size -- the prefix-cache branch, where
 *     the new tokens were stored first and are read back with the cached prefix [P2 §5.3].
 * out: [num_q_tokens, num_q_heads, head_dim], contiguous, same dtype as q.
 * max_seqlen_q must be >= every Lq (rows beyond it are not computed); max_seqlen_k is accepted for
 *   signature parity with the pages' call and only checked to be >= 0.
 * workspace: NULL, or device memory of at least attn_prefill_workspace_bytes(...) bytes (contents on
 *   entry do not matter).  With it the bf16 head_dim-128 kernels run a one-work-group planner.  For GQA
 *   groups of 2 it cuts every query tile whose chain of key tiles is longer than the work each resident
 *   work-group gets into pieces of about that length, lists the pieces longest first, and a second kernel
 *   merges the pieces' partial softmax states by the exact online-softmax rescaling [P2 §5.2]; when no tile
 *   is that long it keeps the grid order.  For other groups it lists the query tiles longest first (long
 *   cached prefixes, non-causal rows), and for causal attention over a step's own tokens it is not used.
 *   Without it the tiles are launched latest-first.  Results do not depend on the order; a split tile
 *   differs from an unsplit one only by the rounding of its sums.
 * Unspecified (but in-bounds) results: query rows past num_q_tokens are skipped; key rows past
 *   num_k_rows and block-table entries outside [0, num_blocks) give unspecified values without any
 *   out-of-bounds access.
 */
int attn_prefill_varlen(const void* q, int64_t q_stride, const void* k, int64_t k_stride, const void* v,
                        int64_t v_stride, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t batch, int32_t num_q_tokens,
                        int64_t num_k_rows, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        float softmax_scale, int32_t causal, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, int32_t block_size, void* out, void* workspace,
                        size_t workspace_bytes, pkv_dtype dtype, hipStream_t stream);

/*
 * attn_prefill_workspace_bytes -- bytes of device workspace attn_prefill_varlen can use for these sizes
 * (0: it takes none): a header, one 32-byte entry per possible query tile or piece, and room for the
 * partial states of split query tiles -- 2 * (W / num_kv_heads + 1) states of 68 KiB per kv head, W the
 * work-groups the current device holds at once (about 107 MB on a 256-CU MI355X).  Sized for the device
 * current at the call; a smaller workspace is refused with -3.
 */
size_t attn_prefill_workspace_bytes(int32_t batch, int32_t num_q_tokens, int32_t max_seqlen_q, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype);

/*
 * attn_decode_workspace_bytes -- bytes of device workspace attn_decode_paged needs for these sizes
 * (0 if none, and 0 for sizes the call refuses: batch or num_q_heads above 65535, contexts beyond 2^31
 * tokens, invalid head counts or dtype).  The split of long contexts into independently reduced pieces
 * depends only on these arguments, so the same workspace serves every call with the same sizes.
 */
size_t attn_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_blocks_per_seq, int32_t block_size, pkv_dtype dtype);

/*
 * attn_decode_paged -- single-token decode over the paged cache [P2 §5.3 decode call; P3 §4 point 2].
 *
 * q: [batch, num_q_heads, head_dim] with token stride q_stride (the pages' [batch, 1, heads, dim] with
 *   the unit axis dropped).  Sequence b attends over its context_lens[b] cached keys, the newest one
 *   included (store it first) [P3 §4 note]; key j is at slot block_tables[b][j / block_size] *
 *   block_size + j % block_size.  context_lens[b] <= 0 gives a zero output row (padding entries).
 * k_cache, v_cache: [num_blocks, block_size, num_kv_heads, head_dim].
 * out: [batch, num_q_heads, head_dim], contiguous.
 * workspace: device memory of at least attn_decode_workspace_bytes(...) bytes (may be NULL when that is
 *   0); its contents on entry do not matter and are overwritten.
 * Unspecified (but in-bounds) results: context_lens above max_blocks_per_seq * block_size are clamped to
 *   it; block-table entries outside [0, num_blocks) are treated as masked keys.
 */
int attn_decode_paged(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                      int32_t num_blocks, const int32_t* context_lens, const int32_t* block_tables,
                      int32_t batch, int32_t max_blocks_per_seq, int32_t block_size, int32_t num_q_heads,
                      int32_t num_kv_heads, int32_t head_dim, float softmax_scale, void* out,
                      void* workspace, size_t workspace_bytes, pkv_dtype dtype, hipStream_t stream);

/*
 * attn_decode_paged_store -- the decode step's store and its attention in one call: store_kvcache of each
 * row's new token [P2 §5.1; P3 §3], then attn_decode_paged over the cache that includes it [P2 §5.3; P3 §4
 * note on the order], with the slot computed from the block table [P3 §9 exercise C].
 *
 * Results equal kv_slot_mapping(context_lens mode) + kv_store + attn_decode_paged on the same arguments, bit
 * for bit (output and cache).  Row b's new token sits at position context_lens[b] - 1; its K and V rows
 * (k_new, v_new: [batch, num_kv_heads, head_dim], token strides k_new_stride / v_new_stride in elements) are
 * written to slot block_tables[b][p / block_size] * block_size + p % block_size and attended as key p.  Rows
 * with context_lens[b] <= 0, a position past the table, or a block-table entry outside [0, num_blocks) write
 * nothing (padding rows give a zero output).  With bf16 and head_dim 128 the store happens inside the decode
 * kernel (the new rows are read once, from k_new / v_new, and written from registers); other shapes launch a
 * store kernel, then the decode.
 * slot_mapping_out: NULL, or [batch] int32 receiving the same slots as kv_slot_mapping (-1: none).
 * Other arguments, workspace (attn_decode_workspace_bytes) and errors: as attn_decode_paged.  The caches must
 * not overlap k_new / v_new.  Limits: num_blocks * block_size < 2^31.
 */
int attn_decode_paged_store(const void* q, int64_t q_stride, const void* k_new, int64_t k_new_stride,
                            const void* v_new, int64_t v_new_stride, void* k_cache, void* v_cache,
                            int32_t num_blocks, const int32_t* context_lens, const int32_t* block_tables,
                            int32_t batch, int32_t max_blocks_per_seq, int32_t block_size, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, float softmax_scale, void* out,
                            int32_t* slot_mapping_out, void* workspace, size_t workspace_bytes, pkv_dtype dtype,
                            hipStream_t stream);

/*
 * attn_decode_paged_store_noalloc -- attn_decode_paged_store for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): no workspace
 * argument; the workspace lives in a static device array of 32 MiB inside the library (one per GPU, held
 * from the first call on that GPU until the process ends).  Nothing is allocated: no hipMalloc, no hipFree.
 *
 * Arguments, results (bit for bit) and errors: as attn_decode_paged_store without workspace /
 * workspace_bytes.  The caller still provides every input and output.  Arguments are checked first, as in
 * attn_decode_paged_store; then a call whose workspace (attn_decode_workspace_bytes) exceeds 32 MiB returns
 * PKV_ERR_WORKSPACE before anything is enqueued (batch
 * 64 with 16 query heads needs about 9 MiB; up to about 3000 rows of 16 query heads fit).  Every call on one GPU
 * shares its array, whose contents after a call are left as they are: calls that may overlap on one GPU
 * (different streams without ordering between them, several host threads) race on it and must be
 * serialised by the caller; calls on one stream are ordered and safe.
 */
int attn_decode_paged_store_noalloc(const void* q, int64_t q_stride, const void* k_new, int64_t k_new_stride,
                                    const void* v_new, int64_t v_new_stride, void* k_cache, void* v_cache,
                                    int32_t num_blocks, const int32_t* context_lens, const int32_t* block_tables,
                                    int32_t batch, int32_t max_blocks_per_seq, int32_t block_size,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    float softmax_scale, void* out, int32_t* slot_mapping_out, pkv_dtype dtype,
                                    hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* PAGEDKV_H */
