// Host-side launchers of the gfx950 kernels; arguments are already validated by the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pkv {

hipError_t launch_slot_mapping(const int32_t* cu_q, const int32_t* cu_k, const int32_t* ctx_lens,
                               const int32_t* block_tables, int batch, int max_blocks, int block_size,
                               int num_tokens, int32_t* slot_mapping, hipStream_t stream);

// elem_bytes is 2 (bf16) or 4 (f32); strides in elements.
hipError_t launch_kv_store(const void* key, int64_t key_stride, const void* value, int64_t value_stride,
                           void* k_cache, void* v_cache, int64_t num_slots, const int32_t* slot_mapping,
                           int num_tokens, int row_elems, int elem_bytes, hipStream_t stream);

// QK-Norm + RoPE of q and k, then the store of k and v (head_dim 16 .. 256, powers of two).
bool qknorm_rope_supported(int head_dim);
hipError_t launch_qknorm_rope_store(const void* q, int64_t q_stride, const void* k, int64_t k_stride,
                                    const void* v, int64_t v_stride, const int32_t* positions,
                                    const void* q_norm_weight, const void* k_norm_weight, float eps,
                                    float rope_theta, void* q_out, void* k_cache, void* v_cache,
                                    int64_t num_slots, const int32_t* slot_mapping, int num_tokens,
                                    int num_q_heads, int num_kv_heads, int head_dim, bool bf16,
                                    hipStream_t stream);

// Any dtype, head_dim <= 256, any block size; prefill (cu_q != NULL) or decode (ctx_lens != NULL).
struct AttnArgs {
  const void* q; int64_t q_stride;
  const void* k; int64_t k_stride;
  const void* v; int64_t v_stride;
  const int32_t* cu_q; const int32_t* cu_k; const int32_t* ctx_lens;
  const int32_t* block_tables; int max_blocks; int block_size;
  int64_t num_k_rows;  // contiguous rows, or slots of the paged cache
  int num_blocks;      // paged mode
  int batch; int max_seqlen_q; int max_seqlen_k; int num_q_tokens;
  int num_q_heads; int num_kv_heads; int head_dim;
  float scale; int causal;
  void* out;
};

hipError_t launch_attn_generic(const AttnArgs& a, bool bf16, hipStream_t stream);

// bf16, head_dim 128 decode with split-KV.
struct DecodePlan {
  int split_tokens;  // keys per work-group (multiple of 128)
  int max_splits;    // splits per sequence at the longest context
  size_t workspace_bytes;
};
bool decode_fast_supported(int head_dim, int group, bool bf16);
DecodePlan decode_plan(int batch, int num_q_heads, int num_kv_heads, int max_ctx);
// The step's new K/V rows for the fused store + decode (token strides in elements; slot_out may be NULL).
struct DecodeStoreArgs {
  const void* k_new; int64_t k_new_stride;
  const void* v_new; int64_t v_new_stride;
  int32_t* slot_out;
};
// fused == NULL: decode over the cache as it is; else the new token of each row is stored and attended too.
hipError_t launch_decode_bf16(const AttnArgs& a, const DecodePlan& plan, void* workspace, hipStream_t stream,
                              const DecodeStoreArgs* fused = nullptr);
// The decode workspace of attn_decode_paged_store_noalloc: a static device array of kDecodeScratchBytes, its
// address on the current device (looked up on the first call on each device).
constexpr size_t kDecodeScratchBytes = size_t(32) << 20;
hipError_t decode_static_scratch(void** ptr);
// Any dtype and shape: the new token of each decode row to its slot (context_lens[b] - 1 through the block
// table), optionally writing slot_mapping; rows with no slot write nothing.
hipError_t launch_decode_store(const DecodeStoreArgs& s, const int32_t* context_lens, const int32_t* block_tables,
                               int batch, int max_blocks, int block_size, int num_blocks, void* k_cache,
                               void* v_cache, int row_elems, int elem_bytes, hipStream_t stream);

// bf16, head_dim 128 prefill on MFMA.
bool prefill_fast_supported(int head_dim, int group, bool bf16);
// Contiguous K/V rows: a 64-row tile must span < 2^31 bytes.
bool prefill_fast_strides_ok(int64_t k_stride, int64_t v_stride);
// Workspace of the planners: the longest-first list, and for the 32x32 kernel the pieces of split query tiles and
// their partial states (0: not available for these sizes).
size_t prefill_workspace_bytes(int batch, int num_q_tokens, int max_seqlen_q, int num_kv_heads);
// Whether the longest-first order can beat the grid's launch order for this call (16x16 kernels).
bool prefill_wants_order(const AttnArgs& a);
// Whether a workspace can help this call: the longest-first order, or the splitting of long query tiles.
bool prefill_wants_plan(const AttnArgs& a);
// workspace == NULL: grid order; else the planner orders the query tiles longest first.
hipError_t launch_prefill_bf16(const AttnArgs& a, void* workspace, size_t workspace_bytes, hipStream_t stream);

}  // namespace pkv
