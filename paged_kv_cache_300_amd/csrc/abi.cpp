// C ABI of the paged-KV attention path: host-side argument checks, then dispatch to the gfx950 kernels.
// Every check runs before anything is enqueued, so a rejected call has no device side effect.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <string>

#include "pagedkv.h"
#include "launch.h"

namespace {

thread_local std::string g_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_error = buf;
  return code;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return PKV_OK;
  return fail(PKV_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool valid_dtype(pkv_dtype d) { return d == PKV_F32 || d == PKV_BF16; }
int elem_bytes(pkv_dtype d) { return d == PKV_BF16 ? 2 : 4; }

constexpr int kMaxHeadDim = 256;
constexpr int kMaxGridYZ = 65535;

int check_heads(int32_t hq, int32_t hkv, int32_t hd) {
  if (hq < 1 || hkv < 1 || hd < 1) return fail(PKV_ERR_INVALID_ARG, "head counts and head_dim must be >= 1");
  if (hq % hkv != 0)
    return fail(PKV_ERR_INVALID_ARG, "num_q_heads (%d) must be a multiple of num_kv_heads (%d)", hq, hkv);
  if (hd > kMaxHeadDim) return fail(PKV_ERR_UNSUPPORTED, "head_dim %d > %d is not supported", hd, kMaxHeadDim);
  if (hq > kMaxGridYZ) return fail(PKV_ERR_UNSUPPORTED, "num_q_heads %d too large", hq);
  return PKV_OK;
}

// attn_decode_paged and attn_decode_paged_store share their checks and dispatch; fused != NULL also stores each
// row's new token (fast path: inside the decode kernel; other shapes: a store kernel, then the decode).
// static_ws: the workspace is the library's static scratch (looked up only once every check has passed).
int decode_call(const char* name, const void* q, int64_t q_stride, const void* k_cache, const void* v_cache,
                int32_t num_blocks, const int32_t* context_lens, const int32_t* block_tables, int32_t batch,
                int32_t max_blocks_per_seq, int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                int32_t head_dim, float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                pkv_dtype dtype, hipStream_t stream, const pkv::DecodeStoreArgs* fused, bool static_ws = false) {
  if (!valid_dtype(dtype)) return fail(PKV_ERR_INVALID_ARG, "unknown dtype %d", int(dtype));
  if (int rc = check_heads(num_q_heads, num_kv_heads, head_dim)) return rc;
  if (batch < 0 || num_blocks < 0) return fail(PKV_ERR_INVALID_ARG, "batch and num_blocks must be >= 0");
  if (batch > kMaxGridYZ) return fail(PKV_ERR_UNSUPPORTED, "batch %d too large", batch);
  if (block_size < 1 || max_blocks_per_seq < 1)
    return fail(PKV_ERR_INVALID_ARG, "block_size and max_blocks_per_seq must be >= 1");
  if (int64_t(max_blocks_per_seq) * block_size > INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, "contexts beyond 2^31 tokens are not supported");
  if (fused && int64_t(num_blocks) * block_size > INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, "caches beyond 2^31 slots are not supported by the int32 slot_mapping");
  if (!isfinite(softmax_scale)) return fail(PKV_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (q_stride < int64_t(num_q_heads) * head_dim)
    return fail(PKV_ERR_INVALID_ARG, "q_stride must be >= num_q_heads*head_dim");
  const int64_t kv_row = int64_t(num_kv_heads) * head_dim;
  if (fused && (fused->k_new_stride < kv_row || fused->v_new_stride < kv_row))
    return fail(PKV_ERR_INVALID_ARG, "k_new_stride and v_new_stride must be >= num_kv_heads*head_dim");
  if (batch == 0) return PKV_OK;
  if (!q || !k_cache || !v_cache || !context_lens || !block_tables || !out)
    return fail(PKV_ERR_INVALID_ARG, "q, caches, context_lens, block_tables and out must be non-null");
  if (fused && (!fused->k_new || !fused->v_new)) return fail(PKV_ERR_INVALID_ARG, "k_new and v_new must be non-null");
  if (num_blocks < 1) return fail(PKV_ERR_INVALID_ARG, "num_blocks must be >= 1");
  const bool bf16 = dtype == PKV_BF16;
  pkv::AttnArgs a{};
  a.q = q; a.q_stride = q_stride; a.k = k_cache; a.v = v_cache;
  a.k_stride = a.v_stride = kv_row;
  a.cu_q = nullptr; a.cu_k = nullptr; a.ctx_lens = context_lens;
  a.block_tables = block_tables; a.max_blocks = max_blocks_per_seq; a.block_size = block_size;
  a.num_k_rows = int64_t(num_blocks) * block_size; a.num_blocks = num_blocks;
  a.batch = batch; a.max_seqlen_q = 1; a.num_q_tokens = batch;
  a.num_q_heads = num_q_heads; a.num_kv_heads = num_kv_heads; a.head_dim = head_dim;
  a.scale = softmax_scale; a.causal = 1; a.out = out;
  bool fast = pkv::decode_fast_supported(head_dim, num_q_heads / num_kv_heads, bf16) && aligned16(q) &&
              q_stride % 8 == 0 && aligned16(k_cache) && aligned16(v_cache);
  if (fast && fused)
    fast = aligned16(fused->k_new) && aligned16(fused->v_new) && fused->k_new_stride % 8 == 0 &&
           fused->v_new_stride % 8 == 0;
  if (fast) {
    const pkv::DecodePlan plan =
        pkv::decode_plan(batch, num_q_heads, num_kv_heads, max_blocks_per_seq * block_size);
    if (static_ws) {
      if (plan.workspace_bytes > pkv::kDecodeScratchBytes)
        return fail(PKV_ERR_WORKSPACE, "%s: %zu bytes of workspace needed (batch %d, %d query heads), the static "
                    "scratch holds %zu", name, plan.workspace_bytes, batch, num_q_heads, pkv::kDecodeScratchBytes);
      if (const hipError_t e = pkv::decode_static_scratch(&workspace); e != hipSuccess)
        return hip_status(e, name);
      workspace_bytes = pkv::kDecodeScratchBytes;
    }
    if (plan.workspace_bytes > 0 && (!workspace || workspace_bytes < plan.workspace_bytes))
      return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", plan.workspace_bytes,
                  workspace ? workspace_bytes : size_t(0));
    return hip_status(pkv::launch_decode_bf16(a, plan, workspace, stream, fused), name);
  }
  if (fused) {
    const hipError_t e = pkv::launch_decode_store(*fused, context_lens, block_tables, batch, max_blocks_per_seq,
                                                  block_size, num_blocks, const_cast<void*>(k_cache),
                                                  const_cast<void*>(v_cache), int(kv_row), bf16 ? 2 : 4, stream);
    if (e != hipSuccess) return hip_status(e, name);
  }
  return hip_status(pkv::launch_attn_generic(a, bf16, stream), name);
}

}  // namespace

extern "C" {

const char* pkv_last_error(void) { return g_error.c_str(); }

int kv_slot_mapping(const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k, const int32_t* context_lens,
                    const int32_t* block_tables, int32_t batch, int32_t max_blocks_per_seq, int32_t block_size,
                    int32_t num_tokens, int32_t* slot_mapping, hipStream_t stream) {
  g_error.clear();
  if (batch < 0 || num_tokens < 0 || max_blocks_per_seq < 0)
    return fail(PKV_ERR_INVALID_ARG, "batch, max_blocks_per_seq and num_tokens must be >= 0");
  if (block_size < 1) return fail(PKV_ERR_INVALID_ARG, "block_size must be >= 1");
  const bool decode = context_lens != nullptr;
  if (decode && (cu_seqlens_q || cu_seqlens_k))
    return fail(PKV_ERR_INVALID_ARG, "pass either context_lens (decode) or cu_seqlens (prefill), not both");
  if (!decode && !cu_seqlens_q && batch > 0)
    return fail(PKV_ERR_INVALID_ARG, "prefill mode needs cu_seqlens_q");
  if (num_tokens > 0 && !slot_mapping) return fail(PKV_ERR_INVALID_ARG, "slot_mapping is null");
  if (batch > 0 && max_blocks_per_seq > 0 && !block_tables)
    return fail(PKV_ERR_INVALID_ARG, "block_tables is null");
  if (int64_t(max_blocks_per_seq) * block_size > INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, "positions beyond 2^31 are not addressable by int32 slots");
  if (num_tokens == 0) return PKV_OK;
  // A table of width 0 maps every position to -1: pass a width-0 table the kernel never reads.
  return hip_status(pkv::launch_slot_mapping(cu_seqlens_q, cu_seqlens_k, context_lens, block_tables,
                                             max_blocks_per_seq > 0 ? batch : 0, max_blocks_per_seq, block_size,
                                             num_tokens, slot_mapping, stream),
                    "kv_slot_mapping launch");
}

int kv_store(const void* key, int64_t key_stride, const void* value, int64_t value_stride, void* k_cache,
             void* v_cache, int64_t num_slots, const int32_t* slot_mapping, int32_t num_tokens,
             int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype, hipStream_t stream) {
  g_error.clear();
  if (!valid_dtype(dtype)) return fail(PKV_ERR_INVALID_ARG, "unknown dtype %d", int(dtype));
  if (num_tokens < 0 || num_slots < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens and num_slots must be >= 0");
  if (num_kv_heads < 1 || head_dim < 1) return fail(PKV_ERR_INVALID_ARG, "num_kv_heads and head_dim must be >= 1");
  const int64_t row = int64_t(num_kv_heads) * head_dim;
  if (row > (int64_t(1) << 24)) return fail(PKV_ERR_UNSUPPORTED, "row of %lld elements is too large", (long long)row);
  if (key_stride < row || value_stride < row)
    return fail(PKV_ERR_INVALID_ARG, "key_stride/value_stride (%lld/%lld) must be >= num_kv_heads*head_dim (%lld)",
                (long long)key_stride, (long long)value_stride, (long long)row);
  if (num_tokens == 0) return PKV_OK;
  if (!key || !value || !k_cache || !v_cache || !slot_mapping)
    return fail(PKV_ERR_INVALID_ARG, "key, value, k_cache, v_cache and slot_mapping must be non-null");
  if (int64_t(num_tokens) * row / 256 + 1 >= INT32_MAX)
    return fail(PKV_ERR_UNSUPPORTED, "too many elements for one launch");
  return hip_status(pkv::launch_kv_store(key, key_stride, value, value_stride, k_cache, v_cache, num_slots,
                                         slot_mapping, num_tokens, int(row), elem_bytes(dtype), stream),
                    "kv_store launch");
}

int kv_store_qk_norm_rope(const void* q, int64_t q_stride, const void* k, int64_t k_stride, const void* v,
                          int64_t v_stride, const int32_t* positions, const void* q_norm_weight,
                          const void* k_norm_weight, float eps, float rope_theta, void* q_out, void* k_cache,
                          void* v_cache, int64_t num_slots, const int32_t* slot_mapping, int32_t num_tokens,
                          int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype,
                          hipStream_t stream) {
  g_error.clear();
  if (!valid_dtype(dtype)) return fail(PKV_ERR_INVALID_ARG, "unknown dtype %d", int(dtype));
  if (int rc = check_heads(num_q_heads, num_kv_heads, head_dim)) return rc;
  if (!pkv::qknorm_rope_supported(head_dim))
    return fail(PKV_ERR_UNSUPPORTED, "head_dim %d: 16, 32, 64, 128 or 256 are supported", head_dim);
  if (num_tokens < 0 || num_slots < 0) return fail(PKV_ERR_INVALID_ARG, "num_tokens and num_slots must be >= 0");
  if (q_stride < int64_t(num_q_heads) * head_dim || k_stride < int64_t(num_kv_heads) * head_dim ||
      v_stride < int64_t(num_kv_heads) * head_dim)
    return fail(PKV_ERR_INVALID_ARG, "token strides must cover a row of heads * head_dim elements");
  if (!(eps >= 0.f) || !isfinite(eps)) return fail(PKV_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (!(rope_theta > 0.f) || !isfinite(rope_theta)) return fail(PKV_ERR_INVALID_ARG, "rope_theta must be > 0");
  if (num_tokens == 0) return PKV_OK;
  if (!q || !k || !v || !positions || !q_norm_weight || !k_norm_weight || !q_out || !k_cache || !v_cache ||
      !slot_mapping)
    return fail(PKV_ERR_INVALID_ARG, "every pointer must be non-null");
  return hip_status(pkv::launch_qknorm_rope_store(q, q_stride, k, k_stride, v, v_stride, positions, q_norm_weight,
                                                  k_norm_weight, eps, rope_theta, q_out, k_cache, v_cache,
                                                  num_slots, slot_mapping, num_tokens, num_q_heads,
                                                  num_kv_heads, head_dim, dtype == PKV_BF16, stream),
                    "kv_store_qk_norm_rope launch");
}

int attn_prefill_varlen(const void* q, int64_t q_stride, const void* k, int64_t k_stride, const void* v,
                        int64_t v_stride, const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int32_t max_seqlen_q, int32_t max_seqlen_k, int32_t batch, int32_t num_q_tokens,
                        int64_t num_k_rows, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                        float softmax_scale, int32_t causal, const int32_t* block_tables,
                        int32_t max_blocks_per_seq, int32_t block_size, void* out, void* workspace,
                        size_t workspace_bytes, pkv_dtype dtype, hipStream_t stream) {
  g_error.clear();
  if (!valid_dtype(dtype)) return fail(PKV_ERR_INVALID_ARG, "unknown dtype %d", int(dtype));
  if (int rc = check_heads(num_q_heads, num_kv_heads, head_dim)) return rc;
  if (batch < 0 || num_q_tokens < 0 || num_k_rows < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(PKV_ERR_INVALID_ARG, "sizes must be >= 0");
  if (batch > kMaxGridYZ) return fail(PKV_ERR_UNSUPPORTED, "batch %d too large", batch);
  if (causal != 0 && causal != 1) return fail(PKV_ERR_INVALID_ARG, "causal must be 0 or 1");
  if (!isfinite(softmax_scale)) return fail(PKV_ERR_INVALID_ARG, "softmax_scale must be finite");
  if (q_stride < int64_t(num_q_heads) * head_dim)
    return fail(PKV_ERR_INVALID_ARG, "q_stride must be >= num_q_heads*head_dim");
  const bool paged = block_tables != nullptr;
  const int64_t kv_row = int64_t(num_kv_heads) * head_dim;
  int num_blocks = 0;
  if (paged) {
    if (block_size < 1 || max_blocks_per_seq < 1)
      return fail(PKV_ERR_INVALID_ARG, "paged mode needs block_size >= 1 and max_blocks_per_seq >= 1");
    if (num_k_rows % block_size != 0)
      return fail(PKV_ERR_INVALID_ARG, "num_k_rows (cache slots) must be a multiple of block_size");
    if (num_k_rows / block_size > INT32_MAX) return fail(PKV_ERR_UNSUPPORTED, "too many cache blocks");
    if (int64_t(max_blocks_per_seq) * block_size > INT32_MAX)
      return fail(PKV_ERR_UNSUPPORTED, "positions beyond 2^31 are not supported");
    num_blocks = int(num_k_rows / block_size);
    k_stride = v_stride = kv_row;
  } else if (k_stride < kv_row || v_stride < kv_row) {
    return fail(PKV_ERR_INVALID_ARG, "k_stride/v_stride must be >= num_kv_heads*head_dim");
  }
  if (batch == 0 || num_q_tokens == 0 || max_seqlen_q == 0) return PKV_OK;
  if (!q || !k || !v || !cu_seqlens_q || !cu_seqlens_k || !out)
    return fail(PKV_ERR_INVALID_ARG, "q, k, v, cu_seqlens_q, cu_seqlens_k and out must be non-null");
  pkv::AttnArgs a{};
  a.q = q; a.q_stride = q_stride; a.k = k; a.k_stride = k_stride; a.v = v; a.v_stride = v_stride;
  a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k; a.ctx_lens = nullptr;
  a.block_tables = block_tables; a.max_blocks = max_blocks_per_seq; a.block_size = paged ? block_size : 1;
  a.num_k_rows = num_k_rows; a.num_blocks = num_blocks;
  a.batch = batch; a.max_seqlen_q = max_seqlen_q; a.max_seqlen_k = max_seqlen_k; a.num_q_tokens = num_q_tokens;
  a.num_q_heads = num_q_heads; a.num_kv_heads = num_kv_heads; a.head_dim = head_dim;
  a.scale = softmax_scale; a.causal = causal; a.out = out;
  const bool bf16 = dtype == PKV_BF16;
  const bool fast = pkv::prefill_fast_supported(head_dim, num_q_heads / num_kv_heads, bf16) && aligned16(q) &&
                    aligned16(k) && aligned16(v) && aligned16(out) && q_stride % 8 == 0 &&
                    k_stride % 8 == 0 && v_stride % 8 == 0 && pkv::prefill_fast_strides_ok(k_stride, v_stride);
  if (fast) {
    if (workspace) {
      const size_t need = pkv::prefill_workspace_bytes(batch, num_q_tokens, max_seqlen_q, num_kv_heads);
      if (need > 0 && workspace_bytes < need)
        return fail(PKV_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, need);
      if (need == 0 || !pkv::prefill_wants_plan(a)) workspace = nullptr;
    }
    return hip_status(pkv::launch_prefill_bf16(a, workspace, workspace_bytes, stream),
                      "attn_prefill_varlen launch");
  }
  return hip_status(pkv::launch_attn_generic(a, bf16, stream), "attn_prefill_varlen launch");
}

size_t attn_prefill_workspace_bytes(int32_t batch, int32_t num_q_tokens, int32_t max_seqlen_q, int32_t num_q_heads,
                                    int32_t num_kv_heads, int32_t head_dim, pkv_dtype dtype) {
  if (batch <= 0 || num_q_tokens < 0 || max_seqlen_q < 0 || num_q_heads < 1 || num_kv_heads < 1 ||
      num_q_heads % num_kv_heads || dtype != PKV_BF16)
    return 0;
  if (!pkv::prefill_fast_supported(head_dim, num_q_heads / num_kv_heads, true)) return 0;
  return pkv::prefill_workspace_bytes(batch, num_q_tokens, max_seqlen_q, num_kv_heads);
}

size_t attn_decode_workspace_bytes(int32_t batch, int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                   int32_t max_blocks_per_seq, int32_t block_size, pkv_dtype dtype) {
  // Sizes the calls refuse (batch or query heads beyond a grid dimension) need no workspace either.
  if (batch <= 0 || batch > kMaxGridYZ || num_q_heads < 1 || num_q_heads > kMaxGridYZ || num_kv_heads < 1 ||
      num_q_heads % num_kv_heads || max_blocks_per_seq < 1 || block_size < 1 || !valid_dtype(dtype))
    return 0;
  if (!pkv::decode_fast_supported(head_dim, num_q_heads / num_kv_heads, dtype == PKV_BF16)) return 0;
  const int64_t max_ctx = int64_t(max_blocks_per_seq) * block_size;
  if (max_ctx > INT32_MAX) return 0;
  return pkv::decode_plan(batch, num_q_heads, num_kv_heads, int(max_ctx)).workspace_bytes;
}

int attn_decode_paged(const void* q, int64_t q_stride, const void* k_cache, const void* v_cache, int32_t num_blocks,
                      const int32_t* context_lens, const int32_t* block_tables, int32_t batch,
                      int32_t max_blocks_per_seq, int32_t block_size, int32_t num_q_heads, int32_t num_kv_heads,
                      int32_t head_dim, float softmax_scale, void* out, void* workspace, size_t workspace_bytes,
                      pkv_dtype dtype, hipStream_t stream) {
  g_error.clear();
  return decode_call("attn_decode_paged launch", q, q_stride, k_cache, v_cache, num_blocks, context_lens,
                     block_tables, batch, max_blocks_per_seq, block_size, num_q_heads, num_kv_heads, head_dim,
                     softmax_scale, out, workspace, workspace_bytes, dtype, stream, nullptr);
}

int attn_decode_paged_store(const void* q, int64_t q_stride, const void* k_new, int64_t k_new_stride,
                            const void* v_new, int64_t v_new_stride, void* k_cache, void* v_cache, int32_t num_blocks,
                            const int32_t* context_lens, const int32_t* block_tables, int32_t batch,
                            int32_t max_blocks_per_seq, int32_t block_size, int32_t num_q_heads,
                            int32_t num_kv_heads, int32_t head_dim, float softmax_scale, void* out,
                            int32_t* slot_mapping_out, void* workspace, size_t workspace_bytes, pkv_dtype dtype,
                            hipStream_t stream) {
  g_error.clear();
  pkv::DecodeStoreArgs f;
  f.k_new = k_new; f.k_new_stride = k_new_stride; f.v_new = v_new; f.v_new_stride = v_new_stride;
  f.slot_out = slot_mapping_out;
  return decode_call("attn_decode_paged_store launch", q, q_stride, k_cache, v_cache, num_blocks, context_lens,
                     block_tables, batch, max_blocks_per_seq, block_size, num_q_heads, num_kv_heads, head_dim,
                     softmax_scale, out, workspace, workspace_bytes, dtype, stream, &f);
}

int attn_decode_paged_store_noalloc(const void* q, int64_t q_stride, const void* k_new, int64_t k_new_stride,
                                    const void* v_new, int64_t v_new_stride, void* k_cache, void* v_cache,
                                    int32_t num_blocks, const int32_t* context_lens, const int32_t* block_tables,
                                    int32_t batch, int32_t max_blocks_per_seq, int32_t block_size,
                                    int32_t num_q_heads, int32_t num_kv_heads, int32_t head_dim,
                                    float softmax_scale, void* out, int32_t* slot_mapping_out, pkv_dtype dtype,
                                    hipStream_t stream) {
  g_error.clear();
  pkv::DecodeStoreArgs f;
  f.k_new = k_new; f.k_new_stride = k_new_stride; f.v_new = v_new; f.v_new_stride = v_new_stride;
  f.slot_out = slot_mapping_out;
  return decode_call("attn_decode_paged_store_noalloc", q, q_stride, k_cache, v_cache, num_blocks, context_lens,
                     block_tables, batch, max_blocks_per_seq, block_size, num_q_heads, num_kv_heads, head_dim,
                     softmax_scale, out, nullptr, 0, dtype, stream, &f, /*static_ws=*/true);
}

}  // extern "C"
