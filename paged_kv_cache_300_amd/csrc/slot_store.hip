// slot_mapping construction and the store_kvcache scatter on gfx950.
//
// Scatter [P2 §5.1; P3 §3]: token i's K row and V row (D = num_kv_heads * head_dim elements each) are
// copied to slot slot_mapping[i] of the paged caches; a negative slot is a padding token and writes nothing.
// The pages launch one program per token; here one 64-lane wave moves 1 KiB of a row per instruction
// (16 B per lane), rows are addressed with 64-bit offsets (slot * D * 2 bytes passes 2^31 in large caches),
// and a token's work is spread over as many waves as its row needs so that small batches still fill the chip.
#include "common.h"
#include "launch.h"

namespace pkv {

// Slot of position p through one block-table row, or -1 when there is none: p < 0, a logical block past the
// row, a negative entry, or a slot that an int32 slot_mapping cannot hold (the product is formed in 64 bits,
// so a large block id never wraps into a small slot).
__device__ __forceinline__ int32_t slot_of_position(const int32_t* bt_row, int max_blocks, int block_size, int p) {
  if (p < 0) return -1;
  const int i = p / block_size;
  if (i >= max_blocks) return -1;
  const int blk = bt_row[i];
  if (blk < 0) return -1;
  const int64_t slot = int64_t(blk) * block_size + p % block_size;
  return slot <= int64_t(INT32_MAX) ? int32_t(slot) : -1;
}

// Prefill: token t belongs to the sequence b with cu_q[b] <= t < cu_q[b+1] (binary search); it sits at
// position Lk - Lq + (t - cu_q[b]) [P2 §5.3 prefix branch; P3 §7 chunked pass].
__global__ void slot_mapping_prefill_kernel(const int32_t* __restrict__ cu_q, const int32_t* __restrict__ cu_k,
                                            const int32_t* __restrict__ bt, int batch, int max_blocks,
                                            int block_size, int num_tokens, int32_t* __restrict__ out) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= num_tokens) return;
  int32_t slot = -1;
  if (batch > 0 && t >= cu_q[0] && t < cu_q[batch]) {
    int lo = 0, hi = batch;  // cu_q[lo] <= t < cu_q[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (cu_q[mid] <= t) lo = mid; else hi = mid;
    }
    const int lq = cu_q[lo + 1] - cu_q[lo];
    const int lk = cu_k ? cu_k[lo + 1] - cu_k[lo] : lq;
    slot = slot_of_position(bt + int64_t(lo) * max_blocks, max_blocks, block_size, lk - lq + (t - cu_q[lo]));
  }
  out[t] = slot;
}

// Decode: row b writes position context_lens[b] - 1 [P3 §9 exercise C].
__global__ void slot_mapping_decode_kernel(const int32_t* __restrict__ ctx, const int32_t* __restrict__ bt,
                                           int batch, int max_blocks, int block_size, int num_tokens,
                                           int32_t* __restrict__ out) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= num_tokens) return;
  out[t] = t < batch ? slot_of_position(bt + int64_t(t) * max_blocks, max_blocks, block_size, ctx[t] - 1) : -1;
}

// Decode store of any shape: row b's new token (position context_lens[b] - 1) to its slot, one work-group per
// row copying the K and V rows in 2-byte units; the slot is also written to slot_out when given.  A position
// with no usable block (outside the table, a negative entry, a block past the cache) writes nothing.
__global__ void __launch_bounds__(256) decode_store_kernel(DecodeStoreArgs s, const int32_t* __restrict__ ctx,
                                                           const int32_t* __restrict__ bt, int max_blocks,
                                                           int block_size, int64_t num_slots, uint16_t* k_cache,
                                                           uint16_t* v_cache, int row_units, int elem_units) {
  const int b = blockIdx.x;
  const int32_t slot = slot_of_position(bt + int64_t(b) * max_blocks, max_blocks, block_size, ctx[b] - 1);
  if (threadIdx.x == 0 && s.slot_out) s.slot_out[b] = slot;
  if (slot < 0 || slot >= num_slots) return;
  const uint16_t* kr = static_cast<const uint16_t*>(s.k_new) + int64_t(b) * s.k_new_stride * elem_units;
  const uint16_t* vr = static_cast<const uint16_t*>(s.v_new) + int64_t(b) * s.v_new_stride * elem_units;
  uint16_t* kd = k_cache + int64_t(slot) * row_units;
  uint16_t* vd = v_cache + int64_t(slot) * row_units;
  for (int i = threadIdx.x; i < row_units; i += blockDim.x) {
    kd[i] = kr[i];
    vd[i] = vr[i];
  }
}

hipError_t launch_decode_store(const DecodeStoreArgs& s, const int32_t* context_lens, const int32_t* block_tables,
                               int batch, int max_blocks, int block_size, int num_blocks, void* k_cache,
                               void* v_cache, int row_elems, int elem_bytes, hipStream_t stream) {
  if (batch == 0) return hipSuccess;
  const int elem_units = elem_bytes / 2;
  hipLaunchKernelGGL(decode_store_kernel, dim3(batch), dim3(256), 0, stream, s, context_lens, block_tables,
                     max_blocks, block_size, int64_t(num_blocks) * block_size, static_cast<uint16_t*>(k_cache),
                     static_cast<uint16_t*>(v_cache), row_elems * elem_units, elem_units);
  return hipGetLastError();
}

hipError_t launch_slot_mapping(const int32_t* cu_q, const int32_t* cu_k, const int32_t* ctx_lens,
                               const int32_t* block_tables, int batch, int max_blocks, int block_size,
                               int num_tokens, int32_t* slot_mapping, hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  const int threads = 256;
  const int blocks = (num_tokens + threads - 1) / threads;
  if (ctx_lens)
    hipLaunchKernelGGL(slot_mapping_decode_kernel, dim3(blocks), dim3(threads), 0, stream, ctx_lens, block_tables,
                       batch, max_blocks, block_size, num_tokens, slot_mapping);
  else
    hipLaunchKernelGGL(slot_mapping_prefill_kernel, dim3(blocks), dim3(threads), 0, stream, cu_q, cu_k,
                       block_tables, batch, max_blocks, block_size, num_tokens, slot_mapping);
  return hipGetLastError();
}

// Vector path: a row of C 16-byte chunks is copied by C / VPT lanes, lane r moving chunks r + (C / VPT) j,
// j < VPT, of the token's K row and of its V row (each load instruction of a wave covers contiguous
// bytes).  All loads, the slot included, are issued before the slot is tested, so a token costs one memory
// round trip before its stores.  The cache rows are written with non-temporal stores (streamed to memory,
// not kept in the caches): measured on the 16384-token sweep, 4.48 -> 5.68 TB/s.  Every row start and stride
// is 16-byte aligned (checked by the launcher).
template <int VPT>
__global__ void __launch_bounds__(256) kv_store_vec16_kernel(
    const u32x4* __restrict__ key, int64_t key_stride16, const u32x4* __restrict__ value, int64_t value_stride16,
    u32x4* __restrict__ k_cache, u32x4* __restrict__ v_cache, int64_t num_slots,
    const int32_t* __restrict__ slot_mapping, int num_tokens, int chunks_per_row) {
  const int lanes_per_row = chunks_per_row / VPT;
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  const int64_t tok = gid / lanes_per_row;
  if (tok >= num_tokens) return;
  const int r = int(gid - tok * lanes_per_row);
  const u32x4* kr = key + tok * key_stride16 + r;
  const u32x4* vr = value + tok * value_stride16 + r;
  u32x4 kx[VPT], vx[VPT];
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    kx[j] = kr[j * lanes_per_row];
    vx[j] = vr[j * lanes_per_row];
  }
  const int64_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;  // padding token (-1) or out-of-range slot: nothing is written
  u32x4* kd = k_cache + slot * chunks_per_row + r;
  u32x4* vd = v_cache + slot * chunks_per_row + r;
#pragma unroll
  for (int j = 0; j < VPT; ++j) {
    __builtin_nontemporal_store(kx[j], &kd[j * lanes_per_row]);
    __builtin_nontemporal_store(vx[j], &vd[j * lanes_per_row]);
  }
}

// Element path for rows that are not 16-byte aligned.
template <typename T>
__global__ void __launch_bounds__(256) kv_store_elem_kernel(
    const T* __restrict__ key, int64_t key_stride, const T* __restrict__ value, int64_t value_stride,
    T* __restrict__ k_cache, T* __restrict__ v_cache, int64_t num_slots, const int32_t* __restrict__ slot_mapping,
    int64_t total, int row_elems) {
  const int64_t gid = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  if (gid >= total) return;
  const int64_t tok = gid / row_elems;
  const int e = int(gid - tok * row_elems);
  const int64_t slot = slot_mapping[tok];
  if (slot < 0 || slot >= num_slots) return;
  k_cache[slot * row_elems + e] = key[tok * key_stride + e];
  v_cache[slot * row_elems + e] = value[tok * value_stride + e];
}

hipError_t launch_kv_store(const void* key, int64_t key_stride, const void* value, int64_t value_stride,
                           void* k_cache, void* v_cache, int64_t num_slots, const int32_t* slot_mapping,
                           int num_tokens, int row_elems, int elem_bytes, hipStream_t stream) {
  if (num_tokens == 0 || row_elems == 0) return hipSuccess;
  const int threads = 256;
  const int64_t row_bytes = int64_t(row_elems) * elem_bytes;
  auto aligned16 = [](const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; };
  const bool vec = row_bytes % 16 == 0 && (key_stride * elem_bytes) % 16 == 0 &&
                   (value_stride * elem_bytes) % 16 == 0 && aligned16(key) && aligned16(value) &&
                   aligned16(k_cache) && aligned16(v_cache);
  if (vec) {
    const int chunks = int(row_bytes / 16);
    const int vpt = chunks % 4 == 0 ? 4 : (chunks % 2 == 0 ? 2 : 1);
    const int64_t total = int64_t(num_tokens) * (chunks / vpt);
    const int64_t blocks = (total + threads - 1) / threads;
    auto* kp = static_cast<const u32x4*>(key);
    auto* vp = static_cast<const u32x4*>(value);
    auto* kc = static_cast<u32x4*>(k_cache);
    auto* vc = static_cast<u32x4*>(v_cache);
    const int64_t ks = key_stride * elem_bytes / 16, vs = value_stride * elem_bytes / 16;
    if (vpt == 4)
      hipLaunchKernelGGL(kv_store_vec16_kernel<4>, dim3(unsigned(blocks)), dim3(threads), 0, stream, kp, ks, vp, vs,
                         kc, vc, num_slots, slot_mapping, num_tokens, chunks);
    else if (vpt == 2)
      hipLaunchKernelGGL(kv_store_vec16_kernel<2>, dim3(unsigned(blocks)), dim3(threads), 0, stream, kp, ks, vp, vs,
                         kc, vc, num_slots, slot_mapping, num_tokens, chunks);
    else
      hipLaunchKernelGGL(kv_store_vec16_kernel<1>, dim3(unsigned(blocks)), dim3(threads), 0, stream, kp, ks, vp, vs,
                         kc, vc, num_slots, slot_mapping, num_tokens, chunks);
  } else {
    const int64_t total = int64_t(num_tokens) * row_elems;
    const int64_t blocks = (total + threads - 1) / threads;
    if (elem_bytes == 2)
      hipLaunchKernelGGL(kv_store_elem_kernel<uint16_t>, dim3(unsigned(blocks)), dim3(threads), 0, stream,
                         static_cast<const uint16_t*>(key), key_stride, static_cast<const uint16_t*>(value),
                         value_stride, static_cast<uint16_t*>(k_cache), static_cast<uint16_t*>(v_cache), num_slots,
                         slot_mapping, total, row_elems);
    else
      hipLaunchKernelGGL(kv_store_elem_kernel<uint32_t>, dim3(unsigned(blocks)), dim3(threads), 0, stream,
                         static_cast<const uint32_t*>(key), key_stride, static_cast<const uint32_t*>(value),
                         value_stride, static_cast<uint32_t*>(k_cache), static_cast<uint32_t*>(v_cache), num_slots,
                         slot_mapping, total, row_elems);
  }
  return hipGetLastError();
}

}  // namespace pkv
