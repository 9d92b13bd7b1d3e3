// QK-Norm + RoPE fused into the KV store, on gfx950.
//
// What it computes [P2 §2 steps 4-6; §4; §5.1; P1 layernorm.py walkthrough]: for each new token and each
// head, q and k are RMS-normalised over head_dim and scaled by their learned weights, then rotated by the
// token's position -- element i paired with i + head_dim/2 at angle position * theta^(-2i/head_dim) --
// and k together with the untouched v is written to the paged cache at the token's slot (slot < 0 skips
// the cache, as the store does); the normalised, rotated q goes to q_out for the attention call.
//
// How: one work-group per token, one wave per head row at a time (q rows, then k rows, then v rows).  A lane
// holds elements l + 64 j of the row; the rotation partner of an element is in the same lane for head_dim
// >= 128 and in lane l ^ head_dim/2 otherwise.  The mean square is a wave reduction; everything is float32
// with one rounding to the storage type at the end.  The rotation angles are formed in float64 and reduced
// modulo 2 pi before the float32 sine and cosine, so large positions keep their accuracy; each wave forms
// them once per token and reuses them for every head.  The pass reads each q, k, v row once and writes each
// output row once: it is bound by HBM bandwidth.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace pkv {
namespace {

struct QkrArgs {
  const void* q; int64_t q_stride;
  const void* k; int64_t k_stride;
  const void* v; int64_t v_stride;
  const int32_t* positions;
  const void* wq; const void* wk;
  float eps; double log2_theta;
  void* q_out; void* k_cache; void* v_cache;
  int64_t num_slots;
  const int32_t* slot_mapping;
  int num_tokens, num_q_heads, num_kv_heads;
};

__device__ __forceinline__ float lane_sum(float x) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) x += shfl_xor_f32(x, o);
  return x;
}

template <typename T, int HD>
__global__ void __launch_bounds__(256) qknorm_rope_store_kernel(QkrArgs a) {
  constexpr int E = HD >= 64 ? HD / 64 : 1;  // elements per lane
  constexpr int ACTIVE = HD >= 64 ? 64 : HD; // lanes holding elements
  constexpr bool IN_LANE = HD >= 128;        // rotation partner in the same lane
  const int tok = blockIdx.x;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, waves = blockDim.x >> 6;
  const bool active = lane < ACTIVE;
  const int64_t slot = a.slot_mapping[tok];
  const bool store = slot >= 0 && slot < a.num_slots;
  const double pos = double(a.positions[tok]);

  // cos / sin for this lane's elements: element e uses frequency index e mod (HD / 2).
  float cs[E], sn[E];
#pragma unroll
  for (int j = 0; j < E; ++j) {
    const int e = lane + 64 * j;
    const int fi = e % (HD / 2);
    const double ang = pos * exp2(-(2.0 * fi / HD) * a.log2_theta);
    const double two_pi = 6.283185307179586476925287;
    const double r = ang - two_pi * rint(ang / two_pi);
    sincosf(float(r), &sn[j], &cs[j]);
  }

  const int rows = a.num_q_heads + 2 * a.num_kv_heads;
  for (int row = wave; row < rows; row += waves) {
    const bool is_q = row < a.num_q_heads;
    const bool is_k = !is_q && row < a.num_q_heads + a.num_kv_heads;
    const int h = is_q ? row : (is_k ? row - a.num_q_heads : row - a.num_q_heads - a.num_kv_heads);
    const T* src = is_q ? static_cast<const T*>(a.q) + int64_t(tok) * a.q_stride
                        : (is_k ? static_cast<const T*>(a.k) + int64_t(tok) * a.k_stride
                                : static_cast<const T*>(a.v) + int64_t(tok) * a.v_stride);
    src += int64_t(h) * HD;
    float x[E];
#pragma unroll
    for (int j = 0; j < E; ++j) x[j] = active ? Elem<T>::load(src + lane + 64 * j) : 0.f;

    if (!is_q && !is_k) {  // v: copied to the cache unchanged
      if (store && active) {
        T* dst = static_cast<T*>(a.v_cache) + (slot * a.num_kv_heads + h) * HD;
#pragma unroll
        for (int j = 0; j < E; ++j) dst[lane + 64 * j] = src[lane + 64 * j];
      }
      continue;
    }
    // RMSNorm over the row, then the weight.
    float ss = 0.f;
#pragma unroll
    for (int j = 0; j < E; ++j) ss = fmaf(x[j], x[j], ss);
    const float inv = 1.f / sqrtf(lane_sum(ss) / float(HD) + a.eps);
    const T* w = static_cast<const T*>(is_q ? a.wq : a.wk);
#pragma unroll
    for (int j = 0; j < E; ++j) x[j] = active ? x[j] * inv * Elem<T>::load(w + lane + 64 * j) : 0.f;
    // Rotation of the pairs (e, e + HD / 2).
    float y[E];
    if constexpr (IN_LANE) {
#pragma unroll
      for (int j = 0; j < E / 2; ++j) {
        const float x1 = x[j], x2 = x[j + E / 2];
        y[j] = x1 * cs[j] - x2 * sn[j];
        y[j + E / 2] = x2 * cs[j + E / 2] + x1 * sn[j + E / 2];
      }
    } else {
      const float other = shfl_xor_f32(x[0], HD / 2);
      const bool first = (lane & (HD / 2)) == 0;
      y[0] = first ? x[0] * cs[0] - other * sn[0] : x[0] * cs[0] + other * sn[0];
    }
    if (active) {
      T* dst = is_q ? static_cast<T*>(a.q_out) + (int64_t(tok) * a.num_q_heads + h) * HD
                    : static_cast<T*>(a.k_cache) + (slot * a.num_kv_heads + h) * HD;
      if (is_q || store) {
#pragma unroll
        for (int j = 0; j < E; ++j) Elem<T>::store(dst + lane + 64 * j, y[j]);
      }
    }
  }
}

template <typename T>
hipError_t launch_t(const QkrArgs& a, int head_dim, hipStream_t stream) {
  const dim3 grid(a.num_tokens), block(256);
  switch (head_dim) {
    case 16: hipLaunchKernelGGL((qknorm_rope_store_kernel<T, 16>), grid, block, 0, stream, a); break;
    case 32: hipLaunchKernelGGL((qknorm_rope_store_kernel<T, 32>), grid, block, 0, stream, a); break;
    case 64: hipLaunchKernelGGL((qknorm_rope_store_kernel<T, 64>), grid, block, 0, stream, a); break;
    case 128: hipLaunchKernelGGL((qknorm_rope_store_kernel<T, 128>), grid, block, 0, stream, a); break;
    case 256: hipLaunchKernelGGL((qknorm_rope_store_kernel<T, 256>), grid, block, 0, stream, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool qknorm_rope_supported(int head_dim) {
  return head_dim == 16 || head_dim == 32 || head_dim == 64 || head_dim == 128 || head_dim == 256;
}

hipError_t launch_qknorm_rope_store(const void* q, int64_t q_stride, const void* k, int64_t k_stride,
                                    const void* v, int64_t v_stride, const int32_t* positions,
                                    const void* q_norm_weight, const void* k_norm_weight, float eps,
                                    float rope_theta, void* q_out, void* k_cache, void* v_cache,
                                    int64_t num_slots, const int32_t* slot_mapping, int num_tokens,
                                    int num_q_heads, int num_kv_heads, int head_dim, bool bf16,
                                    hipStream_t stream) {
  if (num_tokens == 0) return hipSuccess;
  QkrArgs a;
  a.q = q; a.q_stride = q_stride; a.k = k; a.k_stride = k_stride; a.v = v; a.v_stride = v_stride;
  a.positions = positions; a.wq = q_norm_weight; a.wk = k_norm_weight;
  a.eps = eps; a.log2_theta = log2(double(rope_theta));
  a.q_out = q_out; a.k_cache = k_cache; a.v_cache = v_cache; a.num_slots = num_slots;
  a.slot_mapping = slot_mapping; a.num_tokens = num_tokens; a.num_q_heads = num_q_heads;
  a.num_kv_heads = num_kv_heads;
  return bf16 ? launch_t<uint16_t>(a, head_dim, stream) : launch_t<float>(a, head_dim, stream);
}

}  // namespace pkv
