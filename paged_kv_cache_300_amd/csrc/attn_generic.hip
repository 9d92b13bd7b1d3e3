// Generic attention kernel: any element type (f32 / bf16), any head_dim <= 256, any block size, contiguous or
// paged K/V, prefill or decode.  It serves the float32 path and shapes the tuned bf16 kernels do not cover.
//
// One 64-lane wave per (query row, query head).  Keys are visited in chunks of 64, one key per lane for
// the scores, then one head-dim element per lane for the weighted sum of V, with the running maximum,
// normaliser and unnormalised output kept as in the online softmax [P2 §5.2 ②]; the output is divided by
// the normaliser once at the end.  Which keys a row sees, and where they live, follow the varlen and paged
// calls [P2 §5.3; P3 §4]: bottom-right causal alignment, block-table gather in paged mode.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace pkv {

template <typename T>
__global__ void __launch_bounds__(64) attn_generic_kernel(AttnArgs a) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int lane = threadIdx.x;
  const bool paged = a.block_tables != nullptr;
  int lq, lk, qrow;
  int64_t krow0 = 0;
  if (a.ctx_lens) {  // decode: one query per sequence at position context_len - 1
    lq = 1;
    lk = a.ctx_lens[b];
    qrow = b;
  } else {
    const int q0 = a.cu_q[b];
    lq = a.cu_q[b + 1] - q0;
    lk = a.cu_k[b + 1] - a.cu_k[b];
    krow0 = a.cu_k[b];
    qrow = q0 + i;
  }
  if (i >= lq || qrow < 0 || qrow >= a.num_q_tokens) return;
  const int pos = lk - lq + i;  // absolute position of this query (bottom-right alignment)
  lk = max(lk, 0);
  if (paged) lk = min(lk, a.max_blocks * a.block_size);
  const int nvis = a.causal ? min(lk, pos + 1) : lk;
  const int group = a.num_q_heads / a.num_kv_heads;
  const int kvh = h / group;
  const int hd = a.head_dim;
  const int64_t slot_elems = int64_t(a.num_kv_heads) * hd;
  const T* q = static_cast<const T*>(a.q) + int64_t(qrow) * a.q_stride + int64_t(h) * hd;
  const T* kbase = static_cast<const T*>(a.k) + int64_t(kvh) * hd;
  const T* vbase = static_cast<const T*>(a.v) + int64_t(kvh) * hd;
  const int32_t* bt_row = paged ? a.block_tables + int64_t(b) * a.max_blocks : nullptr;

  __shared__ float sq[256];
  __shared__ float sp[64];
  __shared__ int64_t sv[64];
  for (int d = lane; d < hd; d += 64) sq[d] = Elem<T>::load(q + d);
  __syncthreads();

  float m = -INFINITY, l = 0.f;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int j0 = 0; j0 < nvis; j0 += 64) {
    const int j = j0 + lane;
    int64_t koff = -1, voff = -1;
    if (j < nvis) {
      if (paged) {
        const int64_t slot = paged_slot(bt_row, j, a.block_size, a.num_blocks);
        if (slot >= 0) { koff = slot * slot_elems; voff = koff; }
      } else if (krow0 + j >= 0 && krow0 + j < a.num_k_rows) {
        koff = (krow0 + j) * a.k_stride;
        voff = (krow0 + j) * a.v_stride;
      }
    }
    float s = -INFINITY;
    if (koff >= 0) {
      float dot = 0.f;
      for (int d = 0; d < hd; ++d) dot = fmaf(sq[d], Elem<T>::load(kbase + koff + d), dot);
      s = dot * a.scale;
    }
    const float mn = fmaxf(m, wave_max(s));
    if (mn == -INFINITY) continue;  // nothing visible so far
    const float p = koff >= 0 ? expf(s - mn) : 0.f;
    const float alpha = m == -INFINITY ? 0.f : expf(m - mn);
    l = l * alpha + wave_sum(p);
    m = mn;
    sp[lane] = p;
    sv[lane] = voff;
    __syncthreads();
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] *= alpha;
    const int n = min(64, nvis - j0);
    for (int jj = 0; jj < n; ++jj) {
      const int64_t off = sv[jj];
      if (off < 0) continue;
      const float pj = sp[jj];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d = lane + 64 * r;
        if (d < hd) acc[r] = fmaf(pj, Elem<T>::load(vbase + off + d), acc[r]);
      }
    }
    __syncthreads();
  }
  T* o = static_cast<T*>(a.out) + (int64_t(qrow) * a.num_q_heads + h) * hd;
  const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int d = lane + 64 * r;
    if (d < hd) Elem<T>::store(o + d, acc[r] * inv);
  }
}

hipError_t launch_attn_generic(const AttnArgs& a, bool bf16, hipStream_t stream) {
  if (a.batch == 0) return hipSuccess;
  const int rows = a.ctx_lens ? 1 : a.max_seqlen_q;
  if (rows == 0) return hipSuccess;
  const dim3 grid(rows, a.num_q_heads, a.batch);
  if (bf16)
    hipLaunchKernelGGL(attn_generic_kernel<uint16_t>, grid, dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(attn_generic_kernel<float>, grid, dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace pkv
