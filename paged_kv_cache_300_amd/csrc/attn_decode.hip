// Paged single-token decode attention, bf16 storage, head_dim 128, on gfx950.
//
// What it computes [P2 §5.3 decode call; P3 §4]: for every sequence b and query head h,
// o = softmax(scale * q K^T) V over the context_lens[b] keys of b, key j read from slot
// block_tables[b][j / block_size] * block_size + j % block_size of the paged caches, with kv head
// h / (Hq / Hkv) [P2 §3].
//
// How (gfx950 design, not the pages' library call):
//  * Split-KV: a work-group owns one (sequence, kv head, split of `split_tokens` keys) and serves every
//    query head of that kv head's GQA group, so each K/V row is read from HBM once for the whole group.
//    Short and long contexts alike become many equal-sized work-groups, which keeps all 256 CUs busy.
//  * A token's 256-byte K (or V) row for one kv head is read by 8 lanes, 2 x 16 bytes each; a wave reads
//    8 tokens per instruction (8 full 128-byte lines) and 32 tokens per iteration, all loads issued before
//    any arithmetic so 16 KiB per wave are in flight.  The block-table entries a split touches are staged
//    once in LDS.
//  * q.k uses the packed bf16 dot instruction (exact products, float32 sums); the 8 partial sums of a
//    token are combined with three DPP moves inside the 8-lane group.
//  * Each 8-lane group runs its own online softmax (running max m, normaliser l, unnormalised output) over
//    its tokens [P2 §5.2 ②], in base 2 with log2(e) folded into the scale.  At the end the 8 groups of a wave
//    are merged with lane shuffles, the 4 waves through LDS, and splits by a second small kernel -- every
//    merge is the same exact rescaling by exp(m_i - m).
//  * A sequence that fits in one split writes its output directly; longer ones write (m, l, unnormalised
//    output) per split to the workspace for the combine kernel.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace pkv {
namespace {

constexpr int HD = 128;
constexpr int THREADS = 256;  // 4 waves
constexpr int WAVE_TOKENS = 32;
constexpr int WG_TOKENS = 4 * WAVE_TOKENS;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMinusBig = -1e30f;  // finite "no key yet" maximum, so exp2(m_old - m_new) never sees inf - inf

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;

__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

struct DecodeKernelArgs {
  const uint16_t* q;
  int64_t q_stride;
  const uint16_t* kc;
  const uint16_t* vc;
  int num_blocks;
  const int32_t* ctx;
  const int32_t* bt;
  int max_blocks;
  int bs;
  int bs_shift;  // log2(block_size) when it is a power of two, else -1
  int num_q_heads;
  int num_kv_heads;
  float scale_log2;
  int split_tokens;
  int max_splits;
  uint16_t* out;
  float* ws_acc;  // [B][Hq][max_splits][HD]
  float* ws_ml;   // [B][Hq][max_splits][2]
};

template <int G>
__global__ void __launch_bounds__(THREADS) decode_split_kernel(DecodeKernelArgs p) {
  const int split = blockIdx.x, kvh = blockIdx.y, b = blockIdx.z;
  const int ctx = min(p.ctx[b], p.max_blocks * p.bs);
  const int t0 = split * p.split_tokens;
  if (t0 >= ctx) return;  // whole work-group: this split is past the end of the context
  const int t1 = min(ctx, t0 + p.split_tokens);
  const int nsplit = (ctx + p.split_tokens - 1) / p.split_tokens;

  extern __shared__ int s_blk[];  // block-table entries of the logical blocks [t0, t1) touches
  __shared__ float s_acc[4][G][HD];
  __shared__ float s_m[4][G], s_l[4][G];

  const int bs = p.bs;
  const int first_lb = t0 / bs;
  const int nlb = (t1 - 1) / bs - first_lb + 1;
  const int32_t* bt_row = p.bt + int64_t(b) * p.max_blocks;
  for (int i = threadIdx.x; i < nlb; i += THREADS) {
    const int blk = bt_row[first_lb + i];
    s_blk[i] = (blk >= 0 && blk < p.num_blocks) ? blk : -1;
  }

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int grp = lane >> 3, sub = lane & 7;

  // This lane's 16 query dims (sub*8 .. +8 and 64 + sub*8 .. +8) of each head in the group, as bf16 pairs.
  uint32_t qa[G][4], qb[G][4];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    const uint16_t* qp = p.q + int64_t(b) * p.q_stride + (kvh * G + g) * HD + sub * 8;
    const uint4 x = *reinterpret_cast<const uint4*>(qp);
    const uint4 y = *reinterpret_cast<const uint4*>(qp + 64);
    qa[g][0] = x.x; qa[g][1] = x.y; qa[g][2] = x.z; qa[g][3] = x.w;
    qb[g][0] = y.x; qb[g][1] = y.y; qb[g][2] = y.z; qb[g][3] = y.w;
  }
  __syncthreads();

  float m[G], l[G], acc[G][16];
#pragma unroll
  for (int g = 0; g < G; ++g) {
    m[g] = kMinusBig;
    l[g] = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[g][i] = 0.f;
  }

  const int64_t slot_elems = int64_t(p.num_kv_heads) * HD;
  const uint16_t* kbase = p.kc + kvh * HD + sub * 8;
  const uint16_t* vbase = p.vc + kvh * HD + sub * 8;

  for (int base = t0 + wave * WAVE_TOKENS; base < t1; base += WG_TOKENS) {
    uint4 ka[4], kb[4], va[4], vb[4];
    bool ok[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int t = base + u * 8 + grp;
      bool valid = t < t1;
      const int tt = valid ? t : t0;
      int lb, cell;
      if (p.bs_shift >= 0) {
        lb = tt >> p.bs_shift;
        cell = tt & (bs - 1);
      } else {
        lb = tt / bs;
        cell = tt - lb * bs;
      }
      const int blk = s_blk[lb - first_lb];
      // A key past the split reads the split's first key instead (a real, finite row): its weight is 0, and
      // 0 * (stale or poisoned data) could be NaN.  Only an unusable block-table entry falls back to slot 0.
      const int64_t off = blk >= 0 ? (int64_t(blk) * bs + cell) * slot_elems : 0;
      ok[u] = valid && blk >= 0;
      ka[u] = *reinterpret_cast<const uint4*>(kbase + off);
      kb[u] = *reinterpret_cast<const uint4*>(kbase + off + 64);
      va[u] = *reinterpret_cast<const uint4*>(vbase + off);
      vb[u] = *reinterpret_cast<const uint4*>(vbase + off + 64);
    }

    float pr[4][G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      float s[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float d = 0.f;
        d = dot2(qa[g][0], ka[u].x, d);
        d = dot2(qa[g][1], ka[u].y, d);
        d = dot2(qa[g][2], ka[u].z, d);
        d = dot2(qa[g][3], ka[u].w, d);
        d = dot2(qb[g][0], kb[u].x, d);
        d = dot2(qb[g][1], kb[u].y, d);
        d = dot2(qb[g][2], kb[u].z, d);
        d = dot2(qb[g][3], kb[u].w, d);
        d = sum8(d);
        s[u] = ok[u] ? d * p.scale_log2 : -INFINITY;
      }
      const float mx = fmaxf(fmaxf(s[0], s[1]), fmaxf(s[2], s[3]));
      const float mn = fmaxf(m[g], mx);
      const float alpha = fast_exp2(m[g] - mn);
      float sum = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        pr[u][g] = fast_exp2(s[u] - mn);
        sum += pr[u][g];
      }
      l[g] = l[g] * alpha + sum;
      m[g] = mn;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[g][i] *= alpha;
    }

#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const uint32_t w[8] = {va[u].x, va[u].y, va[u].z, va[u].w, vb[u].x, vb[u].y, vb[u].z, vb[u].w};
      float vf[16];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        vf[2 * i] = bf16_lo(w[i]);
        vf[2 * i + 1] = bf16_hi(w[i]);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[g][i] = fmaf(pr[u][g], vf[i], acc[g][i]);
      }
    }
  }

  // Merge the 8 lane groups of the wave (lanes with equal `sub` hold the same dims).
#pragma unroll
  for (int off = 8; off < 64; off <<= 1) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const float mo = shfl_xor_f32(m[g], off);
      const float lo = shfl_xor_f32(l[g], off);
      const float mn = fmaxf(m[g], mo);
      const float a = fast_exp2(m[g] - mn), c = fast_exp2(mo - mn);
      l[g] = l[g] * a + lo * c;
      m[g] = mn;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[g][i] = acc[g][i] * a + shfl_xor_f32(acc[g][i], off) * c;
    }
  }
  if (grp == 0) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        s_acc[wave][g][sub * 8 + i] = acc[g][i];
        s_acc[wave][g][64 + sub * 8 + i] = acc[g][8 + i];
      }
      if (sub == 0) {
        s_m[wave][g] = m[g];
        s_l[wave][g] = l[g];
      }
    }
  }
  __syncthreads();

  // Merge the 4 waves; one thread per (head of the group, dim).
  for (int idx = threadIdx.x; idx < G * HD; idx += THREADS) {
    const int g = idx / HD, d = idx % HD;
    float M = s_m[0][g];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, s_m[w][g]);
    float L = 0.f, A = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float e = fast_exp2(s_m[w][g] - M);
      L = fmaf(s_l[w][g], e, L);
      A = fmaf(s_acc[w][g][d], e, A);
    }
    const int qh = kvh * G + g;
    if (nsplit == 1) {
      p.out[(int64_t(b) * p.num_q_heads + qh) * HD + d] = f32_to_bf16(L > 0.f ? A / L : 0.f);
    } else {
      const int64_t row = (int64_t(b) * p.num_q_heads + qh) * p.max_splits + split;
      p.ws_acc[row * HD + d] = A;
      if (d == 0) {
        p.ws_ml[2 * row] = M;
        p.ws_ml[2 * row + 1] = L;
      }
    }
  }
}

// One work-group of 128 threads per (query head, sequence): merge the splits' partial states.
__global__ void __launch_bounds__(HD) decode_combine_kernel(const int32_t* __restrict__ ctx_lens, int max_ctx,
                                                           int split_tokens, int max_splits, int num_q_heads,
                                                           const float* __restrict__ ws_acc,
                                                           const float* __restrict__ ws_ml, uint16_t* __restrict__ out) {
  const int qh = blockIdx.x, b = blockIdx.y, d = threadIdx.x;
  const int ctx = min(ctx_lens[b], max_ctx);
  uint16_t* o = out + (int64_t(b) * num_q_heads + qh) * HD + d;
  if (ctx <= 0) {  // padding row or empty context: zeros
    *o = 0;
    return;
  }
  const int n = (ctx + split_tokens - 1) / split_tokens;
  if (n == 1) return;  // written by the split kernel
  const int64_t row0 = (int64_t(b) * num_q_heads + qh) * max_splits;
  float M = -INFINITY;
  for (int s = 0; s < n; ++s) M = fmaxf(M, ws_ml[2 * (row0 + s)]);
  float L = 0.f, A = 0.f;
  for (int s = 0; s < n; ++s) {
    const float e = fast_exp2(ws_ml[2 * (row0 + s)] - M);
    L = fmaf(ws_ml[2 * (row0 + s) + 1], e, L);
    A = fmaf(ws_acc[(row0 + s) * HD + d], e, A);
  }
  *o = f32_to_bf16(L > 0.f ? A / L : 0.f);
}

template <int G>
hipError_t launch_g(const DecodeKernelArgs& p, int batch, hipStream_t stream) {
  const size_t lds = size_t((p.split_tokens - 1) / p.bs + 2) * sizeof(int);
  hipLaunchKernelGGL(decode_split_kernel<G>, dim3(p.max_splits, p.num_kv_heads, batch), dim3(THREADS), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

bool decode_fast_supported(int head_dim, int group, bool bf16) {
  return bf16 && head_dim == HD && (group == 1 || group == 2 || group == 4);
}

DecodePlan decode_plan(int batch, int num_q_heads, int num_kv_heads, int max_ctx) {
  // Enough work-groups to cover 256 CUs many times over at the longest context, without splits so short
  // that the per-split partial state becomes a noticeable share of the traffic.
  const int64_t units = int64_t(batch) * num_kv_heads;
  int64_t want = units * int64_t(max_ctx) / 8192;
  int split = 256;
  while (split < want && split < 2048) split *= 2;
  DecodePlan plan;
  plan.split_tokens = split;
  plan.max_splits = int((int64_t(max_ctx) + split - 1) / split);
  plan.workspace_bytes = plan.max_splits > 1
                             ? size_t(batch) * num_q_heads * plan.max_splits * (HD + 2) * sizeof(float)
                             : 0;
  return plan;
}

hipError_t launch_decode_bf16(const AttnArgs& a, const DecodePlan& plan, void* workspace, hipStream_t stream) {
  DecodeKernelArgs p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.q_stride = a.q_stride;
  p.kc = static_cast<const uint16_t*>(a.k);
  p.vc = static_cast<const uint16_t*>(a.v);
  p.num_blocks = a.num_blocks;
  p.ctx = a.ctx_lens;
  p.bt = a.block_tables;
  p.max_blocks = a.max_blocks;
  p.bs = a.block_size;
  p.bs_shift = (a.block_size & (a.block_size - 1)) == 0 ? __builtin_ctz(unsigned(a.block_size)) : -1;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.scale_log2 = a.scale * kLog2e;
  p.split_tokens = plan.split_tokens;
  p.max_splits = plan.max_splits;
  p.out = static_cast<uint16_t*>(a.out);
  float* ws = static_cast<float*>(workspace);
  const size_t acc_elems = size_t(a.batch) * a.num_q_heads * plan.max_splits * HD;
  p.ws_acc = plan.max_splits > 1 ? ws : nullptr;
  p.ws_ml = plan.max_splits > 1 ? ws + acc_elems : nullptr;
  const int group = a.num_q_heads / a.num_kv_heads;
  hipError_t e = group == 1 ? launch_g<1>(p, a.batch, stream)
                 : group == 2 ? launch_g<2>(p, a.batch, stream)
                              : launch_g<4>(p, a.batch, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel, dim3(a.num_q_heads, a.batch), dim3(HD), 0, stream, a.ctx_lens,
                     a.max_blocks * a.block_size, plan.split_tokens, plan.max_splits, a.num_q_heads, p.ws_acc, p.ws_ml,
                     p.out);
  return hipGetLastError();
}

}  // namespace pkv
