// Paged single-token decode attention, bf16 storage, head_dim 128, on gfx950.
//
// What it computes [P2 §5.3 decode call; P3 §4]: for every sequence b and query head h,
// o = softmax(scale * q K^T) V over the context_lens[b] keys of b, key j read from slot
// block_tables[b][j / block_size] * block_size + j % block_size of the paged caches, with kv head
// h / (Hq / Hkv) [P2 §3].
//
// How (gfx950 design, not the pages' library call):
//  * Even split of the whole batch: the keys of all sequences, laid end to end (T = sum of context
//    lengths), are cut into W equal ranges, one per worker (two workers per CU, each worker one work-group
//    per group of 4 kv heads, all resident at once).  Every work-group therefore streams the same number of
//    bytes and the launch is a single round with no tail, whatever the mix of context lengths (a range may
//    cover the end of one sequence and the start of the next).
//  * A work-group has one wave per kv head, so together its waves read whole contiguous token rows of the
//    cache; each wave serves every query head of its kv head's GQA group, so each K/V row is read from HBM
//    once for the whole group.
//  * A token's 256-byte K (or V) row for one kv head is read by 8 lanes, 2 x 16 bytes each; a wave reads
//    8 tokens per instruction (8 full 128-byte lines) and 32 tokens per iteration, all loads issued before
//    any arithmetic; the block-table entries of the next iteration are fetched one iteration ahead.  The
//    cache is read with non-temporal loads (each byte is used once): measured 5.2 -> 5.6 TB/s at batch 64.
//  * q.k uses the packed bf16 dot instruction (exact products, float32 sums); the 8 partial sums of a
//    token are combined with three DPP moves inside the 8-lane group.
//  * Each 8-lane group runs its own online softmax (running max m, normaliser l, unnormalised output) over
//    its tokens [P2 §5.2 ②], in base 2 with log2(e) folded into the scale.  At the end of a sequence's
//    range the 8 groups are merged with lane shuffles; a sequence wholly inside one range is written
//    directly, otherwise each range writes (m, l, unnormalised output) and a combine kernel merges them with
//    the same exact rescaling by exp(m_i - m).
//  * Fused with the store (attn_decode_paged_store) [P2 §5.1 then §5.3; P3 §4 note on the order]: the new
//    token of sequence b sits at position context_lens[b] - 1, the last key of b.  Only the worker whose key
//    range ends b reads that slot, so that worker itself copies the token's K and V rows from the step's
//    k_new / v_new rows into the slot (each wave its kv head's 512 bytes) and waits for the write before
//    its first read of the sequence; no other work-group reads the slot and nothing else waits.  The first
//    work-group can also write the step's slot_mapping.
#include <math.h>

#include <algorithm>
#include <atomic>

#include "common.h"
#include "launch.h"

namespace pkv {
namespace {

constexpr int HD = 128;
constexpr int MAX_WAVES = 4;  // kv heads per work-group, one wave each
constexpr int WAVE_TOKENS = 32;
constexpr int MAX_WORKERS = 1024;  // upper bound of W, used to size the workspace
constexpr int LDS_CU_MAX = 2048;   // prefix sums staged in LDS up to this many entries
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
  int batch;
  int max_blocks;
  int bs;
  int bs_shift;  // log2(block_size) when it is a power of two, else -1
  int num_q_heads;
  int num_kv_heads;
  float scale_log2;
  int workers;     // W
  int64_t* cu;     // [batch + 1] prefix sums of the clamped context lengths (workspace)
  float* ws_acc;   // [W + batch][Hq][HD] unnormalised partial outputs (workspace)
  float* ws_ml;    // [W + batch][Hq][2] partial (m, l) (workspace)
  uint16_t* out;
  // Fused store (STORE kernels only): the step's new K/V rows [batch][Hkv][HD] with token strides in
  // elements, and an optional slot_mapping output.
  const uint16_t* knew;
  int64_t knew_stride;
  const uint16_t* vnew;
  int64_t vnew_stride;
  int32_t* slot_out;
};

__device__ __forceinline__ int clamp_ctx(const DecodeKernelArgs& p, int b) {
  return min(max(p.ctx[b], 0), p.max_blocks * p.bs);
}

// Prefix sums of the clamped context lengths: cu[b] = sum_{i<b} ctx_i.  One work-group of 1024 threads.
__global__ void __launch_bounds__(1024) decode_prefix_kernel(DecodeKernelArgs p) {
  __shared__ int64_t part[1024];
  __shared__ int64_t carry;
  if (threadIdx.x == 0) carry = 0;
  __syncthreads();
  for (int base = 0; base < p.batch; base += 1024) {
    const int b = base + threadIdx.x;
    const int64_t x = b < p.batch ? clamp_ctx(p, b) : 0;
    part[threadIdx.x] = x;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {  // inclusive scan
      const int64_t y = threadIdx.x >= o ? part[threadIdx.x - o] : 0;
      __syncthreads();
      part[threadIdx.x] += y;
      __syncthreads();
    }
    if (b < p.batch) p.cu[b] = carry + part[threadIdx.x] - x;
    __syncthreads();
    if (threadIdx.x == 1023) carry += part[1023];
    __syncthreads();
  }
  if (threadIdx.x == 0) p.cu[p.batch] = carry;
}

// A wave-uniform 64-bit value held in SGPRs (values read from LDS arrive in VGPRs).
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x)));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(uint64_t(x) >> 32));
  return int64_t((uint64_t(hi) << 32) | lo);
}

// Workers that get keys: at most the launched W, and at least MIN_KEYS keys each, so that a small batch is not
// cut into hundreds of tiny ranges whose partial outputs cost more to merge than to compute (one row of 2.9k keys
// over every worker: 60 us per step).  Measured on MI355X per decode step at 1 / 8 rows (2.9k / 13k keys): 20.3 /
// 26.8 us with at least 128 keys per worker, 19.3 / 25.1 with 64, 23.3 / 29.5 with 32; batch 64 and up have more
// keys than that per worker.  Every work-group and the combine kernel derive it from T the same way.
constexpr int MIN_KEYS = 64;
__device__ __forceinline__ int active_workers(int64_t T, int W) {
  return int(max(int64_t(1), min(int64_t(W), T / MIN_KEYS)));
}

__device__ __forceinline__ int64_t range_begin(int64_t T, int W, int w) { return T * w / W; }

// The worker whose range holds global key index x (ranges are [range_begin(w), range_begin(w + 1))).
__device__ __forceinline__ int worker_of(int64_t T, int W, int64_t x) { return int(((x + 1) * W - 1) / T); }

template <int G, bool STORE>
__global__ void __launch_bounds__(64 * MAX_WAVES) __attribute__((amdgpu_waves_per_eu(G <= 2 ? 3 : 2)))
decode_lean_kernel(DecodeKernelArgs p) {
  const int w = blockIdx.y;
  if (STORE && p.slot_out && blockIdx.x == 0 && blockIdx.y == 0) {
    // The step's slot_mapping: position context_lens[b] - 1 through the block table, -1 when there is none.
    for (int i = threadIdx.x; i < p.batch; i += blockDim.x) {
      const int pos = p.ctx[i] - 1, lb = pos >= 0 ? pos / p.bs : 0;
      const int blk = pos >= 0 && lb < p.max_blocks ? p.bt[int64_t(i) * p.max_blocks + lb] : -1;
      const int64_t slot = blk >= 0 ? int64_t(blk) * p.bs + pos % p.bs : -1;  // 64-bit: no wrap into range
      p.slot_out[i] = slot <= int64_t(INT32_MAX) ? int32_t(slot) : -1;
    }
  }
  // Prefix sums of the clamped context lengths.  Up to LDS_CU_MAX - 1 sequences every work-group scans them
  // into LDS itself (a few hundred cycles, and one kernel launch less); the first work-group also stores them
  // for the combine kernel.  Larger batches read the sums decode_prefix_kernel wrote.
  extern __shared__ int64_t s_cu[];
  const bool cu_in_lds = p.batch + 1 <= LDS_CU_MAX;
  if (cu_in_lds) {
    int64_t* chunk = s_cu + (p.batch + 1);
    const int nt = blockDim.x, tid = threadIdx.x;
    const int per = (p.batch + nt - 1) / nt;
    const int c0 = min(tid * per, p.batch), c1 = min(c0 + per, p.batch);
    int64_t acc = 0;
    for (int i = c0; i < c1; ++i) {
      const int64_t c = clamp_ctx(p, i);
      s_cu[i + 1] = c;
      acc += c;
    }
    // Exclusive prefix of the chunk sums: an inclusive scan inside each wave (lane shuffles), then the totals of
    // the preceding waves (one barrier).
    const int lane = tid & 63, wv = tid >> 6;
    int64_t inc = acc;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int src = lane >= off ? lane - off : lane;
      const uint32_t lo = __builtin_amdgcn_ds_bpermute(src << 2, int(uint32_t(uint64_t(inc))));
      const uint32_t hi = __builtin_amdgcn_ds_bpermute(src << 2, int(uint32_t(uint64_t(inc) >> 32)));
      if (lane >= off) inc += int64_t((uint64_t(hi) << 32) | lo);
    }
    if (lane == 63) chunk[wv] = inc;
    __syncthreads();
    acc = inc - acc;
    for (int v = 0; v < wv; ++v) acc += chunk[v];
    for (int i = c0; i < c1; ++i) {
      acc += s_cu[i + 1];
      s_cu[i + 1] = acc;
    }
    if (tid == 0) s_cu[0] = 0;
    __syncthreads();
    if (blockIdx.x == 0 && blockIdx.y == 0)
      for (int i = tid; i <= p.batch; i += nt) p.cu[i] = s_cu[i];
  }
  const int64_t T = cu_in_lds ? s_cu[p.batch] : p.cu[p.batch];
  const int W = active_workers(T, p.workers);
  if (w >= W) return;
  int64_t x = range_begin(T, W, w);
  const int64_t x_end = range_begin(T, W, w + 1);
  if (x >= x_end) return;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int kvh = blockIdx.x * (blockDim.x >> 6) + wave;
  const int grp = lane >> 3, sub = lane & 7;
  const int bs = p.bs;
  const int64_t slot_elems = int64_t(p.num_kv_heads) * HD;
  const uint16_t* kbase = p.kc + kvh * HD + sub * 8;
  const uint16_t* vbase = p.vc + kvh * HD + sub * 8;

  // First sequence of the range: the last b with cu[b] <= x (empty sequences are skipped over).
  int b;
  {
    int lo = 0, hi = p.batch;  // cu[lo] <= x < cu[hi]
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if ((cu_in_lds ? s_cu[mid] : p.cu[mid]) <= x) lo = mid; else hi = mid;
    }
    b = __builtin_amdgcn_readfirstlane(lo);  // uniform: keep it (and what derives from it) in SGPRs
  }
  if (kvh >= p.num_kv_heads) return;

  while (x < x_end && b < p.batch) {
    const int64_t seq0 = uniform64(cu_in_lds ? s_cu[b] : p.cu[b]);
    const int64_t seq1 = uniform64(cu_in_lds ? s_cu[b + 1] : p.cu[b + 1]);
    if (seq1 <= x) {  // empty sequence
      ++b;
      continue;
    }
    const int ctx = int(seq1 - seq0);
    const int t0 = int(x - seq0);
    const int t1 = int(min(x_end, seq1) - seq0);
    const int32_t* bt_row = p.bt + int64_t(b) * p.max_blocks;
    // Fused store: when this range ends the sequence and the context was not clamped, key ctx - 1 is the step's
    // new token, whose rows must reach the cache before this wave reads that slot (lanes 0-15 of the wave move
    // its kv head's K row, lanes 16-31 the V row, 16 bytes each).  The rows are loaded here, next to the
    // query and block-table loads the first iteration waits for anyway, written at the top of the first
    // iteration, and the write is waited for at the top of the iteration that reads the slot (the last one).
    int new_blk = -1;  // cache block of the pending write, -1: none
    u32x4 new_row = {0, 0, 0, 0};
    if (STORE && t1 == ctx && p.ctx[b] == ctx) {
      const int blk = bt_row[(ctx - 1) / bs];
      if (blk >= 0 && blk < p.num_blocks) {
        new_blk = blk;
        if (lane < 32) {
          const uint16_t* src = (lane < 16 ? p.knew + int64_t(b) * p.knew_stride : p.vnew + int64_t(b) * p.vnew_stride) +
                                kvh * HD + (lane & 15) * 8;
          new_row = *reinterpret_cast<const u32x4*>(src);
        }
      }
    }
    bool wrote = false;  // the new rows were written and not yet waited for
    // This lane's 16 query dims (sub*8 .. +8 and 64 + sub*8 .. +8) of each head in the group, as bf16 pairs.
    uint32_t qa[G][4], qb[G][4];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      const uint16_t* qp = p.q + int64_t(b) * p.q_stride + (kvh * G + g) * HD + sub * 8;
      const u32x4 xq = *reinterpret_cast<const u32x4*>(qp);
      const u32x4 yq = *reinterpret_cast<const u32x4*>(qp + 64);
      qa[g][0] = xq.x; qa[g][1] = xq.y; qa[g][2] = xq.z; qa[g][3] = xq.w;
      qb[g][0] = yq.x; qb[g][1] = yq.y; qb[g][2] = yq.z; qb[g][3] = yq.w;
    }

    float m[G], l[G], acc[G][16];
#pragma unroll
    for (int g = 0; g < G; ++g) {
      m[g] = kMinusBig;
      l[g] = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[g][i] = 0.f;
    }

    // Slot of this lane's token u in the iteration starting at `base` (token base + 8 u + grp).  A token
    // past the range reads the range's first token instead (a real, finite row whose weight is 0, where
    // 0 * stale or poisoned data could be NaN); an unusable block-table entry reads slot 0 and is masked.
    int64_t off_n[4];  // element offset of the token's K (and V) row from the cache bases
    bool ok_n[4];
    auto locate = [&](int base) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = base + u * 8 + grp;
        const int tt = t < t1 ? t : t0;
        int lb, cell;
        if (p.bs_shift >= 0) {
          lb = tt >> p.bs_shift;
          cell = tt & (bs - 1);
        } else {
          lb = tt / bs;
          cell = tt - lb * bs;
        }
        const int blk = bt_row[lb];
        const bool usable = blk >= 0 && blk < p.num_blocks;
        ok_n[u] = usable && t < t1;
        off_n[u] = usable ? (int64_t(blk) * bs + cell) * slot_elems : 0;
      }
    };
    locate(t0);

    for (int base = t0; base < t1; base += WAVE_TOKENS) {
      if (STORE && new_blk >= 0) {  // first iteration: the rows arrived with the block-table entries
        if (lane < 32) {
          const int64_t dst = (int64_t(new_blk) * bs + (ctx - 1) % bs) * slot_elems + kvh * HD + (lane & 15) * 8;
          uint16_t* cache = const_cast<uint16_t*>(lane < 16 ? p.kc : p.vc);
          *reinterpret_cast<u32x4*>(cache + dst) = new_row;
        }
        new_blk = -1;
        wrote = true;
      }
      if (STORE && wrote && base + WAVE_TOKENS >= t1) {
        // The write completes (s_waitcnt vmcnt(0): acknowledged by L2) before the loads below, whose lanes of
        // another group read the slot; the fence keeps the compiler from moving those loads above it.
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "workgroup");
        __builtin_amdgcn_s_waitcnt(0);
        wrote = false;
      }
      u32x4 ka[4], kb[4], va[4], vb[4];
      bool ok[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int64_t off = off_n[u];
        ok[u] = ok_n[u];
        ka[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + off));
        kb[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(kbase + off + 64));
        va[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + off));
        vb[u] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(vbase + off + 64));
      }
      if (base + WAVE_TOKENS < t1) locate(base + WAVE_TOKENS);

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
        const uint32_t wv[8] = {va[u].x, va[u].y, va[u].z, va[u].w, vb[u].x, vb[u].y, vb[u].z, vb[u].w};
        float vf[16];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          vf[2 * i] = bf16_lo(wv[i]);
          vf[2 * i + 1] = bf16_hi(wv[i]);
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
    // Lanes 0..7 hold the result: dims sub*8 .. +8 and 64 + sub*8 .. +8 of each head of the group.
    if (grp == 0) {
      const bool whole = t0 == 0 && t1 == ctx;
#pragma unroll
      for (int g = 0; g < G; ++g) {
        const int qh = kvh * G + g;
        if (whole) {
          const float inv = l[g] > 0.f ? 1.f / l[g] : 0.f;
          uint16_t* o = p.out + (int64_t(b) * p.num_q_heads + qh) * HD + sub * 8;
          u32x4 lo4, hi4;
          lo4.x = pack_bf16x2(acc[g][0] * inv, acc[g][1] * inv);
          lo4.y = pack_bf16x2(acc[g][2] * inv, acc[g][3] * inv);
          lo4.z = pack_bf16x2(acc[g][4] * inv, acc[g][5] * inv);
          lo4.w = pack_bf16x2(acc[g][6] * inv, acc[g][7] * inv);
          hi4.x = pack_bf16x2(acc[g][8] * inv, acc[g][9] * inv);
          hi4.y = pack_bf16x2(acc[g][10] * inv, acc[g][11] * inv);
          hi4.z = pack_bf16x2(acc[g][12] * inv, acc[g][13] * inv);
          hi4.w = pack_bf16x2(acc[g][14] * inv, acc[g][15] * inv);
          *reinterpret_cast<u32x4*>(o) = lo4;
          *reinterpret_cast<u32x4*>(o + 64) = hi4;
        } else {
          // (worker, sequence) pairs that share keys are distinct in w + b: slot w + b holds this partial.
          const int64_t row = int64_t(w + b) * p.num_q_heads + qh;
          float* a = p.ws_acc + row * HD + sub * 8;
          *reinterpret_cast<float4*>(a) = make_float4(acc[g][0], acc[g][1], acc[g][2], acc[g][3]);
          *reinterpret_cast<float4*>(a + 4) = make_float4(acc[g][4], acc[g][5], acc[g][6], acc[g][7]);
          *reinterpret_cast<float4*>(a + 64) = make_float4(acc[g][8], acc[g][9], acc[g][10], acc[g][11]);
          *reinterpret_cast<float4*>(a + 68) = make_float4(acc[g][12], acc[g][13], acc[g][14], acc[g][15]);
          if (sub == 0) *reinterpret_cast<float2*>(p.ws_ml + 2 * row) = make_float2(m[g], l[g]);
        }
      }
    }
    x = seq0 + t1;
    ++b;
  }
}

// One work-group per (sequence, pair of query heads): merge the partial states of the workers whose ranges
// cut the sequence, or write zeros for an empty context.  Thread t takes dims 2 (t mod 64) and 2 (t mod 64) + 1
// of query head blockIdx.y * blockDim / 64 + t / 64 (then in steps of gridDim.y * blockDim / 64); partials are
// read 8 at a time (independent loads in flight) and merged with a running maximum, the same exact rescaling
// as everywhere else.  Two heads per work-group measured about 1 % faster on the whole decode call than one
// work-group per sequence over all 16 heads (more work-groups start at once; 1, 2 or 4 heads are alike).
__global__ void __launch_bounds__(1024) decode_combine_kernel(DecodeKernelArgs p) {
  const int b = blockIdx.x;
  const int64_t T = p.cu[p.batch];
  const int64_t x0 = p.cu[b], x1 = p.cu[b + 1];
  const int W = active_workers(T, p.workers);
  const int w0 = x1 > x0 ? worker_of(T, W, x0) : 0, w1 = x1 > x0 ? worker_of(T, W, x1 - 1) : 0;
  if (x1 > x0 && w0 == w1) return;  // written by its worker
  const bool dense = T >= W;        // then no range is empty
  const int pair = threadIdx.x & 63;
  for (int qh = blockIdx.y * (blockDim.x >> 6) + (threadIdx.x >> 6); qh < p.num_q_heads; qh += gridDim.y * (blockDim.x >> 6)) {
    uint32_t* o = reinterpret_cast<uint32_t*>(p.out + (int64_t(b) * p.num_q_heads + qh) * HD) + pair;
    if (x1 <= x0) {  // padding row or empty context: zeros
      *o = 0u;
      continue;
    }
    float M = -INFINITY, L = 0.f, A0 = 0.f, A1 = 0.f;
    for (int c0 = w0; c0 <= w1; c0 += 8) {
      float mv[8], lv[8], a0[8], a1[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int w = c0 + j;
        const bool valid = w <= w1 && (dense || range_begin(T, W, w) < range_begin(T, W, w + 1));
        const int64_t row = int64_t(w + b) * p.num_q_heads + qh;
        const float2 ml = valid ? *reinterpret_cast<const float2*>(p.ws_ml + 2 * row) : make_float2(-INFINITY, 0.f);
        const float2 av = valid ? *reinterpret_cast<const float2*>(p.ws_acc + row * HD + 2 * pair) : make_float2(0.f, 0.f);
        mv[j] = ml.x;
        lv[j] = ml.y;
        a0[j] = av.x;
        a1[j] = av.y;
      }
      float cm = mv[0];
#pragma unroll
      for (int j = 1; j < 8; ++j) cm = fmaxf(cm, mv[j]);
      const float mn = fmaxf(M, cm);
      const float sc = fast_exp2(M - mn);
      L *= sc;
      A0 *= sc;
      A1 *= sc;
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const float e = fast_exp2(mv[j] - mn);
        L = fmaf(lv[j], e, L);
        A0 = fmaf(a0[j], e, A0);
        A1 = fmaf(a1[j], e, A1);
      }
      M = mn;
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    *o = pack_bf16x2(A0 * inv, A1 * inv);
  }
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

struct Layout {
  size_t cu, acc, ml, total;
};

Layout workspace_layout(int batch, int num_q_heads) {
  Layout L;
  const size_t slots = size_t(MAX_WORKERS) + size_t(batch);
  L.cu = 0;
  L.acc = align256((size_t(batch) + 1) * sizeof(int64_t));
  L.ml = L.acc + align256(slots * num_q_heads * HD * sizeof(float));
  L.total = L.ml + align256(slots * num_q_heads * 2 * sizeof(float));
  return L;
}

// W: as many work-groups as the device keeps resident at once (cached per device and kernel shape).
// The caches are atomics: several host threads may launch at once (they store equal values).
int resident_workers(const void* kernel, int threads, int key) {
  static std::atomic<int> cached[64][6][MAX_WAVES + 1] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::atomic<int>& slot = cached[dev][key][threads / 64];
  if (const int v = slot.load(std::memory_order_relaxed); v > 0) return v;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads,
                                                   (LDS_CU_MAX + 64 * MAX_WAVES) * sizeof(int64_t)) !=
          hipSuccess || per_cu <= 0)
    per_cu = 1;
  const int v = std::min(MAX_WORKERS, cus * per_cu);
  slot.store(v, std::memory_order_relaxed);
  return v;
}

int device_cus() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (const int v = cached[dev].load(std::memory_order_relaxed); v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}

template <int G, int KEY, bool STORE>
hipError_t launch_g(DecodeKernelArgs& p, hipStream_t stream) {
  const int waves = std::min(MAX_WAVES, p.num_kv_heads);
  const int threads = 64 * waves;
  const int head_groups = (p.num_kv_heads + waves - 1) / waves;
  // W workers x head_groups work-groups, the head groups of a worker adjacent in launch order so they read the
  // two halves of the same token rows at the same time.  W = 2 per CU, within one resident round: enough
  // loads in flight to saturate HBM (measured on MI355X, batch 64: 1024 / 768 / 512 / 256 workers reach
  // 4.93 / 5.07 / 5.14 / 4.99 TB/s; fewer workers also mean fewer partial outputs to merge).
  const int resident =
      resident_workers(reinterpret_cast<const void*>(&decode_lean_kernel<G, STORE>), threads, KEY + (STORE ? 3 : 0));
  p.workers = std::max(1, std::min(resident / head_groups, 2 * device_cus()));
  const bool cu_in_lds = p.batch + 1 <= LDS_CU_MAX;
  if (!cu_in_lds) hipLaunchKernelGGL(decode_prefix_kernel, dim3(1), dim3(1024), 0, stream, p);
  const size_t lds = cu_in_lds ? size_t(p.batch + 1 + threads) * sizeof(int64_t) : 0;
  hipLaunchKernelGGL((decode_lean_kernel<G, STORE>), dim3(head_groups, p.workers), dim3(threads), lds, stream, p);
  hipLaunchKernelGGL(decode_combine_kernel, dim3(p.batch, (p.num_q_heads + 1) / 2), dim3(64 * std::min(2, p.num_q_heads)), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// Scratch for callers that cannot allocate (attn_decode_paged_store_noalloc): the decode workspace in a
// file-scope device array, one copy per GPU, held until the process ends.  Host code never uses the array's
// name as an address (on the host it is only a stand-in); its device address is looked up once per device,
// with that device current, and kept.
static __device__ __align__(256) unsigned char scratch[kDecodeScratchBytes];

hipError_t decode_static_scratch(void** ptr) {
  static std::atomic<void*> per_device[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  void* p = per_device[dev].load(std::memory_order_acquire);
  if (!p) {
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    per_device[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

bool decode_fast_supported(int head_dim, int group, bool bf16) {
  return bf16 && head_dim == HD && (group == 1 || group == 2 || group == 4);
}

DecodePlan decode_plan(int batch, int num_q_heads, int /*num_kv_heads*/, int /*max_ctx*/) {
  DecodePlan plan;
  plan.workspace_bytes = workspace_layout(batch, num_q_heads).total;
  return plan;
}

hipError_t launch_decode_bf16(const AttnArgs& a, const DecodePlan& plan, void* workspace, hipStream_t stream,
                              const DecodeStoreArgs* fused) {
  (void)plan;
  const Layout L = workspace_layout(a.batch, a.num_q_heads);
  char* ws = static_cast<char*>(workspace);
  DecodeKernelArgs p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.q_stride = a.q_stride;
  p.kc = static_cast<const uint16_t*>(a.k);
  p.vc = static_cast<const uint16_t*>(a.v);
  p.num_blocks = a.num_blocks;
  p.ctx = a.ctx_lens;
  p.bt = a.block_tables;
  p.batch = a.batch;
  p.max_blocks = a.max_blocks;
  p.bs = a.block_size;
  p.bs_shift = (a.block_size & (a.block_size - 1)) == 0 ? __builtin_ctz(unsigned(a.block_size)) : -1;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.scale_log2 = a.scale * kLog2e;
  p.workers = 0;
  p.cu = reinterpret_cast<int64_t*>(ws + L.cu);
  p.ws_acc = reinterpret_cast<float*>(ws + L.acc);
  p.ws_ml = reinterpret_cast<float*>(ws + L.ml);
  p.out = static_cast<uint16_t*>(a.out);
  p.knew = fused ? static_cast<const uint16_t*>(fused->k_new) : nullptr;
  p.knew_stride = fused ? fused->k_new_stride : 0;
  p.vnew = fused ? static_cast<const uint16_t*>(fused->v_new) : nullptr;
  p.vnew_stride = fused ? fused->v_new_stride : 0;
  p.slot_out = fused ? fused->slot_out : nullptr;
  const int group = a.num_q_heads / a.num_kv_heads;
  if (fused)
    return group == 1 ? launch_g<1, 0, true>(p, stream)
                      : group == 2 ? launch_g<2, 1, true>(p, stream) : launch_g<4, 2, true>(p, stream);
  return group == 1 ? launch_g<1, 0, false>(p, stream)
                    : group == 2 ? launch_g<2, 1, false>(p, stream) : launch_g<4, 2, false>(p, stream);
}

}  // namespace pkv
