// QK-Norm + RoPE fused into the KV store, on gfx950.
//
// What it computes [P2 §2 steps 4-6; §4; §5.1; P1 layernorm.py walkthrough]: for each new token and each
// head, q and k are RMS-normalised over head_dim and scaled by their learned weights, then rotated by the
// token's position -- element i paired with i + head_dim/2 at angle position * theta^(-2i/head_dim) --
// and k together with the untouched v is written to the paged cache at the token's slot (slot < 0 skips
// the cache, as the store does); the normalised, rotated q goes to q_out for the attention call.
//
// How (aligned inputs, the usual case): a row of head_dim elements is spread over LPR lanes holding 16
// contiguous bytes each, so every load and store is 16 bytes wide.  A work-group first forms the cosines
// and sines of its tokens once (angles in float64 reduced modulo 2 pi, then the float32 sine and cosine,
// so large positions keep their accuracy) into LDS; then each lane group takes a chunk of 8 rows of one
// token (q rows, then k rows, then v rows), issues all 8 loads before any arithmetic, and for q and k rows
// sums the squares over its lanes, fetches the rotation partners (elements e +- head_dim/2, held by lane
// li ^ LPR/2) by lane exchange and writes w_e x_e cos - w_p x_p sin (first half) or w_e x_e cos +
// w_p x_p sin (second half) times the row's reciprocal RMS, all in float32 with one rounding to the
// storage type.  v rows are copied bit for bit.  Inputs whose rows are not 16-byte aligned take a simple
// element-wise kernel (one wave per row) that computes the same thing.  Either pass reads each q, k, v
// row once and writes each output row once: it is bound by HBM bandwidth.
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

// Element-wise form for inputs without 16-byte aligned rows: one work-group per token, one wave per row.
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


// Lane exchange inside aligned groups of 2^k lanes: lane i receives lane (i ^ M)'s value.  M < 16 uses DPP
// moves inside 16-lane rows (xor 4 as a half-row mirror followed by a quad reversal); M >= 16 goes
// through ds_bpermute.
enum : int { DPP_QUAD_REV = 0x1B, DPP_ROW_ROR8 = 0x128 };

template <int M>
__device__ __forceinline__ uint32_t lane_xor(uint32_t x) {
  const int v = int(x);
  if constexpr (M == 1) return uint32_t(__builtin_amdgcn_mov_dpp(v, DPP_QUAD_XOR1, 0xF, 0xF, false));
  else if constexpr (M == 2) return uint32_t(__builtin_amdgcn_mov_dpp(v, DPP_QUAD_XOR2, 0xF, 0xF, false));
  else if constexpr (M == 4)
    return uint32_t(__builtin_amdgcn_mov_dpp(__builtin_amdgcn_mov_dpp(v, DPP_ROW_HALF_MIRROR, 0xF, 0xF, false),
                                             DPP_QUAD_REV, 0xF, 0xF, false));
  else if constexpr (M == 8) return uint32_t(__builtin_amdgcn_mov_dpp(v, DPP_ROW_ROR8, 0xF, 0xF, false));
  else return uint32_t(__builtin_amdgcn_ds_bpermute((((threadIdx.x & 63) ^ M) << 2), v));
}

template <int M>
__device__ __forceinline__ float group_sum(float x) {  // sum over the aligned group of 2M lanes
  if constexpr (M >= 1) {
    x += __uint_as_float(lane_xor<M>(__float_as_uint(x)));
    return group_sum<M / 2>(x);
  } else {
    return x;
  }
}

template <typename T> struct Vec16;  // 16 bytes of T <-> floats
template <> struct Vec16<uint16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void unpack(const u32x4& r, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) { x[2 * i] = bf16_lo(r[i]); x[2 * i + 1] = bf16_hi(r[i]); }
  }
  __device__ __forceinline__ static u32x4 pack(const float* y) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = pack_bf16x2(y[2 * i], y[2 * i + 1]);
    return r;
  }
};
template <> struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void unpack(const u32x4& r, float* x) {
#pragma unroll
    for (int i = 0; i < 4; ++i) x[i] = __uint_as_float(r[i]);
  }
  __device__ __forceinline__ static u32x4 pack(const float* y) {
    u32x4 r;
#pragma unroll
    for (int i = 0; i < 4; ++i) r[i] = __float_as_uint(y[i]);
    return r;
  }
};

constexpr int QKR_THREADS = 256;
constexpr int QKR_CHUNK = 4;  // rows of one kind that a lane group loads together

template <typename T, int HD>
struct QkrShape {
  static constexpr int VEC = Vec16<T>::N;      // elements per lane
  static constexpr int LPR = HD / VEC;         // lanes per row
  static constexpr int GROUPS = QKR_THREADS / LPR;
  static constexpr int HALF = HD / 2;
};

// Work split: a token's q rows, k rows and v rows are cut into chunks of up to QKR_CHUNK rows of one kind;
// a work-group takes tpw tokens and hands out their chunks kind by kind (all q chunks, then all k chunks,
// then all v chunks), so the lane groups of one wave mostly share a kind and v chunks skip the arithmetic.
struct QkrPlan {
  int cq, ck;  // chunks of q rows and of k (= v) rows per token
  int tpw;     // tokens per work-group
};

struct QkrItem {
  int kind;         // 0 q, 1 k, 2 v
  int t;            // token within the work-group
  int row0, nrows;  // first head and head count of the chunk
};

__device__ __forceinline__ QkrItem qkr_item(int item, int ntok, const QkrPlan& pl, int hq, int hkv) {
  QkrItem it;
  int j = item, per = pl.cq, heads = hq;
  it.kind = 0;
  if (j >= ntok * pl.cq) {
    j -= ntok * pl.cq;
    per = pl.ck;
    heads = hkv;
    it.kind = 1;
    if (j >= ntok * pl.ck) {
      j -= ntok * pl.ck;
      it.kind = 2;
    }
  }
  it.t = j / per;
  it.row0 = (j % per) * QKR_CHUNK;
  it.nrows = min(QKR_CHUNK, heads - it.row0);
  return it;
}

template <typename T>
__device__ __forceinline__ const T* qkr_src(const QkrArgs& a, const QkrItem& it, int tok0, int e0, int hd) {
  const int64_t tok = tok0 + it.t;
  const int64_t off = int64_t(it.row0) * hd + e0;
  if (it.kind == 0) return static_cast<const T*>(a.q) + tok * a.q_stride + off;
  if (it.kind == 1) return static_cast<const T*>(a.k) + tok * a.k_stride + off;
  return static_cast<const T*>(a.v) + tok * a.v_stride + off;
}

template <typename T, int HD>
__device__ __forceinline__ void load_rows(u32x4 (&raw)[QKR_CHUNK], const T* src, int nrows) {
#pragma unroll
  for (int r = 0; r < QKR_CHUNK; ++r)
    raw[r] = r < nrows ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(src + r * HD))
                       : u32x4{0, 0, 0, 0};
}

template <typename T, int HD>
__global__ void __launch_bounds__(QKR_THREADS) qknorm_rope_store_vec_kernel(QkrArgs a, QkrPlan pl) {
  using S = QkrShape<T, HD>;
  constexpr int VEC = S::VEC, LPR = S::LPR, HALF = S::HALF;
  static_assert(LPR >= 2 && LPR <= 64 && HALF % VEC == 0, "unsupported head_dim");
  __shared__ float s_cos[S::GROUPS * HALF];
  __shared__ float s_sin[S::GROUPS * HALF];
  const int g = threadIdx.x / LPR, li = threadIdx.x % LPR;
  const int hq = a.num_q_heads, hkv = a.num_kv_heads;
  const int tok0 = blockIdx.x * pl.tpw;
  const int ntok = min(pl.tpw, a.num_tokens - tok0);
  const int items = ntok * (pl.cq + 2 * pl.ck);
  const int e0 = li * VEC;       // this lane's first element
  const bool first = e0 < HALF;  // first half: the partner follows
  const int fi0 = first ? e0 : e0 - HALF;
  const int ep = first ? e0 + HALF : e0 - HALF;

  // Loads first -- positions, then this group's slot, weights and first chunk of rows -- so the angles
  // below are formed while the rows are in flight.
  constexpr int PER = (S::GROUPS * HALF + QKR_THREADS - 1) / QKR_THREADS;  // angles per thread, at most
  int pos[PER];
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int ti = (threadIdx.x + k * QKR_THREADS) / HALF;
    pos[k] = a.positions[tok0 + min(ti, ntok - 1)];  // clamped: no branch, so no wait per load
  }
  int item = g;
  QkrItem it = qkr_item(min(item, items - 1), ntok, pl, hq, hkv);
  int64_t slot = a.slot_mapping[tok0 + it.t];
  u32x4 w_own, w_par;
  {
    const T* w = static_cast<const T*>(it.kind == 0 ? a.wq : a.wk);
    w_own = *reinterpret_cast<const u32x4*>(w + e0);
    w_par = *reinterpret_cast<const u32x4*>(w + ep);
  }
  u32x4 raw[QKR_CHUNK];
  if (item < items) load_rows<T, HD>(raw, qkr_src<T>(a, it, tok0, e0, HD), it.nrows);

  // Cosines and sines of this work-group's tokens, each angle formed once.
#pragma unroll
  for (int k = 0; k < PER; ++k) {
    const int i = threadIdx.x + k * QKR_THREADS, fi = i % HALF;
    if (i < ntok * HALF) {
      const double ang = double(pos[k]) * exp2(-(2.0 * fi / HD) * a.log2_theta);
      const double r = fma(-6.283185307179586476925287, rint(ang * 0.15915494309189533576888376), ang);
      float cv, sv;
      sincosf(float(r), &sv, &cv);
      s_cos[i] = cv;
      s_sin[i] = sv;
    }
  }
  __syncthreads();

  while (item < items) {
    const int64_t tok = tok0 + it.t;
    const bool store = slot >= 0 && slot < a.num_slots;
    if (it.kind == 2) {  // v: copied to the cache unchanged
      if (store) {
        T* dst = static_cast<T*>(a.v_cache) + (slot * hkv + it.row0) * HD + e0;
#pragma unroll
        for (int r = 0; r < QKR_CHUNK; ++r)
          if (r < it.nrows) __builtin_nontemporal_store(raw[r], reinterpret_cast<u32x4*>(dst + r * HD));
      }
    } else {
      // y_e = inv_rms * (x_e w_e cos + x_p w_p (-+) sin), the partner p = e +- HALF held by lane li ^ LPR/2.
      float cf[VEC], sf[VEC];
      {
        float wo[VEC], wp[VEC];
        Vec16<T>::unpack(w_own, wo);
        Vec16<T>::unpack(w_par, wp);
#pragma unroll
        for (int j = 0; j < VEC; ++j) {
          const float cv = s_cos[it.t * HALF + fi0 + j];
          const float sv = s_sin[it.t * HALF + fi0 + j];
          cf[j] = wo[j] * cv;
          sf[j] = first ? -wp[j] * sv : wp[j] * sv;
        }
      }
      T* dst = it.kind == 0 ? static_cast<T*>(a.q_out) + (tok * hq + it.row0) * HD + e0
                            : static_cast<T*>(a.k_cache) + (slot * hkv + it.row0) * HD + e0;
#pragma unroll
      for (int r = 0; r < QKR_CHUNK; ++r) {
        float x[VEC], xp[VEC], y[VEC];
        Vec16<T>::unpack(raw[r], x);
        u32x4 pr;
#pragma unroll
        for (int i = 0; i < 4; ++i) pr[i] = lane_xor<LPR / 2>(raw[r][i]);
        Vec16<T>::unpack(pr, xp);
        float ss = 0.f;
#pragma unroll
        for (int j = 0; j < VEC; ++j) ss = fmaf(x[j], x[j], ss);
        ss = group_sum<LPR / 2>(ss);
        const float inv = rsqrtf(fmaf(ss, 1.f / HD, a.eps));
#pragma unroll
        for (int j = 0; j < VEC; ++j) y[j] = inv * fmaf(x[j], cf[j], xp[j] * sf[j]);
        if (r < it.nrows && (it.kind == 0 || store))
          __builtin_nontemporal_store(Vec16<T>::pack(y), reinterpret_cast<u32x4*>(dst + r * HD));
      }
    }
    item += S::GROUPS;
    if (item >= items) break;
    it = qkr_item(item, ntok, pl, hq, hkv);
    slot = a.slot_mapping[tok0 + it.t];
    const T* w = static_cast<const T*>(it.kind == 0 ? a.wq : a.wk);
    w_own = *reinterpret_cast<const u32x4*>(w + e0);
    w_par = *reinterpret_cast<const u32x4*>(w + ep);
    load_rows<T, HD>(raw, qkr_src<T>(a, it, tok0, e0, HD), it.nrows);
  }
}

template <typename T, int HD>
hipError_t launch_hd(const QkrArgs& a, bool aligned, hipStream_t stream) {
  if (aligned) {
    using S = QkrShape<T, HD>;
    QkrPlan pl;
    pl.cq = (a.num_q_heads + QKR_CHUNK - 1) / QKR_CHUNK;
    pl.ck = (a.num_kv_heads + QKR_CHUNK - 1) / QKR_CHUNK;
    const int per_tok = pl.cq + 2 * pl.ck;
    pl.tpw = per_tok < S::GROUPS ? S::GROUPS / per_tok : 1;
    const dim3 grid((a.num_tokens + pl.tpw - 1) / pl.tpw), block(QKR_THREADS);
    hipLaunchKernelGGL((qknorm_rope_store_vec_kernel<T, HD>), grid, block, 0, stream, a, pl);
  } else {
    hipLaunchKernelGGL((qknorm_rope_store_kernel<T, HD>), dim3(a.num_tokens), dim3(256), 0, stream, a);
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_t(const QkrArgs& a, int head_dim, bool aligned, hipStream_t stream) {
  switch (head_dim) {
    case 16: return launch_hd<T, 16>(a, aligned, stream);
    case 32: return launch_hd<T, 32>(a, aligned, stream);
    case 64: return launch_hd<T, 64>(a, aligned, stream);
    case 128: return launch_hd<T, 128>(a, aligned, stream);
    case 256: return launch_hd<T, 256>(a, aligned, stream);
    default: return hipErrorInvalidValue;
  }
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15) == 0; }

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
  const int64_t esz = bf16 ? 2 : 4;
  const bool aligned = aligned16(q) && aligned16(k) && aligned16(v) && aligned16(q_out) && aligned16(k_cache) &&
                       aligned16(v_cache) && aligned16(q_norm_weight) && aligned16(k_norm_weight) &&
                       (q_stride * esz) % 16 == 0 && (k_stride * esz) % 16 == 0 && (v_stride * esz) % 16 == 0;
  return bf16 ? launch_t<uint16_t>(a, head_dim, aligned, stream) : launch_t<float>(a, head_dim, aligned, stream);
}

}  // namespace pkv
