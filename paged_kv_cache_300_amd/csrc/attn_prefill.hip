// Varlen causal prefill attention on gfx950 bf16 MFMA (head_dim 128), contiguous or paged K/V.
//
// What it computes [P2 §5.3; P3 §4; P1 Q6 §3]: for sequence b, query head h and query row i (the i-th of
// the sequence's Lq new tokens, at absolute position Lk - Lq + i), o = softmax(scale * q K^T) V over keys
// 0 .. Lk - Lq + i (causal) or 0 .. Lk - 1; keys come from this step's k/v rows (contiguous mode) or from the
// paged cache through the block table (prefix-cache / chunked prefill).  Query head h reads kv head
// h / G, G = Hq / Hkv [P2 §3].
//
// How (the FlashAttention tiling of [P2 §5.2], laid out for CDNA4):
//  * A work-group owns 64 query tokens of one sequence for one kv head and ALL G query heads that share it,
//    so every K/V tile is loaded once for the whole GQA group.  Its 4 waves own 16 tokens each; a wave's
//    G heads are G MFMA column blocks over the same 16 tokens (one causal mask serves all of them).
//  * Scores are computed transposed, S^T = K Q^T, with v_mfma_f32_16x16x32_bf16: Q^T stays in registers as
//    the B operand for the whole key loop, K rows are read from LDS as the A operand.  In that layout a
//    lane's accumulators already are the B operand P^T of the second product O^T = V^T P^T, so the
//    probabilities never leave registers; the per-query softmax statistics sit in the same lane as the
//    query's output column, so the online rescale [P2 §5.2 ②] is a per-lane multiply.
//  * K/V tiles of 64 keys are staged through LDS with 16-byte loads, double-buffered: the next tile's global
//    loads are in flight while the current tile is multiplied; rows are padded (272 B) so the 16 lanes of a
//    quarter-wave hit distinct banks.
//  * Softmax in base 2 with log2(e) folded into the scale; the running maximum is shared by the 4 lane
//    groups of a query (two lane swaps per tile).  The normaliser is accumulated on the matrix cores as one
//    more block of V^T whose first row is ones, which takes its sum off the vector units.
//  * Only tiles that cross the causal diagonal or the end of the keys are masked.  Work-groups are
//    launched heaviest query tile first so the long causal rows do not form the tail.
#include <math.h>

#include "common.h"
#include "launch.h"

namespace pkv {
namespace {

constexpr int HD = 128;
constexpr int BM = 64;        // query tokens per work-group
constexpr int BN = 64;        // keys per tile
constexpr int TOKEN_WAVES = 4; // waves per head slice: 4 x 16 query tokens
// LDS row pitch (elements) of the K and V tiles: 288 B, i.e. rows 32 B apart modulo 256 B.  With it both
// the 16-row x 16 B reads of K and the 4-row x 32 B transposing reads of V are free of bank conflicts
// (measured: SQ_LDS_BANK_CONFLICT = 0; pitches of 256, 272 and 304 B all conflict).
constexpr int KROW = HD + 16;
constexpr int VROW = HD + 16;
constexpr float kLog2e = 1.4426950408889634f;
#ifndef PKV_PREFILL_H2
#define PKV_PREFILL_H2 2  // query heads per wave for GQA groups of 2
#endif
constexpr float kMinusBig = -1e30f;

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;

__device__ __forceinline__ f32x4_t mfma_16x16x32(const u32x4& a, const u32x4& b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4_t;

// Transposing LDS read (gfx950): within each 16-lane quarter-wave, result lane i element j comes from the
// 8 bytes addressed by source lane 4 j + i / 4, element i % 4.
__device__ __forceinline__ u32x2 ds_read_tr16(const uint16_t* lds_ptr) {
  const i16x4_t v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4_t*)(lds_ptr));
  return __builtin_bit_cast(u32x2, v);
}

// Maximum over lanes i and i ^ 16 (rows of 16 swapped pairwise), and over lanes i and i ^ 32.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

struct PrefillKernelArgs {
  const uint16_t* q;
  int64_t q_stride;
  const uint16_t* k;
  int64_t k_stride;
  const uint16_t* v;
  int64_t v_stride;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* bt;  // null: contiguous mode
  int max_blocks;
  int bs;
  int bs_shift;  // log2(block_size) if a power of two, else -1
  int num_blocks;
  int64_t num_k_rows;
  int num_q_tokens;
  int num_q_heads;
  int num_kv_heads;
  float scale_log2;
  int causal;
  int max_tiles;
  uint16_t* out;
};

struct TileSource {
  const uint16_t* kbase;  // this thread's chunk of kv head `kvh` at slot/row 0
  const uint16_t* vbase;
  const uint16_t* khead;  // kv head `kvh` at slot/row 0 (uniform)
  const uint16_t* vhead;
  const int32_t* bt_row;  // null: contiguous rows
  int krow;
  int Lk;
  int64_t k_start;
  int64_t slot_elems;
  bool fast;              // full tiles can use the uniform-base path below
  int32_t koff[4], voff[4];  // this thread's element offsets inside a tile (rows krow + 16 i, its chunk)
};

template <int CH>
struct Staged {
  u32x4 k[CH], v[CH];
};

__device__ __forceinline__ int block_of(const PrefillKernelArgs& p, const int32_t* bt_row, int lb) {
  const int blk = bt_row[lb];
  return (blk >= 0 && blk < p.num_blocks) ? blk : 0;
}

// Thread t of NT moves the 16-byte chunk t % 16 of tile rows krow + (NT / 16) i, i < CH = 1024 / NT.
template <int CH>
__device__ __forceinline__ Staged<CH> load_tile(const PrefillKernelArgs& p, const TileSource& s, int kt) {
  constexpr int RSTEP = 64 / CH;
  Staged<CH> r;
  const bool full = (kt + 1) * BN <= s.Lk;
  if (full && s.fast) {
    // The tile's 64 rows are consecutive (contiguous mode) or lie in one block: one uniform base per tile and
    // 32-bit per-thread offsets.
    const uint16_t *kt_base, *vt_base;
    if (s.bt_row) {
      const int key0 = kt * BN;
      const int64_t slot0 = int64_t(block_of(p, s.bt_row, key0 >> p.bs_shift)) * p.bs + (key0 & (p.bs - 1));
      kt_base = s.khead + slot0 * s.slot_elems;
      vt_base = s.vhead + slot0 * s.slot_elems;
    } else {
      const int64_t row0 = s.k_start + int64_t(kt) * BN;
      kt_base = s.khead + row0 * p.k_stride;
      vt_base = s.vhead + row0 * p.v_stride;
    }
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      r.k[i] = *reinterpret_cast<const u32x4*>(kt_base + s.koff[i]);
      r.v[i] = *reinterpret_cast<const u32x4*>(vt_base + s.voff[i]);
    }
    return r;
  }
  if (s.bt_row) {
    const bool tile_in_block = p.bs_shift >= 6;
    const int ublk = tile_in_block ? block_of(p, s.bt_row, (kt * BN) >> p.bs_shift) : 0;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int key = min(kt * BN + s.krow + RSTEP * i, s.Lk - 1);
      int64_t slot;
      if (tile_in_block) {
        slot = int64_t(ublk) * p.bs + (key & (p.bs - 1));
      } else if (p.bs_shift >= 0) {
        slot = int64_t(block_of(p, s.bt_row, key >> p.bs_shift)) * p.bs + (key & (p.bs - 1));
      } else {
        const int lb = key / p.bs;
        slot = int64_t(block_of(p, s.bt_row, lb)) * p.bs + (key - lb * p.bs);
      }
      r.k[i] = *reinterpret_cast<const u32x4*>(s.kbase + slot * s.slot_elems);
      r.v[i] = *reinterpret_cast<const u32x4*>(s.vbase + slot * s.slot_elems);
    }
  } else {
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int key = min(kt * BN + s.krow + RSTEP * i, s.Lk - 1);
      const int64_t row = min(max(s.k_start + key, int64_t(0)), p.num_k_rows - 1);
      r.k[i] = *reinterpret_cast<const u32x4*>(s.kbase + row * p.k_stride);
      r.v[i] = *reinterpret_cast<const u32x4*>(s.vbase + row * p.v_stride);
    }
  }
  return r;
}

template <int CH>
__device__ __forceinline__ void store_tile(const Staged<CH>& st, uint16_t* lk, uint16_t* lv, int tid) {
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const int row = (tid >> 4) + (64 / CH) * i;
    *reinterpret_cast<u32x4*>(&lk[row * KROW + (tid & 15) * 8]) = st.k[i];
    *reinterpret_cast<u32x4*>(&lv[row * VROW + (tid & 15) * 8]) = st.v[i];
  }
}

// G: query heads per kv head; H: query heads per wave (H divides G).  The work-group has 4 x G / H waves:
// wave w takes query tokens 16 (w % 4) .. +16 and heads (w / 4) H .. +H of the group.
template <int G, int H>
__global__ void __launch_bounds__(64 * TOKEN_WAVES * (G / H), 2) prefill_kernel(PrefillKernelArgs p) {
  constexpr int NT = 64 * TOKEN_WAVES * (G / H);
  constexpr int CH = 1024 / NT;
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int tile = p.max_tiles - 1 - int(blockIdx.z);  // heaviest (latest) query tiles are dispatched first
  const int q_start = p.cu_q[b];
  const int Lq = p.cu_q[b + 1] - q_start;
  if (tile * BM >= Lq) return;
  const int64_t k_start = p.cu_k[b];
  int Lk = max(p.cu_k[b + 1] - p.cu_k[b], 0);
  if (p.bt) Lk = min(Lk, p.max_blocks * p.bs);
  const int t0 = tile * BM;
  const int qpos0 = Lk - Lq + t0;  // absolute position of the work-group's first query row
  int kend = p.causal ? min(Lk, qpos0 + BM) : Lk;
  kend = max(kend, 0);
  const int n_tiles = (kend + BN - 1) / BN;

  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][BN * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][BN * VROW];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int tok = t0 + (wave % TOKEN_WAVES) * 16 + col;  // this lane's query token (column of every MFMA block)
  const int hb = (wave / TOKEN_WAVES) * H;                  // first head of the group this wave serves
  const int qpos = Lk - Lq + tok;

  // Q^T operands: head n of the group, dims 32*ks + 8*grp .. +8.  A negative scale is carried by q's sign
  // bits (exact in bf16), so the scale applied to the scores is c = |scale| * log2(e).
  const float c = fabsf(p.scale_log2);
  const uint32_t sign = p.scale_log2 < 0.f ? 0x80008000u : 0u;
  u32x4 qreg[H][4];
  {
    const bool ok = tok < Lq && q_start + tok < p.num_q_tokens;
    const uint16_t* qrow = p.q + int64_t(q_start + tok) * p.q_stride + (int64_t(kvh) * G + hb) * HD + grp * 8;
#pragma unroll
    for (int n = 0; n < H; ++n)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        u32x4 x = ok ? *reinterpret_cast<const u32x4*>(qrow + n * HD + ks * 32) : u32x4{0u, 0u, 0u, 0u};
        x.x ^= sign; x.y ^= sign; x.z ^= sign; x.w ^= sign;
        qreg[n][ks] = x;
      }
  }

  // Staging: thread t moves the 16-byte chunk (t % 16) of key rows t / 16 + 16 i (i < 4) of the K and V tiles.
  // Keys past the end of the sequence read its last key instead (finite data; their scores are masked and
  // their weights are exactly 0), so the loads need no branches.  In paged mode with block_size a multiple
  // of 64 a whole tile lies in one block: one uniform block-table read per tile.
  TileSource src;
  src.kbase = p.k + int64_t(kvh) * HD + (tid & 15) * 8;
  src.vbase = p.v + int64_t(kvh) * HD + (tid & 15) * 8;
  src.bt_row = p.bt ? p.bt + int64_t(b) * p.max_blocks : nullptr;
  src.krow = tid >> 4;
  src.Lk = Lk;
  src.k_start = k_start;
  src.slot_elems = int64_t(p.num_kv_heads) * HD;
  src.khead = p.k + int64_t(kvh) * HD;
  src.vhead = p.v + int64_t(kvh) * HD;
  {
    // Uniform-base path: contiguous rows inside the k rows array, or block_size a multiple of 64; offsets of
    // a 64-row tile must fit 32 bits.
    const int64_t ks = p.bt ? src.slot_elems : p.k_stride, vs = p.bt ? src.slot_elems : p.v_stride;
    src.fast = (!p.bt || p.bs_shift >= 6) && (BN + 1) * max(ks, vs) < (int64_t(1) << 30) &&
               (p.bt || (k_start >= 0 && k_start + Lk <= p.num_k_rows));
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      src.koff[i] = int32_t((src.krow + (64 / CH) * i) * ks + (tid & 15) * 8);
      src.voff[i] = int32_t((src.krow + (64 / CH) * i) * vs + (tid & 15) * 8);
    }
  }
  Staged<CH> st;

  // o_l accumulates the normaliser l = sum of P on the matrix cores, as an extra block of V^T whose first row
  // is all ones: lane (col, grp 0) ends up holding l of query `col` in o_l[n][0].  It is the sum of the same
  // bf16-rounded P that multiplies V, rescaled together with O.
  f32x4_t o[8][H], o_l[H];
  float m[H];
#pragma unroll
  for (int n = 0; n < H; ++n) {
    m[n] = kMinusBig;
    o_l[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t one2 = col == 0 ? 0x3F803F80u : 0u;  // bf16 pair (1, 1) in row 0 of the block, zeros elsewhere
  const u32x4 ones = u32x4{one2, one2, one2, one2};
  // Keys a lane may see: kp <= lim (causal: the query's position; always: the last key).
  const int lim = p.causal ? min(qpos, Lk - 1) : Lk - 1;

  if (n_tiles > 0) {
    st = load_tile<CH>(p, src, 0);
    store_tile(st, lds_k[0], lds_v[0], tid);
  }
  __syncthreads();

  for (int kt = 0; kt < n_tiles; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < n_tiles) st = load_tile<CH>(p, src, kt + 1);

    // S^T = K Q^T for 4 blocks of 16 keys.
    f32x4_t s[4][H];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int n = 0; n < H; ++n) s[kb][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(&lds_k[buf][(kb * 16 + col) * KROW + ks * 32 + grp * 8]);
#pragma unroll
        for (int n = 0; n < H; ++n) s[kb][n] = mfma_16x16x32(a, qreg[n][ks], s[kb][n]);
      }
    }

    // Mask, online softmax.  Lane holds raw scores of keys kt*64 + 16 kb + 4 grp + r for query `tok`; the
    // scale c > 0 is applied inside exp2(s c - m) (q carries the sign of the scale), m is in scaled units.
    const bool need_mask = (kt + 1) * BN > Lk || (p.causal && (kt + 1) * BN - 1 > qpos0);
    if (need_mask) {
      const int room = lim - (kt * BN + grp * 4);  // key kt*64 + 4 grp + 16 kb + r is visible iff 16 kb + r <= room
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const bool vis = kb * 16 + r <= room;
#pragma unroll
          for (int n = 0; n < H; ++n) s[kb][n][r] = vis ? s[kb][n][r] : -INFINITY;
        }
    }
    u32x4 pb[H][2];
    bool grew = false;
    float alpha[H];
#pragma unroll
    for (int n = 0; n < H; ++n) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) mx = fmaxf(mx, s[kb][n][r]);
      mx = max_xor32(max_xor16(mx));
      const float mn = fmaxf(m[n], mx * c);
      alpha[n] = fast_exp2(m[n] - mn);
      grew |= mn > m[n];
      m[n] = mn;
      float pv[4][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int r = 0; r < 4; ++r) pv[kb][r] = fast_exp2(fmaf(s[kb][n][r], c, -mn));
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        pb[n][h].x = pack_bf16x2(pv[2 * h][0], pv[2 * h][1]);
        pb[n][h].y = pack_bf16x2(pv[2 * h][2], pv[2 * h][3]);
        pb[n][h].z = pack_bf16x2(pv[2 * h + 1][0], pv[2 * h + 1][1]);
        pb[n][h].w = pack_bf16x2(pv[2 * h + 1][2], pv[2 * h + 1][3]);
      }
    }
    // Rescale the output only when some running maximum of the wave moved (rare after the first tiles).
    if (__any(grew)) {
#pragma unroll
      for (int n = 0; n < H; ++n) {
        o_l[n] *= alpha[n];
#pragma unroll
        for (int d = 0; d < 8; ++d) o[d][n] *= alpha[n];
      }
    }

    // O^T += V^T P^T.  A operand = V^T: lane (col, grp) needs V[key][16 d + col] for the keys of its P^T slots,
    // {4 grp + j} and {16 + 4 grp + j} (j < 4) of each 32-key half.  ds_read_b64_tr_b16 transposes 16x4 blocks
    // inside each quarter-wave: source lane 4 j + q supplies V[key j][dim0 + 4 q .. + 3] and result lane i
    // receives V[key j][dim0 + i] for j = 0..3.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = h * 32 + grp * 4 + (col >> 2);
      const uint16_t* vrow = &lds_v[buf][row * VROW + (col & 3) * 4];
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const u32x2 lo = ds_read_tr16(vrow + d * 16);
        const u32x2 hi = ds_read_tr16(vrow + 16 * VROW + d * 16);
        const u32x4 a = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int n = 0; n < H; ++n) o[d][n] = mfma_16x16x32(a, pb[n][h], o[d][n]);
      }
#pragma unroll
      for (int n = 0; n < H; ++n) o_l[n] = mfma_16x16x32(ones, pb[n][h], o_l[n]);
    }

    if (kt + 1 < n_tiles) store_tile(st, lds_k[buf ^ 1], lds_v[buf ^ 1], tid);
    __syncthreads();
  }

  // Normalise and write: lane holds dims 16 d + 4 grp + r of query `tok`, head kvh*G + n.
  float inv[H];
#pragma unroll
  for (int n = 0; n < H; ++n) {
    const float lt = __int_as_float(__builtin_amdgcn_ds_bpermute(col << 2, __float_as_int(o_l[n][0])));
    inv[n] = lt > 0.f ? 1.f / lt : 0.f;
  }
  if (tok < Lq && q_start + tok < p.num_q_tokens) {
#pragma unroll
    for (int n = 0; n < H; ++n) {
      uint16_t* orow = p.out + (int64_t(q_start + tok) * p.num_q_heads + kvh * G + hb + n) * HD + grp * 4;
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        u32x2 w;
        w.x = pack_bf16x2(o[d][n][0] * inv[n], o[d][n][1] * inv[n]);
        w.y = pack_bf16x2(o[d][n][2] * inv[n], o[d][n][3] * inv[n]);
        *reinterpret_cast<u32x2*>(orow + d * 16) = w;
      }
    }
  }
}

template <int G, int H>
hipError_t launch_g(const PrefillKernelArgs& p, int batch, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_kernel<G, H>), dim3(p.num_kv_heads, batch, p.max_tiles), dim3(64 * TOKEN_WAVES * (G / H)), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

bool prefill_fast_supported(int head_dim, int group, bool bf16) {
  return bf16 && head_dim == HD && (group == 1 || group == 2 || group == 4);
}

hipError_t launch_prefill_bf16(const AttnArgs& a, hipStream_t stream) {
  PrefillKernelArgs p;
  p.q = static_cast<const uint16_t*>(a.q);
  p.q_stride = a.q_stride;
  p.k = static_cast<const uint16_t*>(a.k);
  p.k_stride = a.k_stride;
  p.v = static_cast<const uint16_t*>(a.v);
  p.v_stride = a.v_stride;
  p.cu_q = a.cu_q;
  p.cu_k = a.cu_k;
  p.bt = a.block_tables;
  p.max_blocks = a.max_blocks;
  p.bs = a.block_size;
  p.bs_shift = (a.block_size & (a.block_size - 1)) == 0 ? __builtin_ctz(unsigned(a.block_size)) : -1;
  p.num_blocks = a.num_blocks;
  p.num_k_rows = a.num_k_rows;
  p.num_q_tokens = a.num_q_tokens;
  p.num_q_heads = a.num_q_heads;
  p.num_kv_heads = a.num_kv_heads;
  p.scale_log2 = a.scale * kLog2e;
  p.causal = a.causal;
  p.max_tiles = (a.max_seqlen_q + BM - 1) / BM;
  p.out = static_cast<uint16_t*>(a.out);
  if (p.max_tiles > 65535) return hipErrorInvalidConfiguration;
  const int group = a.num_q_heads / a.num_kv_heads;
  return group == 1   ? launch_g<1, 1>(p, a.batch, stream)
         : group == 2 ? launch_g<2, PKV_PREFILL_H2>(p, a.batch, stream)
                      : launch_g<4, 2>(p, a.batch, stream);
}

}  // namespace pkv
