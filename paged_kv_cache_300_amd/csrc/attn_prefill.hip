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
//  * GQA groups of 2 with contiguous rows or a paged cache of power-of-two blocks >= 64 and a positive scale go to
//    the 32x32 kernel of attn_prefill_w32.hip instead (same units, same planner); these kernels serve the rest.
#include <math.h>

#include <algorithm>
#include <atomic>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "prefill_common.h"

namespace pkv {
namespace {
using namespace pf;

struct TileSource {
  const uint16_t* khead;  // kv head `kvh` at row / slot 0
  const uint16_t* vhead;
  const int32_t* bt_row;  // PAGED / ROWS: this sequence's block-table row
  int krow;               // first tile row this thread moves
  int Lk;
  int64_t k_start;        // CONTIG: first row of the sequence
  int64_t kstride, vstride;  // elements between consecutive rows (CONTIG) or slots (PAGED / ROWS)
  uint32_t koff[4], voff[4];  // CONTIG / PAGED: byte offsets of this thread's chunks inside a tile
};

template <int CH>
struct Staged {
  u32x4 k[CH], v[CH];
};

// Thread t of NT moves the 16-byte chunk t % 16 of tile rows krow + (NT / 16) i, i < CH = 1024 / NT.
// `blk` is the cache block holding tile kt (PAGED only).
template <int MODE, int CH>
__device__ __forceinline__ Staged<CH> load_tile(const PrefillKernelArgs& p, const TileSource& s, int kt, int blk) {
  constexpr int RSTEP = 64 / CH;
  Staged<CH> r;
  if constexpr (MODE == LOAD_CONTIG || MODE == LOAD_PAGED) {
    int rows = min(s.Lk - kt * BN, BN);
    const uint16_t *kb, *vb;
    if constexpr (MODE == LOAD_PAGED) {
      blk = __builtin_amdgcn_readfirstlane(blk);  // uniform by construction; keeps the tile base in SGPRs
      const int64_t slot0 = int64_t(blk) * p.bs + ((kt * BN) & (p.bs - 1));
      kb = s.khead + slot0 * s.kstride;
      vb = s.vhead + slot0 * s.vstride;
    } else {
      const int64_t row0 = s.k_start + int64_t(kt) * BN;
      rows = row0 < 0 ? 0 : int(min(int64_t(rows), p.num_k_rows - row0));
      kb = s.khead + row0 * s.kstride;
      vb = s.vhead + row0 * s.vstride;
    }
    rows = __builtin_amdgcn_readfirstlane(max(rows, 0));  // uniform; keeps the resource in SGPRs
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(kb, uint32_t(rows) * uint32_t(s.kstride) * 2u);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(vb, uint32_t(rows) * uint32_t(s.vstride) * 2u);
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      r.k[i] = buffer_load16(rk, s.koff[i]);
      r.v[i] = buffer_load16(rv, s.voff[i]);
    }
  } else {
    // Keys past the end of the sequence read its last key (finite; masked, weight exactly 0).  Lk >= 1 here.
    const int chunk = (threadIdx.x & 15) * 8;
#pragma unroll
    for (int i = 0; i < CH; ++i) {
      const int key = min(kt * BN + s.krow + RSTEP * i, s.Lk - 1);
      const int lb = key / p.bs;
      const int64_t slot = int64_t(block_of(p, s.bt_row, lb)) * p.bs + (key - lb * p.bs);
      r.k[i] = *reinterpret_cast<const u32x4*>(s.khead + slot * s.kstride + chunk);
      r.v[i] = *reinterpret_cast<const u32x4*>(s.vhead + slot * s.vstride + chunk);
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


// Flash attention of query tile t of sequence `g` (kv head kvh, its G query heads) against key tiles [kt0, kt1):
// leaves the unnormalised output o, the normaliser (o_l[n][0] of lanes with grp 0) and the reference maximum m.
// Ends with a barrier, so the LDS tiles are free on return.
template <int G, int H, int MODE>
__device__ __forceinline__ void attend_tiles(const PrefillKernelArgs& p, const SeqGeom& g, int b, int kvh, int t,
                                             int kt0, int kt1, uint16_t (*lds_k)[BN * KROW],
                                             uint16_t (*lds_v)[BN * VROW], f32x4_t (&o)[8][H], f32x4_t (&o_l)[H],
                                             float (&m)[H]) {
  constexpr int NT = 64 * TOKEN_WAVES * (G / H);
  constexpr int CH = 1024 / NT;
  const int Lq = g.Lq, Lk = g.Lk, q_start = g.q_start;
  const int t0 = t * BM;
  const int qpos0 = Lk - Lq + t0;  // absolute position of the tile's first query row

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int tok = t0 + (wave % TOKEN_WAVES) * 16 + col;  // this lane's query token (column of every MFMA block)
  const int hb = (wave / TOKEN_WAVES) * H;                  // first head of the group this wave serves
  const int qpos = Lk - Lq + tok;

#pragma unroll
  for (int n = 0; n < H; ++n) {
    m[n] = kMinusBig;
    o_l[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  // No query of the tile sees a key (no keys, or every query before the first key): the output is zero and
  // nothing is read.
  if ((p.causal ? min(Lk, qpos0 + BM) : Lk) <= 0) return;

  // Q^T operands: head n of the group, dims 32*ks + 8*grp .. +8.  A negative scale is carried by q's sign
  // bits (exact in bf16), so the scale applied to the scores is c = |scale| * log2(e) > 0 (a zero scale is
  // taken as the smallest normal float: every weight is then 1 to within rounding, as it should be, and
  // masked scores stay -inf).
  const float c = fmaxf(fabsf(p.scale_log2), 1.17549435e-38f);
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

  // Staging: thread t moves the 16-byte chunk (t % 16) of key rows t / 16 + (64 / CH) i of the K and V tiles.
  TileSource src;
  src.khead = p.k + int64_t(kvh) * HD;
  src.vhead = p.v + int64_t(kvh) * HD;
  src.bt_row = p.bt ? p.bt + int64_t(b) * p.max_blocks : nullptr;
  src.krow = tid >> 4;
  src.Lk = Lk;
  src.k_start = g.k_start;
  src.kstride = p.bt ? int64_t(p.num_kv_heads) * HD : p.k_stride;
  src.vstride = p.bt ? int64_t(p.num_kv_heads) * HD : p.v_stride;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    src.koff[i] = uint32_t(((src.krow + (64 / CH) * i) * src.kstride + (tid & 15) * 8) * 2);
    src.voff[i] = uint32_t(((src.krow + (64 / CH) * i) * src.vstride + (tid & 15) * 8) * 2);
  }
  // PAGED: the block of the next tile to load is read one tile ahead, off the critical path.
  auto tile_block = [&](int kt) { return MODE == LOAD_PAGED ? block_of(p, src.bt_row, (kt * BN) >> p.bs_shift) : 0; };
  Staged<CH> st;

  // o_l accumulates the normaliser l = sum of P on the matrix cores, as an extra block of V^T whose first row
  // is all ones: lane (col, grp 0) ends up holding l of query `col` in o_l[n][0].  It is the sum of the same
  // bf16-rounded P that multiplies V, rescaled together with O.
  const uint32_t one2 = col == 0 ? 0x3F803F80u : 0u;  // bf16 pair (1, 1) in row 0 of the block, zeros elsewhere
  const u32x4 ones = u32x4{one2, one2, one2, one2};
  // Keys a lane may see: kp <= lim (causal: the query's position; always: the last key).
  const int lim = p.causal ? min(qpos, Lk - 1) : Lk - 1;

  int next_blk = 0;
  st = load_tile<MODE, CH>(p, src, kt0, tile_block(kt0));
  if (kt0 + 1 < kt1) next_blk = tile_block(kt0 + 1);
  store_tile(st, lds_k[0], lds_v[0], tid);
  __syncthreads();

  // One key tile.  Scores are formed in two halves of 32 keys; the exponentials of the first half are taken
  // with the current reference maximum while the second half's products are still on the matrix core (redone
  // in the rare tiles where the reference moves), and the second half's exponentials run while the first
  // half's P V products execute, so a wave keeps its matrix core and vector unit busy together.  MASKED:
  // the tile crosses the causal diagonal or the end of the keys (only the last one or two tiles of a row).
  auto tile_step = [&](auto masked_tag, int kt) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int buf = (kt - kt0) & 1;
    if (kt + 1 < kt1) {
      st = load_tile<MODE, CH>(p, src, kt + 1, next_blk);
      if (kt + 2 < kt1) next_blk = tile_block(kt + 2);
    }

    // S^T = K Q^T, keys 0-31 (blocks kb 0, 1) then 32-63 (kb 2, 3).  The wave raises its issue priority for
    // this matrix burst, so that on a SIMD shared with a wave in its softmax the matrix core is fed first
    // (measured +6% at 32 x 2048 non-causal, +15% on ragged prefix batches).
    __builtin_amdgcn_s_setprio(1);
    f32x4_t s[4][H];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int n = 0; n < H; ++n) s[kb][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int half = 0; half < 2; ++half)
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
#pragma unroll
        for (int kb = 2 * half; kb < 2 * half + 2; ++kb) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(&lds_k[buf][(kb * 16 + col) * KROW + ks * 32 + grp * 8]);
#pragma unroll
          for (int n = 0; n < H; ++n) s[kb][n] = mfma_16x16x32(a, qreg[n][ks], s[kb][n]);
        }
      }
    __builtin_amdgcn_s_setprio(0);

    // Lane holds raw scores of keys kt*64 + 16 kb + 4 grp + r for query `tok`; the scale c > 0 is applied
    // inside exp2(s c - m) (q carries the sign of the scale), m is in scaled units.
    if constexpr (MASKED) {
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
    // The reference maximum m only moves when a tile's maximum exceeds it by more than kRescaleSlack (in
    // log2 units), so the weights exp2(s c - m) stay <= 2^kRescaleSlack and the O / l rescale -- a multiply
    // of every accumulator -- is rare after the first tile.  Any reference value gives the same O / l.
    float mxc[H];
    bool need = false;
#pragma unroll
    for (int n = 0; n < H; ++n) {
      // Balanced trees over the lane's 16 scores (short dependency chains), the first half's first.
      float m4[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
        m4[kb] = fmax_ieee(fmax_ieee(s[kb][n][0], s[kb][n][1]), fmax_ieee(s[kb][n][2], s[kb][n][3]));
      const float mx = fmax_ieee(fmax_ieee(m4[0], m4[1]), fmax_ieee(m4[2], m4[3]));
      mxc[n] = max_xor32(max_xor16(mx)) * c;
      need |= mxc[n] > m[n] + kRescaleSlack;
    }
    // First half's weights with the current reference, taken while the second half's products run.  In the
    // rare tiles where the reference moves they are redone: the half's scores are formed again (K and Q are
    // still at hand) and weighted with the new reference, since the old one may lie far below (first tile).
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int n = 0; n < H; ++n)
#pragma unroll
        for (int r = 0; r < 4; ++r) s[kb][n][r] = fast_exp2(fmaf(s[kb][n][r], c, -m[n]));
    if (__any(need)) {
#pragma unroll
      for (int n = 0; n < H; ++n) {
        const float mn = fmaxf(m[n], mxc[n]);
        const float alpha = fast_exp2(m[n] - mn);
        m[n] = mn;
        o_l[n] *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d) o[d][n] *= alpha;
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int n = 0; n < H; ++n) s[kb][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const u32x4 a = *reinterpret_cast<const u32x4*>(&lds_k[buf][(kb * 16 + col) * KROW + ks * 32 + grp * 8]);
#pragma unroll
          for (int n = 0; n < H; ++n) s[kb][n] = mfma_16x16x32(a, qreg[n][ks], s[kb][n]);
        }
      if constexpr (MASKED) {
        const int room = lim - (kt * BN + grp * 4);
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const bool vis = kb * 16 + r <= room;
#pragma unroll
            for (int n = 0; n < H; ++n) s[kb][n][r] = vis ? s[kb][n][r] : -INFINITY;
          }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int n = 0; n < H; ++n)
#pragma unroll
          for (int r = 0; r < 4; ++r) s[kb][n][r] = fast_exp2(fmaf(s[kb][n][r], c, -m[n]));
    }

    // O^T += V^T P^T, one 32-key half at a time.  A operand = V^T: lane (col, grp) needs V[key][16 d + col]
    // for the keys of its P^T slots, {4 grp + j} and {16 + 4 grp + j} (j < 4) of the half.
    // ds_read_b64_tr_b16 transposes 16x4 blocks inside each quarter-wave: source lane 4 j + q supplies
    // V[key j][dim0 + 4 q .. + 3] and result lane i receives V[key j][dim0 + i] for j = 0..3.
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      if (h == 1) {
#pragma unroll
        for (int kb = 2; kb < 4; ++kb)
#pragma unroll
          for (int n = 0; n < H; ++n)
#pragma unroll
            for (int r = 0; r < 4; ++r) s[kb][n][r] = fast_exp2(fmaf(s[kb][n][r], c, -m[n]));
      }
      u32x4 pb[H];
#pragma unroll
      for (int n = 0; n < H; ++n) {
        pb[n].x = pack_bf16x2(s[2 * h][n][0], s[2 * h][n][1]);
        pb[n].y = pack_bf16x2(s[2 * h][n][2], s[2 * h][n][3]);
        pb[n].z = pack_bf16x2(s[2 * h + 1][n][0], s[2 * h + 1][n][1]);
        pb[n].w = pack_bf16x2(s[2 * h + 1][n][2], s[2 * h + 1][n][3]);
      }
      const int row = h * 32 + grp * 4 + (col >> 2);
      const uint16_t* vrow = &lds_v[buf][row * VROW + (col & 3) * 4];
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const u32x2 lo = ds_read_tr16(vrow + d * 16);
        const u32x2 hi = ds_read_tr16(vrow + 16 * VROW + d * 16);
        const u32x4 a = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int n = 0; n < H; ++n) o[d][n] = mfma_16x16x32(a, pb[n], o[d][n]);
      }
#pragma unroll
      for (int n = 0; n < H; ++n) o_l[n] = mfma_16x16x32(ones, pb[n], o_l[n]);
    }

    if (kt + 1 < kt1) store_tile(st, lds_k[buf ^ 1], lds_v[buf ^ 1], tid);
    __syncthreads();
  };

  // Tiles kt >= kt_mask need a mask: (kt + 1) * 64 > Lk, or (causal) (kt + 1) * 64 - 1 > qpos0.
  int kt_mask = Lk / BN;
  if (p.causal) kt_mask = min(kt_mask, qpos0 + 1 > 0 ? (qpos0 + 1) / BN : 0);
  kt_mask = min(max(kt_mask, kt0), kt1);
  for (int kt = kt0; kt < kt_mask; ++kt) tile_step(std::integral_constant<bool, false>(), kt);
  for (int kt = kt_mask; kt < kt1; ++kt) tile_step(std::integral_constant<bool, true>(), kt);
}

// ----------------------------------------------------------------------------------------------------------
// Software-pipelined form of attend_tiles, used for the paged cache: while the matrix core forms the scores
// of key tile j + 1, the vector unit takes the exponentials of tile j (the two interleaved in issue order,
// since a wave issues in order); while it forms O += P_j V_j, the vector unit masks and reduces the maxima of
// tile j + 1.  One wave thus keeps both units busy without relying on the other wave of its SIMD being out of
// phase.  K runs one tile ahead of V in LDS: iteration j reads K_{j+1} and V_j, and stages K_{j+2} and V_{j+1}
// (two buffers each, one barrier per tile).  Measured on prefix-cache batches (16 sequences, prefixes of
// 256-4096 and chunks of 64-512 keys, block size 256): +8-10 % over attend_tiles for GQA groups of 2 with the
// longest-first list, +10 % for groups of 1, +18 % for groups of 4.  On this step's contiguous rows the gain
// and loss by shape were within +-4 %, so that mode keeps attend_tiles.
template <int MODE, int CH, bool IS_V>
__device__ __forceinline__ void load_half(const PrefillKernelArgs& p, const TileSource& s, int kt, int blk,
                                          u32x4 (&r)[CH]) {
  const int64_t stride = IS_V ? s.vstride : s.kstride;
  const uint16_t* head = IS_V ? s.vhead : s.khead;
  int rows = min(s.Lk - kt * BN, BN);
  const uint16_t* base;
  if constexpr (MODE == LOAD_PAGED) {
    blk = __builtin_amdgcn_readfirstlane(blk);
    base = head + (int64_t(blk) * p.bs + ((kt * BN) & (p.bs - 1))) * stride;
  } else {
    const int64_t row0 = s.k_start + int64_t(kt) * BN;
    rows = row0 < 0 ? 0 : int(min(int64_t(rows), p.num_k_rows - row0));
    base = head + row0 * stride;
  }
  rows = __builtin_amdgcn_readfirstlane(max(rows, 0));
  // One resource per row group i (base at row 16 i, size = its valid rows): every lane keeps one offset.
  constexpr int RSTEP = 64 / CH;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(base + int64_t(RSTEP * i) * stride, uint32_t(max(rows - RSTEP * i, 0)) * uint32_t(stride) * 2u);
    r[i] = buffer_load16(rs, IS_V ? s.voff[0] : s.koff[0]);
  }
}

template <int CH>
__device__ __forceinline__ void store_half(const u32x4 (&r)[CH], uint16_t* l, int tid) {
#pragma unroll
  for (int i = 0; i < CH; ++i)
    *reinterpret_cast<u32x4*>(&l[((tid >> 4) + (64 / CH) * i) * KROW + (tid & 15) * 8]) = r[i];
}

template <int H>
__device__ __forceinline__ void scores(const uint16_t* lk, const u32x4 (&qreg)[H][4], int col, int grp,
                                       f32x4_t (&s)[4][H]) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int n = 0; n < H; ++n) s[kb][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const u32x4 a = *reinterpret_cast<const u32x4*>(&lk[(kb * 16 + col) * KROW + ks * 32 + grp * 8]);
#pragma unroll
      for (int n = 0; n < H; ++n) s[kb][n] = mfma_16x16x32(a, qreg[n][ks], s[kb][n]);
    }
}

// Keys kt*64 + 16 kb + 4 grp + r past `lim` get -inf.
template <int H>
__device__ __forceinline__ void mask_scores(f32x4_t (&s)[4][H], int room) {
#pragma unroll
  for (int kb = 0; kb < 4; ++kb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const bool vis = kb * 16 + r <= room;
#pragma unroll
      for (int n = 0; n < H; ++n) s[kb][n][r] = vis ? s[kb][n][r] : -INFINITY;
    }
}

// Row maxima (scaled by c) over the tile, for every lane of the query's column.
template <int H>
__device__ __forceinline__ void tile_max(const f32x4_t (&s)[4][H], float c, float (&mxc)[H]) {
#pragma unroll
  for (int n = 0; n < H; ++n) {
    float m4[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
      m4[kb] = fmax_ieee(fmax_ieee(s[kb][n][0], s[kb][n][1]), fmax_ieee(s[kb][n][2], s[kb][n][3]));
    mxc[n] = max_xor32(max_xor16(fmax_ieee(fmax_ieee(m4[0], m4[1]), fmax_ieee(m4[2], m4[3])))) * c;
  }
}

template <int G, int H, int MODE>
__device__ __forceinline__ void attend_tiles_swp(const PrefillKernelArgs& p, const SeqGeom& g, int b, int kvh, int t,
                                                 int kt1, uint16_t (*lds_k)[BN * KROW],
                                                 uint16_t (*lds_v)[BN * VROW], f32x4_t (&o)[8][H],
                                                 f32x4_t (&o_l)[H], float (&m)[H]) {
  static_assert(MODE != LOAD_ROWS, "row-wise loads use attend_tiles");
  constexpr int NT = 64 * TOKEN_WAVES * (G / H);
  constexpr int CH = 1024 / NT;
  const int Lq = g.Lq, Lk = g.Lk, q_start = g.q_start;
  const int t0 = t * BM;
  const int qpos0 = Lk - Lq + t0;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int tok = t0 + (wave % TOKEN_WAVES) * 16 + col;
  const int hb = (wave / TOKEN_WAVES) * H;
  const int qpos = Lk - Lq + tok;

#pragma unroll
  for (int n = 0; n < H; ++n) {
    m[n] = kMinusBig;
    o_l[n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int d = 0; d < 8; ++d) o[d][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  }
  if ((p.causal ? min(Lk, qpos0 + BM) : Lk) <= 0) return;

  const float c = fmaxf(fabsf(p.scale_log2), 1.17549435e-38f);
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
  TileSource src;
  src.khead = p.k + int64_t(kvh) * HD;
  src.vhead = p.v + int64_t(kvh) * HD;
  src.bt_row = p.bt ? p.bt + int64_t(b) * p.max_blocks : nullptr;
  src.krow = tid >> 4;
  src.Lk = Lk;
  src.k_start = g.k_start;
  src.kstride = p.bt ? int64_t(p.num_kv_heads) * HD : p.k_stride;
  src.vstride = p.bt ? int64_t(p.num_kv_heads) * HD : p.v_stride;
#pragma unroll
  for (int i = 0; i < CH; ++i) {
    src.koff[i] = uint32_t(((src.krow + (64 / CH) * i) * src.kstride + (tid & 15) * 8) * 2);
    src.voff[i] = uint32_t(((src.krow + (64 / CH) * i) * src.vstride + (tid & 15) * 8) * 2);
  }
  auto tile_block = [&](int kt) { return MODE == LOAD_PAGED ? block_of(p, src.bt_row, (kt * BN) >> p.bs_shift) : 0; };
  const uint32_t one2 = col == 0 ? 0x3F803F80u : 0u;
  const u32x4 ones = u32x4{one2, one2, one2, one2};
  const int lim = p.causal ? min(qpos, Lk - 1) : Lk - 1;
  int kt_mask = Lk / BN;
  if (p.causal) kt_mask = min(kt_mask, qpos0 + 1 > 0 ? (qpos0 + 1) / BN : 0);

  // Prologue: K_0, V_0 and K_1 staged; scores and maxima of tile 0.
  u32x4 kst[CH], vst[CH];
  {
    const int blk0 = tile_block(0);
    load_half<MODE, CH, false>(p, src, 0, blk0, kst);
    load_half<MODE, CH, true>(p, src, 0, blk0, vst);
    store_half<CH>(kst, lds_k[0], tid);
    store_half<CH>(vst, lds_v[0], tid);
    if (kt1 > 1) {
      load_half<MODE, CH, false>(p, src, 1, tile_block(1), kst);
      store_half<CH>(kst, lds_k[1], tid);
    }
  }
  __syncthreads();
  f32x4_t sc[4][H];
  scores<H>(lds_k[0], qreg, col, grp, sc);
  if (0 >= kt_mask) mask_scores<H>(sc, lim - grp * 4);
  {
    float mxc[H];
    tile_max<H>(sc, c, mxc);
#pragma unroll
    for (int n = 0; n < H; ++n) m[n] = fmaxf(m[n], mxc[n]);
  }
  if (kt1 > 1) __syncthreads();  // every wave's reads of K_0 are done before K_2 replaces it

  // Weights of the scores in sc (reference m), packed as the P^T operands of the two 32-key halves.
  auto weights = [&](u32x4 (&pb)[2][H]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int n = 0; n < H; ++n) {
        float e[8];
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          e[r] = fast_exp2(fmaf(sc[2 * h][n][r], c, -m[n]));
          e[4 + r] = fast_exp2(fmaf(sc[2 * h + 1][n][r], c, -m[n]));
        }
        pb[h][n] = u32x4{pack_bf16x2(e[0], e[1]), pack_bf16x2(e[2], e[3]), pack_bf16x2(e[4], e[5]),
                         pack_bf16x2(e[6], e[7])};
      }
  };
  // O += P V over tile kt (V in lds_v[kt & 1]); o_l accumulates the normaliser as in attend_tiles.
  auto accumulate = [&](const u32x4 (&pb)[2][H], int kt) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = h * 32 + grp * 4 + (col >> 2);
      const uint16_t* vrow = &lds_v[kt & 1][row * VROW + (col & 3) * 4];
#pragma unroll
      for (int d = 0; d < 8; ++d) {
        const u32x2 lo = ds_read_tr16(vrow + d * 16);
        const u32x2 hi = ds_read_tr16(vrow + 16 * VROW + d * 16);
        const u32x4 a = u32x4{lo.x, lo.y, hi.x, hi.y};
#pragma unroll
        for (int n = 0; n < H; ++n) o[d][n] = mfma_16x16x32(a, pb[h][n], o[d][n]);
      }
#pragma unroll
      for (int n = 0; n < H; ++n) o_l[n] = mfma_16x16x32(ones, pb[h][n], o_l[n]);
    }
  };

  // Steady state: tile kt + 1 exists.  Loads past the last tile (K_{kt+2} near the end) have zero valid rows:
  // they read nothing and stage zeros into a buffer no one reads.  MASKED: tile kt + 1 needs the mask.
  const int last_lb = p.bt ? p.max_blocks - 1 : 0;
  auto step = [&](auto masked_tag, int kt) {
    constexpr bool MASKED = decltype(masked_tag)::value;
    const int blk2 = MODE == LOAD_PAGED ? block_of(p, src.bt_row, min(((kt + 2) * BN) >> p.bs_shift, last_lb)) : 0;
    load_half<MODE, CH, false>(p, src, kt + 2, blk2, kst);
    // A: scores of tile kt + 1 on the matrix core, weights of tile kt on the vector unit.
    f32x4_t sn[4][H];
    u32x4 pb[2][H];
    // Sixteen groups, each: the H products of one (ks, kb) K fragment, then 8 H / 16 pairs of weights, in that
    // issue order (scheduling barriers between groups); K fragments are read two groups ahead.
    {
      const uint16_t* lk = lds_k[(kt + 1) & 1];
      auto kfrag = [&](int i) {
        return *reinterpret_cast<const u32x4*>(&lk[((i & 3) * 16 + col) * KROW + (i >> 2) * 32 + grp * 8]);
      };
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int n = 0; n < H; ++n) sn[kb][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      u32x4 kf[3];
      kf[0] = kfrag(0);
      kf[1] = kfrag(1);
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        if (i + 2 < 16) kf[(i + 2) % 3] = kfrag(i + 2);
#pragma unroll
        for (int n = 0; n < H; ++n) sn[i & 3][n] = mfma_16x16x32(kf[i % 3], qreg[n][i >> 2], sn[i & 3][n]);
#pragma unroll
        for (int cidx = i * H / 2; cidx < (i + 1) * H / 2; ++cidx) {
          const int h = cidx / (4 * H), n = (cidx / 4) % H, j = cidx % 4;
          const int kbs = 2 * h + (j >> 1), r0 = (j & 1) * 2;
          const float e0 = fast_exp2(fmaf(sc[kbs][n][r0], c, -m[n]));
          const float e1 = fast_exp2(fmaf(sc[kbs][n][r0 + 1], c, -m[n]));
          pb[h][n][j] = pack_bf16x2(e0, e1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    // K_{kt+2} replaces K_kt (last read in the previous tile); V_{kt+1} is fetched now and replaces V_{kt-1}
    // (also read in the previous tile), so each staging set is live for half a tile only.
    store_half<CH>(kst, lds_k[kt & 1], tid);
    load_half<MODE, CH, true>(p, src, kt + 1, tile_block(kt + 1), vst);
    // B: O += P V of tile kt on the matrix core, mask and maxima of tile kt + 1 on the vector unit.
    if constexpr (MASKED) mask_scores<H>(sn, lim - ((kt + 1) * BN + grp * 4));
    accumulate(pb, kt);
    float mxc[H];
    tile_max<H>(sn, c, mxc);
    bool need = false;
#pragma unroll
    for (int n = 0; n < H; ++n) need |= mxc[n] > m[n] + kRescaleSlack;
    if (__any(need)) {
#pragma unroll
      for (int n = 0; n < H; ++n) {
        const float mn = fmaxf(m[n], mxc[n]);
        const float alpha = fast_exp2(m[n] - mn);
        m[n] = mn;
        o_l[n] *= alpha;
#pragma unroll
        for (int d = 0; d < 8; ++d) o[d][n] *= alpha;
      }
    }
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int n = 0; n < H; ++n) sc[kb][n] = sn[kb][n];
    store_half<CH>(vst, lds_v[(kt + 1) & 1], tid);
    __syncthreads();
  };
  // Tile kt + 1 needs no mask while kt + 1 < kt_mask.
  const int split = min(max(kt_mask - 1, 0), kt1 - 1);
  for (int kt = 0; kt < split; ++kt) step(std::integral_constant<bool, false>(), kt);
  for (int kt = split; kt < kt1 - 1; ++kt) step(std::integral_constant<bool, true>(), kt);
  // Last tile: weights and O += P V only.
  {
    u32x4 pb[2][H];
    weights(pb);
    accumulate(pb, kt1 - 1);
    __syncthreads();
  }
}

// Normalise and write: lane holds dims 16 d + 4 grp + r of query `tok`, head kvh*G + hb + n.
template <int G, int H>
__device__ __forceinline__ void write_output(const PrefillKernelArgs& p, const SeqGeom& g, int kvh, int t,
                                             const f32x4_t (&o)[8][H], const f32x4_t (&o_l)[H]) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp = lane >> 4;
  const int tok = t * BM + (wave % TOKEN_WAVES) * 16 + col;
  const int hb = (wave / TOKEN_WAVES) * H;
  float inv[H];
#pragma unroll
  for (int n = 0; n < H; ++n) {
    const float lt = __int_as_float(__builtin_amdgcn_ds_bpermute(col << 2, __float_as_int(o_l[n][0])));
    inv[n] = lt > 0.f ? 1.f / lt : 0.f;
  }
  if (tok < g.Lq && g.q_start + tok < p.num_q_tokens) {
#pragma unroll
    for (int n = 0; n < H; ++n) {
      uint16_t* orow = p.out + (int64_t(g.q_start + tok) * p.num_q_heads + kvh * G + hb + n) * HD + grp * 4;
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

// G: query heads per kv head; H: query heads per wave (H divides G).  The work-group has 4 x G / H waves:
// wave w takes query tokens 16 (w % 4) .. +16 and heads (w / 4) H .. +H of the group.
// Grid form: one work-group per (kv head, sequence, query tile), heaviest (latest) query tiles dispatched first.
template <int G, int H, int MODE>
__global__ void __launch_bounds__(64 * TOKEN_WAVES * (G / H), 2) prefill_kernel(PrefillKernelArgs p) {
  const int kvh = blockIdx.x, b = blockIdx.y;
  const int t = p.max_tiles - 1 - int(blockIdx.z);
  const SeqGeom g = seq_geom(p, b);
  if (t >= g.T) return;
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][BN * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][BN * VROW];
  f32x4_t o[8][H], o_l[H];
  float m[H];
  if constexpr (MODE == LOAD_PAGED)
    attend_tiles_swp<G, H, MODE>(p, g, b, kvh, t, unit_tiles(g, t), lds_k, lds_v, o, o_l, m);
  else
    attend_tiles<G, H, MODE>(p, g, b, kvh, t, 0, unit_tiles(g, t), lds_k, lds_v, o, o_l, m);
  write_output<G, H>(p, g, kvh, t, o, o_l);
}

// Longest-first order.  When the work of a query tile is not given by its index (cached prefixes of different
// lengths, non-causal rows), a one-work-group planner lists the (sequence, query tile) units by key-tile count,
// largest first, and the ordered kernel takes unit `rank` = its launch index / Hkv: the hardware hands out work-
// groups in launch order, so the longest rows start first and the short ones fill the tail (greedy
// longest-processing-time scheduling, with no communication between work-groups).
constexpr int PLAN_THREADS = 256;
constexpr int PLAN_MAX_BATCH = 4096;
constexpr int PLAN_BUCKETS = 4096;  // at most; units with more key tiles share the last bucket
constexpr size_t PLAN_HEADER_BYTES = 256;

struct PlanArgs {
  int batch;
  int buckets;   // key-tile counts 1 .. buckets (larger counts share the last), from max_seqlen_k
  int unit_cap;  // list capacity; units past it are dropped (the host sizes it from num_q_tokens)
  void* list;    // [unit_cap] (sequence, query tile) entries, longest first
  int* count;    // number of listed units; the 32x32 form also writes count[1] = 0 splits, count[2] = 1 (listed)
};

// A listed unit: (sequence, tile) for the 16x16 kernels, a whole-unit piece for the 32x32 kernel.
__device__ __forceinline__ void put_unit(int2* list, int i, int b, int t) { list[i] = make_int2(b, t); }
__device__ __forceinline__ void put_unit(PrefillPiece* list, int i, int b, int t) {
  list[i] = PrefillPiece{b, t, 0, -1, -1, 0, 0, 0};
}

// Exclusive prefix sum of a[0 .. n) in place; returns the total.  All threads call it.
__device__ int block_exclusive_scan(int* a, int n, int* chunk) {
  const int tid = threadIdx.x;
  const int per = (n + PLAN_THREADS - 1) / PLAN_THREADS;
  const int c_beg = min(tid * per, n), c_end = min(c_beg + per, n);
  int acc = 0;
  for (int i = c_beg; i < c_end; ++i) acc += a[i];
  chunk[tid] = acc;
  __syncthreads();
  for (int off = 1; off < PLAN_THREADS; off <<= 1) {
    const int x = tid >= off ? chunk[tid - off] : 0;
    __syncthreads();
    chunk[tid] += x;
    __syncthreads();
  }
  const int total = chunk[PLAN_THREADS - 1];
  acc = tid > 0 ? chunk[tid - 1] : 0;
  for (int i = c_beg; i < c_end; ++i) {
    const int x = a[i];
    a[i] = acc;
    acc += x;
  }
  __syncthreads();
  return total;
}

template <typename Entry>
__global__ void __launch_bounds__(PLAN_THREADS) prefill_plan_kernel(PrefillKernelArgs p, PlanArgs pa) {
  __shared__ int uoff[PLAN_MAX_BATCH + 1];  // first unit of each sequence
  __shared__ int sc0[PLAN_MAX_BATCH], snk[PLAN_MAX_BATCH];
  __shared__ int start[PLAN_BUCKETS];       // bucket i holds units with `buckets` - i key tiles (clamped)
  __shared__ int chunk[PLAN_THREADS];
  const int tid = threadIdx.x, nb = pa.batch, nbk = pa.buckets;
  for (int b = tid; b < nb; b += PLAN_THREADS) {
    const SeqGeom g = seq_geom(p, b);
    const int T = min(g.T, p.max_tiles);  // rows past max_seqlen_q are not computed
    uoff[b] = T;
    sc0[b] = g.c0;
    snk[b] = g.NKe;
  }
  for (int i = tid; i < nbk; i += PLAN_THREADS) start[i] = 0;
  __syncthreads();
  const int units = min(block_exclusive_scan(uoff, nb, chunk), pa.unit_cap);
  if (tid == 0) uoff[nb] = units;
  __syncthreads();
  // Unit u -> (sequence, tile, bucket).
  auto locate = [&](int u, int& b, int& t) {
    int lo = 0, hi = nb - 1;  // last b with uoff[b] <= u
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (uoff[mid] <= u) lo = mid; else hi = mid - 1;
    }
    b = lo;
    t = u - uoff[lo];
    const int nk = min(max(t + 1 + sc0[lo], 1), snk[lo]);
    return nbk - min(nk, nbk);
  };
  for (int u = tid; u < units; u += PLAN_THREADS) {
    int b, t;
    atomicAdd(&start[locate(u, b, t)], 1);
  }
  __syncthreads();
  block_exclusive_scan(start, nbk, chunk);
  for (int u = tid; u < units; u += PLAN_THREADS) {
    int b, t;
    const int slot = atomicAdd(&start[locate(u, b, t)], 1);
    put_unit(static_cast<Entry*>(pa.list), slot, b, t);
  }
  if (tid == 0) {
    pa.count[0] = units;
    if constexpr (!std::is_same<Entry, int2>::value) {
      pa.count[1] = 0;
      pa.count[2] = 1;
    }
  }
}

// Splitting planner for the 32x32 kernel.  A query tile's keys are a chain of key tiles that one work-group walks
// in order; when the longest chains are much longer than the share of work each resident work-group gets, they
// set the kernel's length.  With W the batch's key tiles over all units and S the work-groups the device holds at
// once, P = max(kPieceMin, ceil(W Hkv / S)) is that share: a unit of nk > P key tiles is cut into ceil(nk / P)
// pieces of (nearly) equal length whose partial softmax states the merge kernel combines, and the pieces are listed
// longest first.  Bounds that size the workspace: every split unit has nk > P, so there are fewer than W / P <= S /
// Hkv of them, the extra pieces number fewer than W / P, and the partial slots (pieces of split units) fewer than
// 2 S / Hkv.  The host runs it only where whole units cannot fill half of the resident work-groups (few query
// tiles over long keys: a chunk of new tokens on a long cached prefix); elsewhere the merge's extra launch and
// partial-state traffic cost more than the balance gains, and the units run whole.
constexpr int kPieceMin = 16;

struct SplitPlanArgs {
  int batch;
  int buckets;    // piece lengths 1 .. buckets (longer ones share the last)
  int unit_cap;   // units the workspace was sized for (units past it are dropped)
  int list_cap;   // pieces that fit the list
  int split_cap;  // split units that fit the split list (their partial slots: 2 split_cap)
  int slots;      // work-groups resident at once
  PrefillPiece* list;
  PrefillSplit* splits;
  int* hdr;       // [0] pieces listed, [1] split units, [2] 1: listed order, 0: grid order
};

__global__ void __launch_bounds__(PLAN_THREADS) prefill_split_plan_kernel(PrefillKernelArgs p, SplitPlanArgs pa) {
  __shared__ int uoff[PLAN_MAX_BATCH + 1];  // first unit of each sequence
  __shared__ int sc0[PLAN_MAX_BATCH], snk[PLAN_MAX_BATCH];
  __shared__ int start[PLAN_BUCKETS];       // bucket i holds pieces of `buckets` - i key tiles (clamped)
  __shared__ int chunk[PLAN_THREADS];
  __shared__ unsigned long long s_w[PLAN_THREADS / 64];
  __shared__ int s_pieces, s_split, s_parts, s_sid, s_pbase;
  const int tid = threadIdx.x, nb = pa.batch, nbk = pa.buckets;
  for (int b = tid; b < nb; b += PLAN_THREADS) {
    const SeqGeom g = seq_geom(p, b);
    uoff[b] = min(g.T, p.max_tiles);  // rows past max_seqlen_q are not computed
    sc0[b] = g.c0;
    snk[b] = g.NKe;
  }
  for (int i = tid; i < nbk; i += PLAN_THREADS) start[i] = 0;
  if (tid == 0) s_pieces = s_split = s_parts = s_sid = s_pbase = 0;
  __syncthreads();
  const int units = min(block_exclusive_scan(uoff, nb, chunk), pa.unit_cap);
  if (tid == 0) uoff[nb] = units;
  __syncthreads();
  // Unit u -> (sequence, tile) and its key-tile count.
  auto locate = [&](int u, int& b, int& t) {
    int lo = 0, hi = nb - 1;  // last b with uoff[b] <= u
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (uoff[mid] <= u) lo = mid; else hi = mid - 1;
    }
    b = lo;
    t = u - uoff[lo];
    return min(max(t + 1 + sc0[lo], 1), snk[lo]);
  };
  {
    unsigned long long w = 0;
    for (int u = tid; u < units; u += PLAN_THREADS) {
      int b, t;
      w += unsigned(locate(u, b, t));
    }
    // the total over the work-group: wave sums by lane shuffles, then one value per wave
    for (int off = 32; off >= 1; off >>= 1) {
      const unsigned lo = __shfl_xor(unsigned(w), off), hi = __shfl_xor(unsigned(w >> 32), off);
      w += (static_cast<unsigned long long>(hi) << 32) | lo;
    }
    if ((tid & 63) == 0) s_w[tid >> 6] = w;
  }
  __syncthreads();
  unsigned long long wsum = 0;
#pragma unroll
  for (int i = 0; i < PLAN_THREADS / 64; ++i) wsum += s_w[i];
  const unsigned long long share = (wsum * unsigned(p.num_kv_heads) + unsigned(pa.slots) - 1) / unsigned(pa.slots);
  const int P = int(min(max(share, (unsigned long long)kPieceMin), (unsigned long long)INT32_MAX));
  auto npieces = [&](int nk) { return nk > P ? int((int64_t(nk) + P - 1) / P) : 1; };
  // first key tile of piece k of np (k = np: the end); 64-bit products for the longest key ranges
  auto cut_at = [](int k, int nk, int np) { return int(int64_t(k) * nk / np); };
  auto bucket = [&](int len) { return nbk - min(len, nbk); };
  bool listed = true;
  {  // counting pass
    for (int u = tid; u < units; u += PLAN_THREADS) {
      int b, t;
      const int nk = locate(u, b, t), np = npieces(nk);
      for (int k = 0; k < np; ++k) atomicAdd(&start[bucket(cut_at(k + 1, nk, np) - cut_at(k, nk, np))], 1);
      atomicAdd(&s_pieces, np);
      if (np > 1) {
        atomicAdd(&s_split, 1);
        atomicAdd(&s_parts, np);
      }
    }
    __syncthreads();
    // The bounds above guarantee these fit; the check keeps an inconsistent sizing from writing past the lists.
    listed = s_pieces <= pa.list_cap && s_split <= pa.split_cap && s_parts <= 2 * pa.split_cap;
  }
  if (!listed) {
    if (tid == 0) {
      pa.hdr[0] = 0;
      pa.hdr[1] = 0;
      pa.hdr[2] = 0;
    }
    return;
  }
  block_exclusive_scan(start, nbk, chunk);
  for (int u = tid; u < units; u += PLAN_THREADS) {
    int b, t;
    const int nk = locate(u, b, t), np = npieces(nk);
    int pbase = -1;
    if (np > 1) {
      const int sid = atomicAdd(&s_sid, 1);
      pbase = atomicAdd(&s_pbase, np);
      pa.splits[sid] = PrefillSplit{b, t, np, pbase};
    }
    for (int k = 0; k < np; ++k) {
      const int k0 = cut_at(k, nk, np), k1 = cut_at(k + 1, nk, np);
      const int pos = atomicAdd(&start[bucket(k1 - k0)], 1);
      pa.list[pos] = PrefillPiece{b, t, k0, k1, np > 1 ? pbase + k : -1, 0, 0, 0};
    }
  }
  if (tid == 0) {
    pa.hdr[0] = s_pieces;
    pa.hdr[1] = s_split;
    pa.hdr[2] = 1;
  }
}

template <int G, int H, int MODE>
__global__ void __launch_bounds__(64 * TOKEN_WAVES * (G / H), 2)
    prefill_ordered_kernel(PrefillKernelArgs p, const int2* list, const int* count) {
  const int kvh = int(blockIdx.x % unsigned(p.num_kv_heads));
  const int rank = int(blockIdx.x / unsigned(p.num_kv_heads));
  if (rank >= *count) return;
  const int2 u = list[rank];
  const SeqGeom g = seq_geom(p, u.x);
  __shared__ __attribute__((aligned(16))) uint16_t lds_k[2][BN * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t lds_v[2][BN * VROW];
  f32x4_t o[8][H], o_l[H];
  float m[H];
  if constexpr (MODE == LOAD_PAGED)
    attend_tiles_swp<G, H, MODE>(p, g, u.x, kvh, u.y, unit_tiles(g, u.y), lds_k, lds_v, o, o_l, m);
  else
    attend_tiles<G, H, MODE>(p, g, u.x, kvh, u.y, 0, unit_tiles(g, u.y), lds_k, lds_v, o, o_l, m);
  write_output<G, H>(p, g, kvh, u.y, o, o_l);
}

template <int G, int H>
hipError_t launch_g(const PrefillKernelArgs& p, int batch, int mode, const PlanArgs* plan, hipStream_t stream) {
  constexpr int NT = 64 * TOKEN_WAVES * (G / H);
  if (plan) {
    hipLaunchKernelGGL(prefill_plan_kernel<int2>, dim3(1), dim3(PLAN_THREADS), 0, stream, p, *plan);
    const dim3 grid(unsigned(plan->unit_cap) * unsigned(p.num_kv_heads));
    const int2* list = static_cast<const int2*>(plan->list);
    if (mode == LOAD_CONTIG)
      hipLaunchKernelGGL((prefill_ordered_kernel<G, H, LOAD_CONTIG>), grid, dim3(NT), 0, stream, p, list,
                         plan->count);
    else if (mode == LOAD_PAGED)
      hipLaunchKernelGGL((prefill_ordered_kernel<G, H, LOAD_PAGED>), grid, dim3(NT), 0, stream, p, list,
                         plan->count);
    else
      hipLaunchKernelGGL((prefill_ordered_kernel<G, H, LOAD_ROWS>), grid, dim3(NT), 0, stream, p, list,
                         plan->count);
    return hipGetLastError();
  }
  const dim3 grid(p.num_kv_heads, batch, p.max_tiles), block(NT);
  if (mode == LOAD_CONTIG)
    hipLaunchKernelGGL((prefill_kernel<G, H, LOAD_CONTIG>), grid, block, 0, stream, p);
  else if (mode == LOAD_PAGED)
    hipLaunchKernelGGL((prefill_kernel<G, H, LOAD_PAGED>), grid, block, 0, stream, p);
  else
    hipLaunchKernelGGL((prefill_kernel<G, H, LOAD_ROWS>), grid, block, 0, stream, p);
  return hipGetLastError();
}

int load_mode(const AttnArgs& a) {
  if (!a.block_tables) return LOAD_CONTIG;
  const int64_t row_elems = int64_t(a.num_kv_heads) * HD;
  const bool pow2_64 = a.block_size >= 64 && (a.block_size & (a.block_size - 1)) == 0;
  return pow2_64 && int64_t(BN) * row_elems * 2 < (int64_t(1) << 31) ? LOAD_PAGED : LOAD_ROWS;
}

// Upper bound on the (sequence, query tile) units: every sequence has at most one partial tile.
int64_t unit_cap(int batch, int num_q_tokens, int max_seqlen_q) {
  const int64_t by_tokens = (int64_t(num_q_tokens) + BM - 1) / BM + batch;
  const int64_t by_max = int64_t(batch) * ((int64_t(max_seqlen_q) + BM - 1) / BM);
  return std::min(by_tokens, by_max);
}

}  // namespace

bool prefill_fast_supported(int head_dim, int group, bool bf16) {
  return bf16 && head_dim == HD && (group == 1 || group == 2 || group == 4);
}

bool prefill_fast_strides_ok(int64_t k_stride, int64_t v_stride) {
  return int64_t(BN) * max(k_stride, v_stride) * 2 < (int64_t(1) << 31);
}

namespace {

// Work-groups of the 32x32 kernel the current device holds at once (cached per device; several host threads may
// ask at once and store equal values).
int w32_slots() {
  static std::atomic<int> cached[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  if (const int v = cached[dev].load(std::memory_order_relaxed); v > 0) return v;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) cus = 256;
  const int v = cus * kW32PerCU;
  cached[dev].store(v, std::memory_order_relaxed);
  return v;
}

size_t align256(size_t x) { return (x + 255) & ~size_t(255); }

// Workspace of the planners: a header, then the piece list (the 16x16 planner's (sequence, tile) list uses its
// start), the split list and the partial states of the pieces of split units.
struct PlanLayout {
  int unit_cap, split_cap, list_cap;
  size_t list, splits, parts, total;
};
PlanLayout plan_layout(int batch, int num_q_tokens, int max_seqlen_q, int num_kv_heads) {
  PlanLayout L{};
  const int64_t cap = unit_cap(batch, num_q_tokens, max_seqlen_q);
  if (batch < 1 || batch > PLAN_MAX_BATCH || num_kv_heads < 1 || cap < 1) return L;
  const int split_cap = w32_slots() / num_kv_heads + 1;
  if ((cap + split_cap) * num_kv_heads > INT32_MAX) return L;
  L.unit_cap = int(cap);
  L.split_cap = split_cap;
  L.list_cap = int(cap) + split_cap;
  L.list = PLAN_HEADER_BYTES;
  L.splits = align256(L.list + size_t(L.list_cap) * sizeof(PrefillPiece));
  L.parts = align256(L.splits + size_t(split_cap) * sizeof(PrefillSplit));
  L.total = L.parts + size_t(2 * split_cap) * size_t(num_kv_heads) * kPartialFloat4 * sizeof(f32x4_t);
  return L;
}

}  // namespace

size_t prefill_workspace_bytes(int batch, int num_q_tokens, int max_seqlen_q, int num_kv_heads) {
  return plan_layout(batch, num_q_tokens, max_seqlen_q, num_kv_heads).total;
}

bool prefill_wants_split(const AttnArgs& a) {
  // 32x32 kernel: the (sequence, query tile) units cannot fill half of the resident work-groups, and some unit
  // may be longer than the shortest piece.  With at most U units the longest chain is at least S / (U Hkv) times
  // the even share, so at U Hkv <= S / 2 splitting at least halves the kernel's critical path.
  const int group = a.num_q_heads / a.num_kv_heads;
  if (!prefill_w32_supported(group, load_mode(a), a.scale)) return false;
  const int64_t units = unit_cap(a.batch, a.num_q_tokens, a.max_seqlen_q);
  return units * a.num_kv_heads * 2 <= w32_slots() && (int64_t(std::max(a.max_seqlen_k, 0)) + BN - 1) / BN > kPieceMin;
}

bool prefill_wants_plan(const AttnArgs& a) { return prefill_wants_split(a) || prefill_wants_order(a); }

bool prefill_wants_order(const AttnArgs& a) {
  // Cached prefixes of different lengths or non-causal rows: a query tile's work is not given by its index.
  if (a.block_tables != nullptr || !a.causal || a.max_seqlen_k != a.max_seqlen_q) return true;
  // Causal self-attention over this step's own tokens: a tile's work grows with its index, so the grid's
  // latest-tile-first launch order already is longest-first -- but the grid holds batch x ceil(max_seqlen_q /
  // 64) work-groups per kv head, and when the lengths vary enough that a tenth of them would find no tile
  // (they still cost a dispatch each), the listed order is worth its planner.
  const int64_t grid_tiles = int64_t(a.batch) * ((int64_t(a.max_seqlen_q) + BM - 1) / BM);
  const int64_t real_tiles_max = (int64_t(a.num_q_tokens) + BM - 1) / BM + a.batch;
  return real_tiles_max * 10 < grid_tiles * 9;
}

hipError_t launch_prefill_bf16(const AttnArgs& a, void* workspace, size_t workspace_bytes, hipStream_t stream) {
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
  if (!a.block_tables && !prefill_fast_strides_ok(a.k_stride, a.v_stride)) return hipErrorInvalidValue;
  const int mode = load_mode(a);
  const int group = a.num_q_heads / a.num_kv_heads;
  PlanArgs plan{};
  const PlanArgs* planp = nullptr;
  const PlanLayout L = plan_layout(a.batch, a.num_q_tokens, a.max_seqlen_q, a.num_kv_heads);
  const bool planned = workspace && L.total > 0 && workspace_bytes >= L.total;
  char* const ws = static_cast<char*>(workspace);
  const int buckets = int(std::min<int64_t>(PLAN_BUCKETS, (int64_t(std::max(a.max_seqlen_k, 0)) + BN - 1) / BN + 1));
  if (planned) {
    plan.batch = a.batch;
    plan.buckets = buckets;
    plan.unit_cap = L.unit_cap;
    plan.count = reinterpret_cast<int*>(ws);
    plan.list = ws + L.list;
    planp = &plan;
  } else if (p.max_tiles > 65535) {
    return hipErrorInvalidConfiguration;
  }
#ifndef PKV_PREFILL_16X16_ONLY
  if (prefill_w32_supported(group, mode, a.scale)) {
    if (!planned) return launch_prefill_w32(p, a.batch, mode, PieceList{}, 0, 0, stream);
    PieceList pl{reinterpret_cast<PrefillPiece*>(ws + L.list), reinterpret_cast<int*>(ws),
                 reinterpret_cast<PrefillSplit*>(ws + L.splits), reinterpret_cast<f32x4_t*>(ws + L.parts)};
    if (!prefill_wants_split(a)) {
      if (!prefill_wants_order(a)) return launch_prefill_w32(p, a.batch, mode, PieceList{}, 0, 0, stream);
      hipLaunchKernelGGL(prefill_plan_kernel<PrefillPiece>, dim3(1), dim3(PLAN_THREADS), 0, stream, p, plan);
      return launch_prefill_w32(p, a.batch, mode, pl, L.unit_cap, 0, stream);
    }
    SplitPlanArgs sp{};
    sp.batch = a.batch;
    sp.buckets = buckets;
    sp.unit_cap = L.unit_cap;
    sp.list_cap = L.list_cap;
    sp.split_cap = L.split_cap;
    sp.slots = std::max(1, std::min(w32_slots(), (L.split_cap - 1) * a.num_kv_heads));
    sp.list = reinterpret_cast<PrefillPiece*>(ws + L.list);
    sp.splits = reinterpret_cast<PrefillSplit*>(ws + L.splits);
    sp.hdr = reinterpret_cast<int*>(ws);
    hipLaunchKernelGGL(prefill_split_plan_kernel, dim3(1), dim3(PLAN_THREADS), 0, stream, p, sp);
    // Grid: the longer of the listed pieces and the grid order (the planner's fallback when its lists would
    // overflow, which the workspace bounds rule out).
    const int64_t grid_units = std::max<int64_t>(L.list_cap, int64_t(a.batch) * p.max_tiles);
    if (grid_units > INT32_MAX) return hipErrorInvalidConfiguration;
    return launch_prefill_w32(p, a.batch, mode, pl, int(grid_units), L.split_cap, stream);
  }
#endif
  if (planp && !prefill_wants_order(a)) planp = nullptr;
  if (!planp && p.max_tiles > 65535) return hipErrorInvalidConfiguration;
  return group == 1   ? launch_g<1, 1>(p, a.batch, mode, planp, stream)
         : group == 2 ? launch_g<2, PKV_PREFILL_H2>(p, a.batch, mode, planp, stream)
                      : launch_g<4, 2>(p, a.batch, mode, planp, stream);
}

}  // namespace pkv
