// Varlen (causal) prefill attention for GQA groups of 2 on gfx950 32x32x16 bf16 MFMA, 32 query rows per wave.
//
// What it computes is the same as attn_prefill.hip [P2 §5.3; P3 §4; P1 Q6 §3]: for sequence b, query head h and
// query row i at absolute position Lk - Lq + i, o = softmax(scale * q K^T) V over keys 0 .. Lk - Lq + i (causal)
// or all Lk keys, K/V from this step's rows or through the block table; query head h reads kv head h / 2 [P2 §3].
//
// How (FlashAttention tiling and online softmax [P2 §5.2], shaped for the gfx950 SIMD):
//  * A work-group owns 64 query tokens of one sequence and one kv head with both query heads that read it; its 4
//    waves own 32 tokens x 1 head each.  Three work-groups share a CU (48 KB of LDS and at most 168 VGPRs each), so
//    every SIMD runs three waves: while one takes its exponentials the others keep the matrix core busy.  32x32x16
//    products matter there: from a single wave a chain of 16x16x32 products falls well short of the matrix-core
//    rate, a chain of 32x32x16 products does not, so the matrix core keeps issuing while another wave is in its
//    vector phase.
//  * Scores are transposed, S^T = K Q^T: Q^T (the B operand) stays in registers; lane (j, half) of a 32x32 block
//    holds 16 keys of query j, so P^T feeds O^T = V^T P^T straight from registers (the contraction order of the
//    keys is permuted alike on both operands), and V^T comes from LDS through the transposing ds_read_b64_tr_b16.
//  * K/V tiles of 64 keys reach LDS by direct-to-LDS buffer loads (no staging registers): lane i of a load lands
//    at 16 i bytes past the wave's base, so each lane fetches the global chunk that the row's swizzle puts there.
//    Rows past the end of the keys read as zeros (buffer bounds).  K rows are swizzled by r & 15 and V rows by
//    4 (r & 3), which makes the 16-byte K reads and the transposing V reads free of bank conflicts.  Two K
//    buffers and one V buffer: in step kt the K loads of tile kt + 2 go into K tile kt's buffer once every wave
//    has formed its last scores from it (barrier A, which also waits for the loads in flight), and the V loads of
//    tile kt + 1 into the V buffer once every wave has finished its P V products (barrier B).  The waits this
//    leaves are covered by the CU's other two work-groups.
//  * Per tile, software-pipelined in two halves of 32 keys: the scores of the next half are formed on the matrix
//    core while the vector unit takes the exponentials of the current half, then O += P V of the current half runs
//    while the next half's mask and row maxima are reduced.  The online-softmax reference maximum moves only when
//    a half's maximum exceeds it by more than 2^8, so the rescale of the 64 output registers is rare; the
//    normaliser sums the packed bf16 weights (the same values P V multiplies) with one dot product per pair.
#include <math.h>

#include <algorithm>
#include <type_traits>

#include "common.h"
#include "launch.h"
#include "prefill_common.h"
#include "prefill_mfma32.h"

namespace pkv {
namespace {
using namespace pf;

constexpr int NBUF = 3;  // K0, K1, V
#ifndef PKV_W32_CHUNK
#define PKV_W32_CHUNK 4
#endif

// This wave's 16 rows (16 w .. +16) of a K or V tile.
__device__ __forceinline__ void dma_rows(const uint16_t* head, int64_t stride, TileRef ref, lds_u16* tile, int w,
                                         const uint32_t (&off)[4]) {
  dma_rows16(tile_rsrc(head, stride, ref), tile, 16 * w, off);
}

// Grid form: sequences are taken in chunks of kChunkSeqs, each chunk's query tiles latest (heaviest) first.  The
// work-groups of one kv head are launch-index neighbours Hkv apart, which the dispatcher hands to the same XCD when
// Hkv is a multiple of 8 (to two when it is 4): the ~64 work-groups an XCD runs at once then read the K/V of about
// kChunkSeqs sequences, which its L2 holds, instead of one tile each of every sequence.
constexpr int kChunkSeqs = PKV_W32_CHUNK;

// 1 / l of a token row: the lane's sum l covers its 16 keys of each block, its partner lane (^ 32) the other 16
// (0 for a row that saw no key).
__device__ __forceinline__ float row_inverse(float l) {
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
  const float lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  return lt > 0.f ? 1.f / lt : 0.f;
}
// O block db of one token row of one query head, times inv, in bf16: lane (j, half) holds dims
// 32 db + 8 (r / 4) + 4 half + r % 4 of the row.
__device__ __forceinline__ void write_block(const PrefillKernelArgs& p, int64_t row, int head, int half, int db,
                                            const f32x16_t& o, float inv) {
  uint16_t* orow = p.out + (row * p.num_q_heads + head) * HD + 32 * db + 4 * half;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    u32x2 w;
    w.x = pack_bf16x2(o[4 * v] * inv, o[4 * v + 1] * inv);
    w.y = pack_bf16x2(o[4 * v + 2] * inv, o[4 * v + 3] * inv);
    *reinterpret_cast<u32x2*>(orow + 8 * v) = w;
  }
}

template <int MODE>
__global__ void __launch_bounds__(256, kW32PerCU) prefill_w32_kernel(PrefillKernelArgs p, PieceList plan, int batch) {
  int kvh, b, t;
  int kt0 = 0, kt1 = -1, pslot = -1;  // key tiles [kt0, kt1) (kt1 < 0: all of the unit's); partial slot or -1
  kvh = int(blockIdx.x % unsigned(p.num_kv_heads));
  const int rank = int(blockIdx.x / unsigned(p.num_kv_heads));
  if (plan.list && plan.hdr[2]) {
    if (rank >= plan.hdr[0]) return;
    const PrefillPiece u = plan.list[rank];
    b = u.b;
    t = u.t;
    kt0 = u.kt0;
    kt1 = u.kt1;
    pslot = u.pslot;
  } else {
    if (int64_t(rank) >= int64_t(batch) * p.max_tiles) return;
    const int chunk = rank / (kChunkSeqs * p.max_tiles), r = rank - chunk * kChunkSeqs * p.max_tiles;
    const int nseq = min(kChunkSeqs, batch - chunk * kChunkSeqs);
    b = chunk * kChunkSeqs + r % nseq;
    t = p.max_tiles - 1 - r / nseq;
  }
  const SeqGeom g = seq_geom(p, b);
  if (t >= g.T) return;

  __shared__ __attribute__((aligned(16))) uint16_t lds[NBUF][WTILE];  // 48 KB: three work-groups per CU
  // The wave index is uniform; saying so keeps the LDS bases of the direct-to-LDS loads in scalar registers.
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int hn = wave & 1;  // query head kvh * 2 + hn
  const int j = lane & 31, half = lane >> 5;
  const int Lq = g.Lq, Lk = g.Lk;
  const int t0 = t * BM;
  const int qpos0 = Lk - Lq + t0;
  const int tok = t0 + 32 * (wave >> 1) + j;  // this lane's query token (column of every 32x32 block)
  const int lim = p.causal ? min(Lk - Lq + tok, Lk - 1) : Lk - 1;
  const bool qok = tok < Lq && g.q_start + tok < p.num_q_tokens;
  // This piece's key tiles (a unit's are [0, unit_tiles)); a planned range is clamped to the unit's.
  const int nt = kt1 < 0 ? unit_tiles(g, t) : min(kt1, unit_tiles(g, t));
  kt0 = min(max(kt0, 0), nt - 1);
  int kt_mask = Lk / BN;  // tiles >= kt_mask need the mask
  if (p.causal) kt_mask = min(kt_mask, qpos0 + 1 > 0 ? (qpos0 + 1) / BN : 0);

  f32x16_t o[4];
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  float l = 0.f, m = kMinusBig;

  // A unit in which no query sees a key writes zeros (uniform over the work-group).
  const bool empty = (p.causal ? min(Lk, qpos0 + BM) : Lk) <= 0;
  if (!empty) {
    // Q^T operands: dims 16 ks + 8 half .. +8 of query token `tok`, head kvh * 2 + hn.  Rows past the sequence
    // load its last row instead (finite values; those columns are never written).  The scale is > 0 here (the
    // launcher sends other scales to the 16x16 kernels): weights are exp2(s c - m), c = scale log2(e).
    const float c = p.scale_log2;
    u32x4 qreg[8];
    {
      const int64_t qr = min(int64_t(g.q_start) + min(tok, Lq - 1), int64_t(p.num_q_tokens) - 1);
      const uint16_t* qrow = p.q + qr * p.q_stride + int64_t(kvh * 2 + hn) * HD + half * 8;
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) qreg[ks] = *reinterpret_cast<const u32x4*>(qrow + ks * 16);
    }
    WSrc src;
    src.khead = p.k + int64_t(kvh) * HD;
    src.vhead = p.v + int64_t(kvh) * HD;
    src.bt_row = p.bt ? p.bt + int64_t(b) * p.max_blocks : nullptr;
    src.kstride = p.bt ? int64_t(p.num_kv_heads) * HD : p.k_stride;
    src.vstride = p.bt ? int64_t(p.num_kv_heads) * HD : p.v_stride;
    uint32_t koff[4], voff[4];
    dma_offsets<false>(src.kstride, 16 * wave, lane, koff);
    dma_offsets<true>(src.vstride, 16 * wave, lane, voff);
    lds_u16* const lbase = (lds_u16*)&lds[0][0];
    auto kbuf = [&](int i) { return lbase + (i & 1) * WTILE; };  // K tile kt in buffer kt % 2
    const lds_u16* const vt = lbase + 2 * WTILE;                   // the V tile

    // Scores of block kb of a K tile (the first product starts from zero).
    auto qk = [&](f32x16_t& s, const lds_u16* ktile, int kb) {
      const uint32_t ka = kaddr(ktile, kb, j, half);
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) s = mfma32(kfrag_at(ka, ks), qreg[ks], ks == 0 ? f32x16_t{} : s);
    };
    // Exponentials of scores r0, r0 + 1 (reference m), summed into l and packed into the P^T operand of the
    // block's 16-key chunk r0 / 8.
    auto weight = [&](const f32x16_t& sc, int r0, u32x4 (&pb)[2]) {
      const uint32_t pk = pack_bf16x2(fast_exp2(fmaf(sc[r0], c, -m)), fast_exp2(fmaf(sc[r0 + 1], c, -m)));
      l = add_pair(l, pk);
      pb[r0 >> 3][(r0 & 7) >> 1] = pk;
    };
    // Scores of block kb of `ktile` into sn, interleaved with the weights of the scores in sc: eight steps of one
    // K fragment (one product) and two exponentials, K fragments read two steps ahead.
    auto qk_weights = [&](f32x16_t& sn, const lds_u16* ktile, int kb, const f32x16_t& sc, u32x4 (&pb)[2]) {
      __builtin_amdgcn_s_setprio(1);
      const uint32_t ka = kaddr(ktile, kb, j, half);
      u32x4 kf[3];
      kf[0] = kfrag_at(ka, 0);
      kf[1] = kfrag_at(ka, 1);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        if (i + 2 < 8) kf[(i + 2) % 3] = kfrag_at(ka, i + 2);
        sn = mfma32(kf[i % 3], qreg[i], i == 0 ? f32x16_t{} : sn);
        weight(sc, 2 * i, pb);
        __builtin_amdgcn_sched_barrier(0);
      }
      __builtin_amdgcn_s_setprio(0);
    };
    // O += P V over block kb of a V tile.
    auto pv = [&](const lds_u16* vtile, int kb, const u32x4 (&pb)[2]) {
      const uint32_t va = vaddr(vtile, lane);
#pragma unroll
      for (int u = 0; u < 2; ++u)
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] = mfma32(vfrag_at(va, 2 * kb + u, db), pb[u], o[db]);
    };
    // A block's maxima: the reference maximum moves only when it is exceeded by more than 2^8 (a uniform branch,
    // rarely taken); then l and O are rescaled at once (O after the block's P V products, which it waits for).
    auto decide = [&](const f32x16_t& s) {
      const float mx = max_blk(s, c);
      if (__any(mx > m + kRescaleSlack)) {
        asm volatile("");  // keeps the branch
        const float mn = fmaxf(m, mx);
        const float alpha = fast_exp2(m - mn);
        l *= alpha;
        m = mn;
#pragma unroll
        for (int db = 0; db < 4; ++db) o[db] *= alpha;
      }
    };
    // Pins the weights above the mask branch that follows (otherwise they would be moved next to their products).
    auto keep = [](const u32x4 (&pb)[2]) { asm volatile("" ::"v"(pb[0]), "v"(pb[1])); };

    // Tile references.  Contiguous: the sequence's rows k_start .. k_start + valid - 1 (valid also bounded by the
    // k/v arrays).  Paged: tile kt lies in the cache block of its first key; the block-table entry of the tile
    // whose K loads the next step issues is fetched a step ahead (fk).
    const int valid = MODE == LOAD_PAGED ? Lk
                                         : (g.k_start < 0 ? 0 : int(min(int64_t(Lk), p.num_k_rows - g.k_start)));
    auto tile_ref = [&](int kt, int blk) {
      TileRef r;
      r.rows = __builtin_amdgcn_readfirstlane(min(max(valid - kt * BN, 0), BN));
      r.row = MODE == LOAD_PAGED ? int64_t(blk) * p.bs + ((kt * BN) & (p.bs - 1)) : g.k_start + int64_t(kt) * BN;
      return r;
    };
    const __amdgpu_buffer_rsrc_t bt_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int32_t*>(MODE == LOAD_PAGED ? src.bt_row : p.cu_k), 0, MODE == LOAD_PAGED ? p.max_blocks * 4 : 0,
        kBufferFlags);
    int fk = 0, b0 = 0, b1 = 0;
    if constexpr (MODE == LOAD_PAGED) {
      b0 = bt_fetch(p, bt_rs, kt0);
      b1 = bt_fetch(p, bt_rs, kt0 + 1);
      fk = bt_fetch(p, bt_rs, kt0 + 2);
      b0 = bt_block(p, b0);
      b1 = bt_block(p, b1);
    }
    const TileRef r0 = tile_ref(kt0, b0);
    TileRef r1 = tile_ref(kt0 + 1, b1);  // the tile whose V loads the next barrier B issues

    // Prologue: K and V of the first tile and K of the second; scores and maximum of the first block.
    dma_rows(src.khead, src.kstride, r0, kbuf(kt0), wave, koff);
    dma_rows(src.vhead, src.vstride, r0, (lds_u16*)vt, wave, voff);
    if (kt0 + 1 < nt) dma_rows(src.khead, src.kstride, r1, kbuf(kt0 + 1), wave, koff);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16_t sa, sb;  // scores of the tile's first block (sa) and second block (sb)
    qk(sa, kbuf(kt0), 0);
    if (kt0 >= kt_mask) mask_blk(sa, lim - (kt0 * BN + 4 * half));
    m = fmaxf(m, max_blk(sa, c));

    // Step kt (whose first block's scores are in sa): the second block's scores while the first block's weights
    // are taken; then (barrier A: V of tile kt and K of tile kt + 1 have landed, K of tile kt is no longer read)
    // the K loads of tile kt + 2 into K tile kt's buffer; the first block's P V while the second block's maximum is
    // reduced; the next tile's first block's scores while the second block's weights are taken, and the second
    // block's P V while the next first block's maximum is reduced; then (barrier B: V of tile kt is no longer
    // read) the V loads of tile kt + 1.  `masked`: tile kt + 1 (and so possibly kt) needs the mask.
    auto step = [&](bool masked, auto last_tag, int kt) {
      constexpr bool LAST = decltype(last_tag)::value;
      u32x4 pb0[2];
      qk_weights(sb, kbuf(kt), 1, sa, pb0);
      keep(pb0);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();  // barrier A
      TileRef r2{};  // tile kt + 2: its K loads now, its V loads at the next step's barrier B
      if (!LAST) {
        r2 = tile_ref(kt + 2, MODE == LOAD_PAGED ? bt_block(p, fk) : 0);
        if (kt + 2 < nt) dma_rows(src.khead, src.kstride, r2, kbuf(kt), wave, koff);
        if constexpr (MODE == LOAD_PAGED) fk = bt_fetch(p, bt_rs, kt + 3);
      }
      if (masked) {
        asm volatile("");  // keeps the branch: the mask is not applied to tiles that need none
        mask_blk(sb, lim - (kt * BN + 32 + 4 * half));
      }
      pv(vt, 0, pb0);
      decide(sb);
      u32x4 pb1[2];
      if constexpr (!LAST) {
        qk_weights(sa, kbuf(kt + 1), 0, sb, pb1);
        keep(pb1);
        if (masked) {
          asm volatile("");
          mask_blk(sa, lim - ((kt + 1) * BN + 4 * half));
        }
        pv(vt, 1, pb1);
        decide(sa);
        __syncthreads();  // barrier B
        dma_rows(src.vhead, src.vstride, r1, (lds_u16*)vt, wave, voff);
        r1 = r2;
      } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) weight(sb, 2 * i, pb1);
        pv(vt, 1, pb1);
      }
    };
    const std::integral_constant<bool, false> no;
    const std::integral_constant<bool, true> yes;
    for (int kt = kt0; kt + 1 < nt; ++kt) step(kt + 1 >= kt_mask, no, kt);
    step(true, yes, nt - 1);
  }

  // A piece of a split unit hands its state (O, m, l) on to the merge kernel, every lane whatever its row (plain
  // stores: the merge, launched next, reads them while they are still in the caches).
  if (pslot >= 0) {
    f32x4_t* dst = plan.parts + ((size_t(pslot) * p.num_kv_heads + kvh) * 4 + wave) * (kPartialChunks * 64) + lane;
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        dst[(4 * db + v) * 64] = f32x4_t{o[db][4 * v], o[db][4 * v + 1], o[db][4 * v + 2], o[db][4 * v + 3]};
    dst[16 * 64] = f32x4_t{m, l, 0.f, 0.f};
    return;
  }
  if (!qok) return;
  const float inv = row_inverse(l);
#pragma unroll
  for (int db = 0; db < 4; ++db) write_block(p, g.q_start + tok, kvh * 2 + hn, half, db, o[db], inv);
}

// Merge of the split units: one work-group per (split unit, kv head, 32-dim block db of the output), the lanes laid
// out as the main kernel's, so each lane combines its own (m, l) and O block of every piece by the exact online-
// softmax rescaling [P2 §5.2 ②]: with M the running maximum, a new piece (m_i, l_i, O_i) gives M' = max(M, m_i),
// l = l 2^(M - M') + l_i 2^(m_i - M'), O likewise (a piece in which a row saw no key has m = -1e30, l = 0, O = 0
// and changes nothing).  One pass, unrolled so that the loads of eight pieces are in flight at once: a unit cut
// into many pieces pays a memory round trip per eight pieces, not per piece.
__global__ void __launch_bounds__(256) prefill_w32_merge_kernel(PrefillKernelArgs p, PieceList plan) {
  const int db = int(blockIdx.x & 3u);
  const int kvh = int((blockIdx.x >> 2) % unsigned(p.num_kv_heads));
  const int s = int((blockIdx.x >> 2) / unsigned(p.num_kv_heads));
  if (s >= plan.hdr[1]) return;
  const PrefillSplit e = plan.splits[s];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int j = lane & 31, half = lane >> 5;
  const int q_start = p.cu_q[e.b], Lq = max(p.cu_q[e.b + 1] - q_start, 0);
  const int tok = e.t * BM + 32 * (wave >> 1) + j;
  const f32x4_t* src = plan.parts + ((size_t(e.pbase) * p.num_kv_heads + kvh) * 4 + wave) * (kPartialChunks * 64) + lane;
  const size_t piece_stride = size_t(p.num_kv_heads) * 4 * kPartialChunks * 64;
  float mrun = kMinusBig, l = 0.f;
  f32x16_t o;
#pragma unroll
  for (int r = 0; r < 16; ++r) o[r] = 0.f;
  constexpr int kBatch = 8;
  for (int i0 = 0; i0 < e.np; i0 += kBatch) {
    // all loads of the batch first (pieces past the last re-read it and are then left out)
    f32x4_t ml[kBatch], x[kBatch][4];
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      const f32x4_t* q = src + size_t(min(i0 + k, e.np - 1)) * piece_stride;
      ml[k] = q[16 * 64];
#pragma unroll
      for (int v = 0; v < 4; ++v) x[k][v] = q[(4 * db + v) * 64];
    }
    __builtin_amdgcn_sched_barrier(0);  // keeps the batch's loads ahead of the arithmetic that waits for them
#pragma unroll
    for (int k = 0; k < kBatch; ++k) {
      // a re-read entry past the last piece folds in with weight 0 and leaves the running maximum alone
      const bool ok = i0 + k < e.np;
      const float mi = ok ? ml[k][0] : kMinusBig;
      const float mn = fmaxf(mrun, mi);
      const float a = fast_exp2(mrun - mn), f = ok ? fast_exp2(mi - mn) : 0.f;
      mrun = mn;
      l = fmaf(ml[k][1], f, l * a);
#pragma unroll
      for (int v = 0; v < 4; ++v)
#pragma unroll
        for (int c = 0; c < 4; ++c) o[4 * v + c] = fmaf(x[k][v][c], f, o[4 * v + c] * a);
    }
  }
  if (tok >= Lq || int64_t(q_start) + tok >= p.num_q_tokens) return;
  write_block(p, int64_t(q_start) + tok, kvh * 2 + (wave & 1), half, db, o, row_inverse(l));
}

}  // namespace

bool prefill_w32_supported(int group, int mode, float scale) {
  return group == 2 && (mode == LOAD_CONTIG || mode == LOAD_PAGED) && scale > 0.f;
}

hipError_t launch_prefill_w32(const PrefillKernelArgs& p, int batch, int mode, PieceList plan, int grid_units,
                              int split_cap, hipStream_t stream) {
  const dim3 block(256);
  const uint64_t units = plan.list ? uint64_t(grid_units) : uint64_t(batch) * uint64_t(p.max_tiles);
  const uint64_t wgs = units * uint64_t(p.num_kv_heads);
  if (wgs == 0) return hipSuccess;
  if (wgs > 0xffffffffull || uint64_t(split_cap) * uint64_t(p.num_kv_heads) * 4u > 0xffffffffull)
    return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<uint32_t>(wgs));
  if (mode == LOAD_CONTIG)
    hipLaunchKernelGGL(prefill_w32_kernel<LOAD_CONTIG>, grid, block, 0, stream, p, plan, batch);
  else
    hipLaunchKernelGGL(prefill_w32_kernel<LOAD_PAGED>, grid, block, 0, stream, p, plan, batch);
  if (plan.list && split_cap > 0)
    hipLaunchKernelGGL(prefill_w32_merge_kernel, dim3(uint32_t(split_cap) * uint32_t(p.num_kv_heads) * 4u), block,
                       0, stream, p, plan);
  return hipGetLastError();
}

}  // namespace pkv
