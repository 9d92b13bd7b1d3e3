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

namespace pkv {
namespace {
using namespace pf;

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
// LDS pointers are kept in the LDS address space (32-bit offsets, no generic-pointer conversions).
typedef __attribute__((address_space(3))) uint16_t lds_u16;
typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
typedef __attribute__((address_space(3))) i16x4_t lds_i16x4;

__device__ __forceinline__ u32x2 ds_read_tr16_l(const lds_u16* p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p));
}

constexpr int WROW = 128;          // LDS row: 128 bf16 = 256 B of 16 swizzled 16-byte chunks
constexpr int WTILE = BN * WROW;   // one K or V tile: 64 keys, 16 KB
constexpr int NBUF = 3;            // K0, K1, V
#ifndef PKV_W32_CHUNK
#define PKV_W32_CHUNK 4
#endif
static_assert(BM == 64 && BN == 64, "a work-group is 2 x 32 tokens; tiles are 64 keys");

__device__ __forceinline__ f32x16_t mfma32(const u32x4& a, const u32x4& b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2_t;
// l + p.lo + p.hi for a packed pair of bf16 weights: the normaliser sums the same rounded weights P V multiplies.
__device__ __forceinline__ float add_pair(float l, uint32_t p) {
  const bf16x2_t one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, p), one, l, false);
}

// 16-byte chunk c of LDS row r is stored at chunk slot c ^ swz(r).
__device__ __forceinline__ int swz_k(int r) { return r & 15; }
__device__ __forceinline__ int swz_v(int r) { return (r & 3) << 2; }

struct WSrc {
  const uint16_t* khead;  // kv head at row / slot 0
  const uint16_t* vhead;
  const int32_t* bt_row;  // paged: the sequence's block-table row
  int64_t kstride, vstride;  // elements between rows (contiguous) or slots (paged)
};

// A wave's share of a tile: four direct-to-LDS loads of 16 bytes per lane, lane i of load k landing at
// `dst` + 1024 k + 16 i.  The immediate offset 1024 k moves both the LDS destination and the global address, so
// the lane offsets off[k] are given less 1024 k (the bounds check covers the whole offset).  Written as inline
// assembly on purpose: the compiler would otherwise make every later LDS read wait for all such loads in flight
// (it cannot tell the tile being filled from the tiles being read), which would expose a memory round trip per
// tile.  The tiles are published by an explicit wait for all loads (s_waitcnt 0) and a barrier before they are
// read.
__device__ __forceinline__ void dma16x4(__amdgpu_buffer_rsrc_t rs, const uint32_t (&off)[4], const lds_u16* dst) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>(dst)));
  asm volatile("s_mov_b32 m0, %4\n\t"
               "buffer_load_dwordx4 %0, %5, 0 offen lds\n\t"
               "buffer_load_dwordx4 %1, %5, 0 offen offset:1024 lds\n\t"
               "buffer_load_dwordx4 %2, %5, 0 offen offset:2048 lds\n\t"
               "buffer_load_dwordx4 %3, %5, 0 offen offset:3072 lds"
               :
               : "v"(off[0]), "v"(off[1]), "v"(off[2]), "v"(off[3]), "s"(m0), "s"(rs)
               : "m0");
}

// A K/V tile's place in memory, uniform over the work-group: its first row (contiguous rows) or slot (paged
// cache), and how many of its 64 rows are valid keys.  Computed once per tile: the K loads of a tile and, one
// step later, its V loads use the same one.
struct TileRef {
  int64_t row;
  int rows;
};

// This wave's 16 rows (16 w .. +16) of a K or V tile into `tile`, as 4 direct-to-LDS loads of 4 rows each.
// Lane i of a load lands at row 16 w + 4 k + i / 16, chunk slot i % 16, so it fetches chunk (i % 16) ^ swz(row);
// off[k] is that byte offset from the tile's first row.  The whole offset is the lane's (vector) offset, which the
// buffer's bounds check covers: rows past `rows` read as zeros and touch no memory.
__device__ __forceinline__ void dma_rows(const uint16_t* head, int64_t stride, TileRef ref, lds_u16* tile, int w,
                                         const uint32_t (&off)[4]) {
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(head + ref.row * stride, uint32_t(ref.rows) * uint32_t(stride) * 2u);
  dma16x4(rs, off, tile + w * 16 * WROW);
}

// Lane offsets of this lane's chunk in each of its wave's four 4-row loads (see dma16x4): row
// r = 16 w + 4 k + lane / 16, chunk (lane % 16) ^ swz(r).  The swizzles only look at r % 16 = 4 k + lane / 16.
template <bool IS_V>
__device__ __forceinline__ void dma_offsets(int64_t stride, int w, int lane, uint32_t (&off)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = w * 16 + k * 4 + (lane >> 4);
    const int c = (lane & 15) ^ (IS_V ? swz_v(r) : swz_k(r));
    // less the immediate offset 1024 k of load k (row r >= 4 k and a row is at least 256 bytes: never negative)
    off[k] = uint32_t(r) * uint32_t(stride) * 2u + uint32_t(c) * 16u - uint32_t(k) * 1024u;
  }
}

// PAGED: the block-table entry of key tile kt, fetched with a vector buffer load one step before the tile's loads
// are issued (a scalar load would put its round trip at the head of the step and, sharing the LDS reads' wait
// counter, make every LDS wait behind it a full wait).  Entries past the row read as 0; an entry outside
// [0, num_blocks) selects block 0 (such rows are outside the sequence's keys or give unspecified results).
__device__ __forceinline__ int bt_fetch(const PrefillKernelArgs& p, __amdgpu_buffer_rsrc_t rs, int kt) {
  const int lb = max(min((kt * BN) >> p.bs_shift, p.max_blocks - 1), 0);
  return __builtin_amdgcn_raw_buffer_load_b32(rs, uint32_t(lb) * 4u, 0, 0);
}
__device__ __forceinline__ int bt_block(const PrefillKernelArgs& p, int fetched) {
  const int blk = __builtin_amdgcn_readfirstlane(fetched);
  return (blk >= 0 && blk < p.num_blocks) ? blk : 0;
}

// LDS fragment reads.  Addresses are byte offsets in the LDS; a buffer starts on a 16 KB boundary and its rows
// are 256 B, so a row's chunk field (bits 4-7) can be flipped with an XOR.  Each fragment is then one XOR of a
// per-buffer lane address with a constant, not an address of its own kept across the loop.
//
// K fragment (A operand) of key block kb (32 keys) and dims 16 ks .. +16: lane (j, half) reads key row
// 32 kb + j, chunk 2 ks + half, stored at chunk (2 ks + half) ^ (j & 15) = ((j & 15) ^ half) ^ 2 ks.
__device__ __forceinline__ uint32_t kaddr(const lds_u16* ktile, int kb, int j, int half) {
  return uint32_t(reinterpret_cast<uintptr_t>(ktile)) + uint32_t((kb * 32 + j) << 8) + uint32_t(((j & 15) ^ half) << 4);
}
__device__ __forceinline__ u32x4 kfrag_at(uint32_t a, int ks) {
  return *(const lds_u32x4*)(uintptr_t)(a ^ (uint32_t(ks) << 5));
}

// V^T fragment (A operand) of dims 32 db .. +32 and keys 16 kc .. +16, in the key order of the P^T operand: lane
// (j, half) slot s holds V[16 kc + 8 (s / 4) + 4 half + s % 4][32 db + j].  Two transposing reads: within each
// 16-lane quarter q, source lane 4 jj + i' names row 16 kc + 4 (q / 2) + jj (+ 8 for the second read), dims
// 32 db + 16 (q % 2) + 4 i' .. +4 (chunk 4 db + 2 (q % 2) + i' / 2, stored at chunk 4 (db ^ jj) + 2 (q % 2) + i' / 2),
// and result lane i receives those four rows at dim 32 db + 16 (q % 2) + i.  vaddr is the lane's address for
// kc = db = 0; chunk group db is reached by an XOR of bits 6-7, chunk kc and the second read by adding whole rows.
__device__ __forceinline__ uint32_t vaddr(const lds_u16* vtile, int lane) {
  const int q = lane >> 4, jj = (lane >> 2) & 3, ip = lane & 3;
  return uint32_t(reinterpret_cast<uintptr_t>(vtile)) + uint32_t((4 * (q >> 1) + jj) << 8) + uint32_t(jj << 6) +
         uint32_t((2 * (q & 1) + (ip >> 1)) << 4) + uint32_t((ip & 1) << 3);
}
__device__ __forceinline__ u32x4 vfrag_at(uint32_t a, int kc, int db) {
  const uint32_t x = (a ^ (uint32_t(db) << 6)) + uint32_t(kc << 12);
  const u32x2 lo = ds_read_tr16_l((const lds_u16*)(uintptr_t)x);
  const u32x2 hi = ds_read_tr16_l((const lds_u16*)(uintptr_t)(x + 2048u));
  return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// Softmax blocks are 32 keys (half an LDS tile): a block's scores are one 32x32 accumulator, lane (j, half)
// holding keys 8 (r / 4) + 4 half + r % 4 (r < 16) of the block for query j.
//
// Keys of the block past `room` (this lane's last visible key minus the block's first key minus 4 half) get -inf.
__device__ __forceinline__ void mask_blk(f32x16_t& s, int room) {
#pragma unroll
  for (int r = 0; r < 16; ++r) s[r] = 8 * (r >> 2) + (r & 3) <= room ? s[r] : -INFINITY;
}

// Maximum of the query's 32 block scores (the lane's 16 and its partner lane's, lane ^ 32), times c.
__device__ __forceinline__ float max_blk(const f32x16_t& x, float c) {
  float a = fmax_ieee(fmax_ieee(x[0], x[1]), x[2]);
  float b = fmax_ieee(fmax_ieee(x[8], x[9]), x[10]);
  a = fmax_ieee(fmax_ieee(a, x[3]), x[4]);
  b = fmax_ieee(fmax_ieee(b, x[11]), x[12]);
  a = fmax_ieee(fmax_ieee(a, x[5]), x[6]);
  b = fmax_ieee(fmax_ieee(b, x[13]), x[14]);
  return max_xor32(fmax_ieee(fmax_ieee(a, x[7]), fmax_ieee(b, x[15]))) * c;
}

// Grid form: sequences are taken in chunks of kChunkSeqs, each chunk's query tiles latest (heaviest) first.  The
// work-groups of one kv head are launch-index neighbours Hkv apart, which the dispatcher hands to the same XCD when
// Hkv is a multiple of 8 (to two when it is 4): the ~64 work-groups an XCD runs at once then read the K/V of about
// kChunkSeqs sequences, which its L2 holds, instead of one tile each of every sequence.
constexpr int kChunkSeqs = PKV_W32_CHUNK;

template <int MODE>
__global__ void __launch_bounds__(256, 3) prefill_w32_kernel(PrefillKernelArgs p, PlanList plan, int batch) {
  int kvh, b, t;
  kvh = int(blockIdx.x % unsigned(p.num_kv_heads));
  const int rank = int(blockIdx.x / unsigned(p.num_kv_heads));
  if (plan.list) {
    if (rank >= *plan.count) return;
    const int2 u = plan.list[rank];
    b = u.x;
    t = u.y;
  } else {
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
  const int nt = unit_tiles(g, t);
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
    dma_offsets<false>(src.kstride, wave, lane, koff);
    dma_offsets<true>(src.vstride, wave, lane, voff);
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
      b0 = bt_fetch(p, bt_rs, 0);
      b1 = bt_fetch(p, bt_rs, 1);
      fk = bt_fetch(p, bt_rs, 2);
      b0 = bt_block(p, b0);
      b1 = bt_block(p, b1);
    }
    const TileRef r0 = tile_ref(0, b0);
    TileRef r1 = tile_ref(1, b1);  // the tile whose V loads the next barrier B issues

    // Prologue: K and V of the first tile and K of the second; scores and maximum of the first block.
    dma_rows(src.khead, src.kstride, r0, kbuf(0), wave, koff);
    dma_rows(src.vhead, src.vstride, r0, (lds_u16*)vt, wave, voff);
    if (nt > 1) dma_rows(src.khead, src.kstride, r1, kbuf(1), wave, koff);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    f32x16_t sa, sb;  // scores of the tile's first block (sa) and second block (sb)
    qk(sa, kbuf(0), 0);
    if (0 >= kt_mask) mask_blk(sa, lim - 4 * half);
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
    for (int kt = 0; kt + 1 < nt; ++kt) step(kt + 1 >= kt_mask, no, kt);
    step(true, yes, nt - 1);
  }

  // Normalise and write: the lane's sum covers its 16 keys of each block, its partner lane (^ 32) the other 16.
  // Lane (j, half) holds dims 32 db + 8 (r / 4) + 4 half + r % 4 of token `tok`.
  if (!qok) return;
  const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(l), __float_as_uint(l), false, false);
  const float lt = __uint_as_float(sw[0]) + __uint_as_float(sw[1]);
  const float inv = lt > 0.f ? 1.f / lt : 0.f;
  uint16_t* orow = p.out + (int64_t(g.q_start + tok) * p.num_q_heads + kvh * 2 + hn) * HD + 4 * half;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      u32x2 w;
      w.x = pack_bf16x2(o[db][4 * v] * inv, o[db][4 * v + 1] * inv);
      w.y = pack_bf16x2(o[db][4 * v + 2] * inv, o[db][4 * v + 3] * inv);
      *reinterpret_cast<u32x2*>(orow + 32 * db + 8 * v) = w;
    }
}

}  // namespace

bool prefill_w32_supported(int group, int mode, float scale) {
  return group == 2 && (mode == LOAD_CONTIG || mode == LOAD_PAGED) && scale > 0.f;
}

hipError_t launch_prefill_w32(const PrefillKernelArgs& p, int batch, int mode, PlanList plan, int grid_units,
                              hipStream_t stream) {
  const dim3 block(256);
  const uint64_t units = plan.list ? uint64_t(grid_units) : uint64_t(batch) * uint64_t(p.max_tiles);
  const uint64_t wgs = units * uint64_t(p.num_kv_heads);
  if (wgs == 0) return hipSuccess;
  if (wgs > 0xffffffffull) return hipErrorInvalidConfiguration;
  const dim3 grid(static_cast<uint32_t>(wgs));
  if (mode == LOAD_CONTIG)
    hipLaunchKernelGGL(prefill_w32_kernel<LOAD_CONTIG>, grid, block, 0, stream, p, plan, batch);
  else
    hipLaunchKernelGGL(prefill_w32_kernel<LOAD_PAGED>, grid, block, 0, stream, p, plan, batch);
  return hipGetLastError();
}

}  // namespace pkv
