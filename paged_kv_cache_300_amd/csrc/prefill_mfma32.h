// 32x32x16 bf16 MFMA building blocks of the GQA-2 prefill kernel (attn_prefill_w32.hip, 32 query rows per wave).
// K/V tiles of 64 keys sit in LDS as 256-byte rows whose 16-byte chunks are XOR-swizzled; scores are transposed
// (S^T = K Q^T), so lane (j, half) of a 32x32 block holds keys 8 (r / 4) + 4 half + r % 4 (r < 16) of query j, and
// P^T feeds O^T = V^T P^T straight from registers.
// Device helpers only; everything is inline.
#pragma once

#include <math.h>
#include <stdint.h>

#include "common.h"
#include "prefill_common.h"

namespace pkv {
namespace pf {

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
static_assert(BM == 64 && BN == 64, "query tiles of 64 tokens; K/V tiles of 64 keys");

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

// The tile's buffer resource: base = its first row, size = its valid rows.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t* head, int64_t stride, TileRef ref) {
  return make_rsrc(head + ref.row * stride, uint32_t(ref.rows) * uint32_t(stride) * 2u);
}

// Rows g0 .. g0 + 16 of a K or V tile into `tile`, as 4 direct-to-LDS loads of 4 rows each (g0 a multiple of 16).
// Lane i of a load lands at row g0 + 4 k + i / 16, chunk slot i % 16, so it fetches chunk (i % 16) ^ swz(row);
// off[k] is that byte offset from the tile's first row.  The whole offset is the lane's (vector) offset, which the
// buffer's bounds check covers: rows past `rows` read as zeros and touch no memory.
__device__ __forceinline__ void dma_rows16(__amdgpu_buffer_rsrc_t rs, lds_u16* tile, int g0, const uint32_t (&off)[4]) {
  dma16x4(rs, off, tile + g0 * WROW);
}

// Lane offsets of this lane's chunk in the four 4-row loads of rows g0 .. g0 + 16 (see dma16x4): row
// r = g0 + 4 k + lane / 16, chunk (lane % 16) ^ swz(r).  The swizzles only look at r % 16 = 4 k + lane / 16.
template <bool IS_V>
__device__ __forceinline__ void dma_offsets(int64_t stride, int g0, int lane, uint32_t (&off)[4]) {
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int r = g0 + k * 4 + (lane >> 4);
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

}  // namespace pf
}  // namespace pkv
