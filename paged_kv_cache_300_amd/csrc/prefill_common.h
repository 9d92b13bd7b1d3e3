// Shared by the prefill kernels (attn_prefill.hip: 16x16 tiles, 16 tokens per wave; attn_prefill_w32.hip: 32x32
// tiles, 32 query rows per wave; both at two waves per SIMD): kernel arguments, per-sequence geometry,
// buffer-resource tile reads and the longest-first planner's output.  Device helpers only; everything is inline.
#pragma once

#include <math.h>
#include <stdint.h>

#include "common.h"
#include "launch.h"

namespace pkv {
namespace pf {

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
constexpr float kRescaleSlack = 8.f;  // log2 units: weights up to 2^8 before the output is rescaled

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

// IEEE maximum (v_maximum3_f32 on gfx950: no operand canonicalisation, NaN propagates).
__device__ __forceinline__ float fmax_ieee(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Maximum over lanes i and i ^ 16 (rows of 16 swapped pairwise), and over lanes i and i ^ 32.
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax_ieee(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmax_ieee(__uint_as_float(r[0]), __uint_as_float(r[1]));
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

// How K/V tiles reach LDS.  CONTIG: rows of this step's k/v arrays; PAGED: the paged cache with a block size
// that is a power of two >= 64, so a 64-key tile lies inside one block.  Both read a tile as one buffer
// resource (base = the tile's first row, size = its valid rows), so rows past the end of the sequence come
// back as zeros without any per-lane check.  ROWS: any other block size, one block-table lookup per row.
enum : int { LOAD_CONTIG = 0, LOAD_PAGED = 1, LOAD_ROWS = 2 };

// Raw buffer: stride 0, 32-bit data format; an offset at or past num_records reads 0 and touches no memory.
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const uint16_t* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), 0, int(bytes), kBufferFlags);
}
__device__ __forceinline__ u32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0));
}

__device__ __forceinline__ int block_of(const PrefillKernelArgs& p, const int32_t* bt_row, int lb) {
  const int blk = bt_row[lb];
  return (blk >= 0 && blk < p.num_blocks) ? blk : 0;
}

// Per-sequence geometry of the work decomposition.
struct SeqGeom {
  int q_start;      // first query row of the sequence
  int Lq, Lk;       // new tokens; visible keys (paged mode: clamped to the block table)
  int64_t k_start;  // contiguous mode: first key row
  int T;            // query tiles
  int NKe;          // key tiles of an unmasked row, at least 1
  int c0;           // query tile t attends key tiles [0, clamp(t + 1 + c0, 1, NKe))
};

__device__ __forceinline__ int ceil_div64(int x) { return x >= 0 ? (x + 63) >> 6 : -((-x) >> 6); }

__device__ __forceinline__ SeqGeom seq_geom(const PrefillKernelArgs& p, int b) {
  SeqGeom g;
  g.q_start = p.cu_q[b];
  g.Lq = max(p.cu_q[b + 1] - g.q_start, 0);
  g.k_start = p.cu_k[b];
  int Lk = max(p.cu_k[b + 1] - p.cu_k[b], 0);
  if (p.bt) Lk = min(Lk, p.max_blocks * p.bs);
  g.Lk = Lk;
  g.T = (g.Lq + BM - 1) / BM;
  g.NKe = max((Lk + BN - 1) / BN, 1);
  // Causal: the last query of tile t sits at position Lk - Lq + 64 t + 63, so it sees ceil((Lk - Lq)/64) + t + 1
  // key tiles.  A tile with no visible key still runs one fully masked key tile, which writes zeros.
  g.c0 = p.causal ? ceil_div64(Lk - g.Lq) : g.NKe;
  return g;
}

__device__ __forceinline__ int unit_tiles(const SeqGeom& g, int t) { return min(max(t + 1 + g.c0, 1), g.NKe); }

// The longest-first planner's output: `count` (sequence, query tile) units, largest key-tile count first.
struct PlanList {
  const int2* list;
  const int* count;
};

// The splitting planner's output for the 32x32 kernel: work pieces, each the key tiles [kt0, kt1) of one
// (sequence, query tile) unit, largest first.  pslot >= 0 marks a piece of a split unit, which writes its partial
// softmax state (O, m, l) to partial slot pslot instead of the output; the merge kernel then combines the pieces
// of each split unit (splits[i] = its sequence, query tile, piece count and first partial slot).
struct PrefillPiece {
  int b, t, kt0, kt1, pslot, pad0, pad1, pad2;
};
struct PrefillSplit {
  int b, t, np, pbase;
};
// Partial state of one piece and kv head: per wave of the work-group and lane, 16 float4 of O (chunk 4 db + v holds
// o[db][4 v .. 4 v + 3]) then one float4 (m, l, 0, 0); chunk-major, so a wave's store of one chunk is 1 KiB
// contiguous.
constexpr int kPartialChunks = 17;
constexpr size_t kPartialFloat4 = size_t(4) * kPartialChunks * 64;  // per (piece, kv head): 4 waves

struct PieceList {
  const PrefillPiece* list;  // NULL: grid order, no planner
  const int* hdr;            // [0] pieces listed, [1] split units, [2] 1: listed order, 0: grid order
  const PrefillSplit* splits;
  f32x4_t* parts;
};

}  // namespace pf

// 32x32 MFMA prefill for GQA groups of 2 with contiguous rows or a paged cache whose block size is a power of two
// >= 64, and a positive softmax scale (attn_prefill_w32.hip).  plan.list == NULL: one work-group per (kv head,
// sequence, query tile), sequences in chunks with each chunk's latest tiles first; else one per listed piece and kv
// head (grid_units pieces at most), followed by the merge of the split units (split_cap of them at most).
bool prefill_w32_supported(int group, int mode, float scale);
hipError_t launch_prefill_w32(const pf::PrefillKernelArgs& p, int batch, int mode, pf::PieceList plan, int grid_units,
                              int split_cap, hipStream_t stream);
// Work-groups of the 32x32 kernel one CU holds at once.
constexpr int kW32PerCU = 3;

}  // namespace pkv
