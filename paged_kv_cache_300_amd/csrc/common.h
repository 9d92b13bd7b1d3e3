// Device helpers shared by the gfx950 kernels of the paged-KV attention path.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

// Raw bf16 storage: the upper half of an IEEE binary32 word.
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Plain clang vector types: unlike HIP's uint4 class they load and store as one register tuple and never
// force a copy through private memory.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 pkv_bf16x2_t;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float pkv_f32x2_t;

// float32 -> bf16 with the hardware converter (v_cvt_pk_bf16_f32: round to nearest even, NaN stays NaN).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const pkv_f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, pkv_bf16x2_t));
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) { return uint16_t(pack_bf16x2(f, 0.f) & 0xffffu); }

// Element load/store as float for the generic kernels.
template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ __forceinline__ static float load(const float* p) { return *p; }
  __device__ __forceinline__ static void store(float* p, float x) { *p = x; }
};
template <> struct Elem<uint16_t> {
  __device__ __forceinline__ static float load(const uint16_t* p) { return bf16_to_f32(*p); }
  __device__ __forceinline__ static void store(uint16_t* p, float x) { *p = f32_to_bf16(x); }
};

// DPP lane moves inside a row of 16 lanes (GFX9 encodings).
enum : int {
  DPP_QUAD_XOR1 = 0xB1,       // quad_perm [1,0,3,2]
  DPP_QUAD_XOR2 = 0x4E,       // quad_perm [2,3,0,1]
  DPP_ROW_HALF_MIRROR = 0x141 // lane i <-> 7-i inside each group of 8
};

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over each aligned group of 8 lanes; every lane of the group receives the sum.
__device__ __forceinline__ float sum8(float x) {
  x += dpp_f32<DPP_QUAD_XOR1>(x);
  x += dpp_f32<DPP_QUAD_XOR2>(x);
  x += dpp_f32<DPP_ROW_HALF_MIRROR>(x);
  return x;
}

__device__ __forceinline__ float shfl_xor_f32(float x, int mask) {
  const int lane = threadIdx.x & 63;
  return __int_as_float(__builtin_amdgcn_ds_bpermute(((lane ^ mask) << 2), __float_as_int(x)));
}

__device__ __forceinline__ float wave_max(float x) {
  for (int o = 32; o >= 1; o >>= 1) x = fmaxf(x, shfl_xor_f32(x, o));
  return x;
}
__device__ __forceinline__ float wave_sum(float x) {
  for (int o = 32; o >= 1; o >>= 1) x += shfl_xor_f32(x, o);
  return x;
}

// Physical slot of key position j of a sequence, or -1 if its block-table entry is unusable.
__device__ __forceinline__ int64_t paged_slot(const int32_t* bt_row, int j, int block_size, int num_blocks) {
  const int blk = bt_row[j / block_size];
  if (blk < 0 || blk >= num_blocks) return -1;
  return int64_t(blk) * block_size + (j % block_size);
}

}  // namespace pkv
