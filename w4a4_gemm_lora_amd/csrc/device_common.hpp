// Device-side helpers shared by the kernels of libw4a4 (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w4a4 {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));
typedef uint32_t v2u __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  return (float)__builtin_bit_cast(_Float16, b);
}

// One 64-group's codes held by a lane: two dwords, dword d nibble i is the
// code at k = 16c + 8d + i of the group (c = lane / 16).  The integer MFMA
// operand is formed by moving every nibble into the high half of a byte,
// i.e. the byte holds 16*q as a signed int8:
//   (d << 4) & 0xF0F0F0F0 -> nibbles 0,2,4,6 ;  d & 0xF0F0F0F0 -> nibbles 1,3,5,7.
// X and W are expanded by the same function, so the byte order seen by the
// MFMA is the same permutation of k on both operands and the dot product is
// 256 * P exactly (|256 P| <= 2^20).
__device__ __forceinline__ v4i expand_group(uint32_t d0, uint32_t d1) {
  v4i r;
  r.x = (int)((d0 << 4) & 0xF0F0F0F0u);
  r.y = (int)(d0 & 0xF0F0F0F0u);
  r.z = (int)((d1 << 4) & 0xF0F0F0F0u);
  r.w = (int)(d1 & 0xF0F0F0F0u);
  return r;
}

__device__ __forceinline__ v4i mfma_i8_16x16x64(v4i a, v4i b, v4i c) {
  return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_f16_16x16x16(v4h a, v4h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x16f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v4f mfma_f16_16x16x32(v8h a, v8h b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
}

// Split an fp32 4-vector into fp16 hi + lo parts (hi + lo carries ~22 bits).
__device__ __forceinline__ void split_f16(v4f v, v4h& hi, v4h& lo) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    _Float16 h = (_Float16)v[i];
    hi[i] = h;
    lo[i] = (_Float16)(v[i] - (float)h);
  }
}

}  // namespace w4a4
