// Per-group quantizer arithmetic shared by the activation pass and the
// gated GEMM epilogue that quantizes its own output for the next layer, so
// that both produce the same codes and scales bit for bit ("W4A4 CUDA Kernel
// for Voice Clone", section 3.6: per (row, 64-group) absmax, scale
// absmax / 7 stored in fp16, round to nearest, clamp to [-8, 7], 4-bit
// two's-complement codes).
#pragma once

#include "device_common.hpp"

namespace w4a4 {

// Codes for 8 values (one dword): q = clamp(rint(fl32(x / s)), -8, 7) with
// round-half-to-even, where s is the group's fp16 scale (sf, exact in fp32)
// and rs ~ 1/s (v_rcp_f32, ~1 ulp).
//
// No IEEE division is needed.  x and s are fp16 values, so x/s is a ratio of
// two integers of at most 11 bits times a power of two; unless it is exactly
// a half-integer, it lies at least 2^-13 away from every half-integer, far
// beyond the error of t = x * rs (< 2^-19 for |x/s| <= 8.5), so rint(t) is the
// nearest integer to x/s -- the same as the nearest integer to fl32(x/s).
// When x/s is exactly a half-integer, fl32(x/s) is that half-integer and the
// rule rounds it to the even neighbour.  The residual f = x - n*s is exact
// (n*s has <= 15 significant bits and |f| <= s/2, so f needs <= 12 bits), and
// x/s is a half-integer exactly when |f| == s/2.  Such ties are rare, so the
// fix-up runs on a wave-uniform branch taken only when some lane has one.
//
// Packing: for an integer n in [-8, 7] and j < 4, n + 1.5 * 2^(23 - 4j) is
// exact and its bit pattern holds n << 4j (two's complement) in bits
// [4j, 4j + 4), so one and-or puts a code in place within a 16-bit half.
__device__ __forceinline__ uint32_t quantize8(v8h v, float sf, float rs) {
  float n[8], f[8];
  bool tie = false;
  const float half_s = 0.5f * sf;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float x = (float)v[i];
    n[i] = __builtin_rintf(x * rs);
    f[i] = __builtin_fmaf(-n[i], sf, x);
    tie |= __builtin_fabsf(f[i]) == half_s;
  }
  if (__builtin_amdgcn_ballot_w64(tie) != 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const bool fix = (__builtin_fabsf(f[i]) == half_s) & ((((int)n[i]) & 1) != 0);
      n[i] = fix ? n[i] + __builtin_copysignf(1.0f, f[i]) : n[i];
    }
  }
  // two 16-bit halves, each built with the biases 1.5 * 2^(23 - 4j), j < 4,
  // whose own set bits (22 and up) stay clear of bits [0, 16)
  uint32_t half[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = i & 3;
    const float q = __builtin_amdgcn_fmed3f(n[i], -8.0f, 7.0f);
    const float biased = q + __builtin_ldexpf(1.5f, 23 - 4 * j);   // constant per i
    half[i >> 2] |= __builtin_bit_cast(uint32_t, biased) & (0xFu << (4 * j));
  }
  return half[0] | (half[1] << 16);
}

// max |x| over 8 fp16 values: for fp16, |x| orders like (bits & 0x7fff) as
// unsigned integers, so the max is taken on the bit patterns.
__device__ __forceinline__ uint32_t absmax8_bits(v8h v, uint32_t m) {
  const v4u w = __builtin_bit_cast(v4u, v);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = w[i] & 0x7FFF7FFFu;
    const uint32_t lo = a & 0xFFFFu, hi = a >> 16;
    m = m > lo ? m : lo;
    m = m > hi ? m : hi;
  }
  return m;
}

// Scale of a group from its absmax: fp16(fp32(amax / 7)) with the IEEE fp32
// division (one per group); a zero scale becomes 2^-24.
__device__ __forceinline__ _Float16 group_scale(float amax) {
  float s32 = amax / 7.0f;
  _Float16 s = (_Float16)s32;
  if (s == (_Float16)0.0f) s = __builtin_bit_cast(_Float16, (uint16_t)1);
  return s;
}

// One 64-group of one row, held by the four lanes l = r + 16c (c = 0..3) of
// that row, lane c with the group's values 16c .. 16c + 15 as lo, hi: the
// group's absmax over the four lanes (two xor shuffles, taken once by every
// lane -- a shuffle under a lane mask reads 0 from inactive source lanes), its
// fp16 scale, and the lane's 16 codes as two dwords (d0: values 16c .. 16c+7).
// Every lane of the wave must call it.
__device__ __forceinline__ _Float16 quantize_group_row4(v8h lo, v8h hi, uint32_t& d0, uint32_t& d1) {
  uint32_t amb = absmax8_bits(hi, absmax8_bits(lo, 0u));
  const uint32_t o16 = (uint32_t)__shfl_xor((int)amb, 16);
  amb = amb > o16 ? amb : o16;
  const uint32_t o32 = (uint32_t)__shfl_xor((int)amb, 32);
  amb = amb > o32 ? amb : o32;
  const float am = half_bits_to_float((uint16_t)amb);
  const _Float16 s = group_scale(am);
  const float sf = (float)s;
  const float rs = __builtin_amdgcn_rcpf(sf);
  d0 = quantize8(lo, sf, rs);
  d1 = quantize8(hi, sf, rs);
  return s;
}

}  // namespace w4a4
