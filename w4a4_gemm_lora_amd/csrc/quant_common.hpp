// Per-group quantizer arithmetic shared by the activation pass and the
// gated GEMM epilogue that quantizes its own output for the next layer, so
// that both produce the same codes and scales bit for bit ("W4A4 CUDA Kernel
// for Voice Clone", section 3.6: per (row, 64-group) absmax, scale
// absmax / 7 stored in fp16, round to nearest, clamp to [-8, 7], 4-bit
// two's-complement codes).
#pragma once

#include "device_common.hpp"

namespace w4a4 {

typedef uint16_t v2u16 __attribute__((ext_vector_type(2)));

// Codes for 8 values (one dword): q = clamp(rint(fl32(x / s)), -8, 7) with
// round-half-to-even, where s is the group's fp16 scale (sf, exact in fp32)
// and rs ~ 1/s (v_rcp_f32, within 1 ulp).
//
// The quotient takes no division, only one Newton step from rs:
//   t0 = fl(x rs),  e = fma(-t0, s, x),  t = fma(e, rs, t0).
// * e is exact: x is a multiple of 2^(E-10) (its fp16 ulp) and t0 s of
//   2^(E-34) (t0 ~ x/s), and |e| = s |x/s - t0| < |x| 2^-22 < 2^(E-21),
//   so e needs fewer than 14 significant bits.
// * t is fl32 of t0 + e rs = x/s + e (rs - 1/s), whose second term is below
//   |x/s| 2^-45: a 2^-20 fraction of t's ulp.
// * If x/s is a half-integer h, it is an fp32 value, so t == h exactly, and
//   rint's ties-to-even rounds it as the rule does.
// * Otherwise, where |x/s| >= 1/4, x/s lies at least 2^-15 from every
//   half-integer (x = a 2^p, s = b 2^r with integers a, b < 2^11; the gap is
//   a nonzero multiple of min(2^p, 2^r) / (2 b 2^r), and p - r >= -3 there),
//   while |x/s| < 11 puts t within 2^-20 of it: rint(t) is the integer
//   nearest x/s, which is rint(fl32(x/s)).  Where |x/s| < 1/4 both give 0.
// No compare, select or branch is needed for ties.
//
// Packing: for an integer n in [-8, 7] and j < 4, n + 1.5 * 2^(23 - 4j) is
// exact and its bit pattern holds n << 4j (two's complement) in bits
// [4j, 4j + 4), so one and-or puts a code in place within a 16-bit half.
__device__ __forceinline__ uint32_t quantize8(v8h v, float sf, float rs) {
  // two 16-bit halves, each built with the biases 1.5 * 2^(23 - 4j), j < 4,
  // whose own set bits (22 and up) stay clear of bits [0, 16)
  uint32_t half[2] = {0u, 0u};
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int j = i & 3;
    const float x = (float)v[i];
    const float t0 = x * rs;
    const float e = __builtin_fmaf(-t0, sf, x);
    const float t = __builtin_fmaf(e, rs, t0);
    const float q = __builtin_amdgcn_fmed3f(__builtin_rintf(t), -8.0f, 7.0f);
    const float biased = q + __builtin_ldexpf(1.5f, 23 - 4 * j);   // constant per i
    half[i >> 2] |= __builtin_bit_cast(uint32_t, biased) & (0xFu << (4 * j));
  }
  return half[0] | (half[1] << 16);
}

// max |x| over 8 fp16 values, two lanes of 16 bits at a time: for fp16, |x|
// orders like (bits & 0x7fff) as unsigned integers, so the max is taken on the
// bit patterns (packed u16 max).
__device__ __forceinline__ v2u16 absmax8_pk(v8h v, v2u16 m) {
  const v4u w = __builtin_bit_cast(v4u, v);
#pragma unroll
  for (int i = 0; i < 4; ++i) m = __builtin_elementwise_max(m, __builtin_bit_cast(v2u16, w[i] & 0x7FFF7FFFu));
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
  const v2u16 pk = absmax8_pk(hi, absmax8_pk(lo, v2u16{0, 0}));
  uint32_t amb = pk[0] > pk[1] ? pk[0] : pk[1];
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
