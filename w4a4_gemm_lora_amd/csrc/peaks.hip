// Measured peaks of the resources the layer is bound by (declared in
// include/w4a4_peaks.h): dense int8 MFMA issue, HBM read bandwidth, the
// unpacked fp32 VALU rate of its per-group epilogue, and how far integer
// MFMA and fp32 VALU work of different waves of one SIMD run at the same
// time.  The roofline fractions are taken against the published peaks; these
// give the attainable figures of the same machine beside them.  Measurement
// only: nothing on the layer's path calls them.
#include "w4a4_peaks.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef uint32_t v4u __attribute__((ext_vector_type(4)));

constexpr int kMfmaWorkgroups = 512;   // 2 per CU of 256: two waves per SIMD
constexpr int kChains = 8;             // independent accumulators per wave

// Every wave issues iters x 8 v_mfma_i32_16x16x64_i8 on 8 independent
// accumulators (a 16 x 16 x 64 int8 product each, 32768 ops), then writes
// one value per lane so that nothing is dead.
__global__ __launch_bounds__(256, 2) void peak_i8_mfma_kernel(int iters, int32_t* out) {
  const int lane = threadIdx.x & 63;
  const v4i a = {lane, lane * 3, lane * 5, lane * 7};
  const v4i b = {lane * 11, lane * 13, 17, 19};
  v4i acc[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) acc[i] = v4i{i, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kChains; ++i) acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[i], 0, 0, 0);
  }
  v4i s = acc[0];
#pragma unroll
  for (int i = 1; i < kChains; ++i) s += acc[i];
  out[blockIdx.x * 256 + threadIdx.x] = s[0] ^ s[1] ^ s[2] ^ s[3];
}

// Grid-stride 16-byte non-temporal loads over n16 16-byte chunks, folded by
// xor into one value per thread.
__global__ __launch_bounds__(256) void peak_hbm_read_kernel(const v4u* __restrict__ src, uint64_t n16,
                                                            uint32_t* __restrict__ out) {
  const uint64_t tid = (uint64_t)blockIdx.x * 256 + threadIdx.x;
  const uint64_t stride = (uint64_t)gridDim.x * 256;
  uint32_t x = 0;
  for (uint64_t i = tid; i < n16; i += stride) {
    const v4u v = __builtin_nontemporal_load(src + i);
    x ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  out[tid] = x;
}

constexpr int kReadWorkgroups = 256 * 8;

// fp32 FMA issue: every wave iters x 32 independent accumulating FMAs
// (wave64), acc += x * y with x and y in VGPRs: the two-operand v_fmac_f32
// form the GEMM's fmas take.  (An FMA with an SGPR multiplicand and an inline
// constant addend issues at about half that rate on gfx950.)
template <int N>
__device__ __forceinline__ float fma_chains(int iters, int lane) {
  float f[N];
#pragma unroll
  for (int i = 0; i < N; ++i) f[i] = (float)(lane + i);
  const float x = 1.0001f + (float)lane * 1e-9f, y = 0.5f - (float)lane * 1e-9f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = __builtin_fmaf(x, y, f[i]);
  }
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < N; ++i) r += f[i];
  return r;
}

__device__ __forceinline__ int32_t mfma_chains(int iters, int lane) {
  const v4i a = {lane, lane * 3, lane * 5, lane * 7};
  const v4i b = {lane * 11, lane * 13, 17, 19};
  v4i acc[kChains];
#pragma unroll
  for (int i = 0; i < kChains; ++i) acc[i] = v4i{i, 0, 0, 0};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < kChains; ++i) acc[i] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, acc[i], 0, 0, 0);
  }
  v4i s = acc[0];
#pragma unroll
  for (int i = 1; i < kChains; ++i) s += acc[i];
  return s[0] ^ s[1] ^ s[2] ^ s[3];
}

typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v4h __attribute__((ext_vector_type(4)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

// The GEMM loop's work per 16 x 16 tile, 8 tiles per iteration: an int8 MFMA
// (a B operand of its own, C the same constant every time, as the
// group-sum MFMAs start from fixed bits) and, on the sums of the tile before,
// 4 fp32 fmas and 2 integer ops (the kind the nibble expansion issues).
// MFMA and VALU select the halves, so the same stream can be timed whole and
// by parts.
template <bool MFMA, bool VALU>
__device__ __forceinline__ int32_t tile_mix(int iters, int lane) {
  v4i a = {lane, lane * 3, lane * 5, lane * 7};
  v4i b[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) b[t] = v4i{lane * 11 + t, lane * 13 - t, 17 * t, 19 + t};
  const v4i c0 = {0x40400000, 0x40400000, 0x40400000, 0x40400000};
  v4i d[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) d[t] = c0;
  v4f acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};
  const v4f sc = {1.0001f, 0.9999f, 1.0002f, 0.9998f};
  const v4f other = {0.5f, 0.25f, 0.125f, 0.0625f};
  uint32_t e0 = lane, e1 = lane * 7;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if constexpr (MFMA) d[t] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b[t], c0, 0, 0, 0);
      if constexpr (VALU) {
        const v4f src = MFMA ? __builtin_bit_cast(v4f, d[(t + 7) & 7]) : other;
#pragma unroll
        for (int q = 0; q < 4; ++q) acc[t][q] = __builtin_fmaf(sc[q], src[q], acc[t][q]);
        e0 = ((e0 << 4) & 0xF0F0F0F0u) ^ (uint32_t)t;
        e1 = (e1 & 0xF0F0F0F0u) + e0;
      }
    }
    a[0] ^= (int)e1;
  }
  float r = (float)e0 + (float)e1;
#pragma unroll
  for (int t = 0; t < 8; ++t) r += acc[t][0] + acc[t][1] + acc[t][2] + acc[t][3] + (float)(d[t][0] ^ d[t][3]);
  return __builtin_bit_cast(int32_t, r);
}

// 8 independent chains of one f16 MFMA form (the scale-product and offset
// forms of the GEMM, and the K = 32 form), for their issue cost.
template <int FORM>   // 0: 16x16x4 with 4 blocks, 1: 16x16x32
__device__ __forceinline__ int32_t f16_mfma_chains(int iters, int lane) {
  v4h a4[8];
  v8h a8[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    a4[t] = v4h{(_Float16)(lane + t), (_Float16)1, (_Float16)2, (_Float16)t};
    a8[t] = v8h{(_Float16)(lane + t), (_Float16)1, (_Float16)2, (_Float16)t,
                (_Float16)3, (_Float16)4, (_Float16)5, (_Float16)6};
  }
  v16f c16[8];
  v4f c4[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    c16[t] = v16f{};
    c4[t] = v4f{};
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      if constexpr (FORM == 0) c16[t] = __builtin_amdgcn_mfma_f32_16x16x4f16(a4[t], a4[(t + 1) & 7], c16[t], 0, 0, 0);
      else c4[t] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a8[t], a8[(t + 1) & 7], c4[t], 0, 0, 0);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if constexpr (FORM == 0) {
#pragma unroll
      for (int q = 0; q < 16; ++q) r += c16[t][q];
    } else {
      r += c4[t][0] + c4[t][1] + c4[t][2] + c4[t][3];
    }
  }
  return __builtin_bit_cast(int32_t, r);
}

// Role-split workgroups of 8 waves, one per CU: waves 0..3 (one per SIMD)
// take role A, waves 4..7 role B.  Roles: 0 none, 1 int8 MFMA chains (8 per
// iteration), 2 fp32 FMA chains (32 per iteration), 3 the GEMM's tile mix
// (tile_mix), 4 its MFMA part alone, 5 its VALU part alone, 6 and 7 f16 MFMA
// chains (16x16x4 4-block, 16x16x32).  One value per lane out.
__global__ __launch_bounds__(512, 1) void peak_roles_kernel(int role_a, int role_b, int iters_a, int iters_b,
                                                            int32_t* out) {
  const int lane = threadIdx.x & 63;
  const int role = threadIdx.x < 256 ? role_a : role_b;
  const int iters = threadIdx.x < 256 ? iters_a : iters_b;
  int32_t r = 0;
  if (role == 1) r = mfma_chains(iters, lane);
  else if (role == 2) r = __builtin_bit_cast(int32_t, fma_chains<32>(iters, lane));
  else if (role == 3) r = tile_mix<true, true>(iters, lane);
  else if (role == 4) r = tile_mix<true, false>(iters, lane);
  else if (role == 5) r = tile_mix<false, true>(iters, lane);
  else if (role == 6) r = f16_mfma_chains<0>(iters, lane);
  else if (role == 7) r = f16_mfma_chains<1>(iters, lane);
  out[blockIdx.x * 512 + threadIdx.x] = r;
}

constexpr int kRoleWorkgroups = 256;

}  // namespace

extern "C" {

int64_t w4a4_peak_i8_mfma_ops(int32_t iters) {
  return (int64_t)kMfmaWorkgroups * 4 * kChains * iters * (2LL * 16 * 16 * 64);
}

int64_t w4a4_peak_i8_mfma_out_ints(void) { return (int64_t)kMfmaWorkgroups * 256; }

int w4a4_peak_i8_mfma(int32_t iters, int32_t* out, void* stream) {
  if (iters < 1 || !out) return 4;
  peak_i8_mfma_kernel<<<kMfmaWorkgroups, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(iters, out);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int64_t w4a4_peak_hbm_read_out_ints(void) { return (int64_t)kReadWorkgroups * 256; }

int64_t w4a4_peak_roles_out_ints(void) { return (int64_t)kRoleWorkgroups * 512; }

int64_t w4a4_peak_roles_ops(int32_t role, int32_t iters) {
  const int64_t waves = (int64_t)kRoleWorkgroups * 4;
  if (role == 1) return waves * kChains * iters * (2LL * 16 * 16 * 64);   // int8 ops
  if (role == 2) return waves * 32 * iters * 64;                        // fp32 FMA lane operations
  return 0;
}

int w4a4_peak_roles(int32_t role_a, int32_t role_b, int32_t iters_a, int32_t iters_b, int32_t* out,
                    void* stream) {
  if (role_a < 0 || role_a > 7 || role_b < 0 || role_b > 7 || iters_a < 0 || iters_b < 0 || !out) return 4;
  peak_roles_kernel<<<kRoleWorkgroups, 512, 0, reinterpret_cast<hipStream_t>(stream)>>>(role_a, role_b, iters_a,
                                                                                        iters_b, out);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

int w4a4_peak_hbm_read(const void* src, uint64_t bytes, uint32_t* out, void* stream) {
  if (!src || !out || bytes % 16 != 0 || (reinterpret_cast<uintptr_t>(src) & 15) != 0) return 4;
  peak_hbm_read_kernel<<<kReadWorkgroups, 256, 0, reinterpret_cast<hipStream_t>(stream)>>>(
      static_cast<const v4u*>(src), bytes / 16, out);
  return hipGetLastError() == hipSuccess ? 0 : 5;
}

}  // extern "C"
