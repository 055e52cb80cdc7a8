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

// fp32 FMA issue: every wave iters x 32 independent v_fma_f32 (wave64).
template <int N>
__device__ __forceinline__ float fma_chains(int iters, int lane) {
  float f[N];
#pragma unroll
  for (int i = 0; i < N; ++i) f[i] = (float)(lane + i);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int i = 0; i < N; ++i) f[i] = __builtin_fmaf(f[i], 1.0001f, 0.5f);
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

// Role-split workgroups of 8 waves, one per CU: waves 0..3 (one per SIMD)
// take role A, waves 4..7 role B.  Roles: 0 none, 1 int8 MFMA chains (8 per
// iteration), 2 fp32 FMA chains (32 per iteration).  One value per lane out.
__global__ __launch_bounds__(512, 1) void peak_roles_kernel(int role_a, int role_b, int iters_a, int iters_b,
                                                            int32_t* out) {
  const int lane = threadIdx.x & 63;
  const int role = threadIdx.x < 256 ? role_a : role_b;
  const int iters = threadIdx.x < 256 ? iters_a : iters_b;
  int32_t r = 0;
  if (role == 1) r = mfma_chains(iters, lane);
  else if (role == 2) r = __builtin_bit_cast(int32_t, fma_chains<32>(iters, lane));
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
  if (role_a < 0 || role_a > 2 || role_b < 0 || role_b > 2 || iters_a < 0 || iters_b < 0 || !out) return 4;
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
