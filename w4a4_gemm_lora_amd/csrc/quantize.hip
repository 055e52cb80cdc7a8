// Activation quantizer with fused LoRA-down, and the offline weight packers.
//
// Method: "W4A4 CUDA Kernel for Voice Clone", section 3.6 -- one read of X
// feeds both the int4 quantizer (per (row, 64-group) absmax, scale absmax/7,
// round to nearest, clamp to [-8, 7], 4-bit two's-complement codes) and the
// LoRA down-projection lora_act = X L_down on the fp16 values.  Section 2.3 /
// 3.10: weights are repacked once at load into the kernel's layout.
//
// gfx950 design: one workgroup per 16-row tile, W = min(16, K/128) waves; a
// wave owns whole 16 x 128 k-pairs.  Lane l = r + 16c loads the 32 fp16 values
// of row r at k = 128p + 64j + 16c + [0,16) (j = group in the pair) with four
// 128-bit loads, and those registers serve three purposes without any LDS
// staging: the absmax (reduced over the four lanes of a row with two xor
// shuffles), the codes (written as one 128-bit store per lane: the packed
// tile is laid out in load order), and the A operand of the f16 MFMA that
// computes LoRA-down (L_down is pre-packed so that its B operand pairs every
// lane's k values with the same k).  The per-wave LoRA partials are summed
// in LDS in a fixed wave order, so results are deterministic (no atomics and
// no separate repack kernel for lora_act).
#include "device_common.hpp"
#include "w4a4_internal.hpp"

namespace w4a4 {

// Codes for 8 values (one dword) with scale `sf`, per the quantizer rule.
// The fp32 division is IEEE (correctly rounded); rintf rounds half to even.
__device__ __forceinline__ uint32_t quantize8(v8h v, float sf) {
  uint32_t out = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    float t = rintf((float)v[i] / sf);
    t = fminf(fmaxf(t, -8.0f), 7.0f);
    int q = (int)t;
    out |= (uint32_t(q) & 0xFu) << (4 * i);
  }
  return out;
}

__device__ __forceinline__ float absmax8(v8h v, float m) {
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf((float)v[i]));
  return m;
}

// Scale of a group from its absmax: fp16(fp32(amax / 7)); 0 -> 2^-24.
__device__ __forceinline__ _Float16 group_scale(float amax) {
  float s32 = amax / 7.0f;
  _Float16 s = (_Float16)s32;
  if (s == (_Float16)0.0f) s = __builtin_bit_cast(_Float16, (uint16_t)1);
  return s;
}

template <int RT>  // RT = R / 16 (0 = no LoRA)
__global__ __launch_bounds__(1024) void quantize_rows_kernel(
    const uint16_t* __restrict__ src, int64_t ld, int64_t rows, int64_t K,
    const uint16_t* __restrict__ ldown, uint8_t* __restrict__ codes,
    uint16_t* __restrict__ scales, float* __restrict__ lora_act) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int nwaves = blockDim.x >> 6;
  const int r = lane & 15, c = lane >> 4;
  const int64_t rt = blockIdx.x;
  const int64_t row = rt * 16 + r;
  const bool valid = row < rows;
  const int64_t KP = K / kKPair;
  const _Float16* xrow = reinterpret_cast<const _Float16*>(src) + (valid ? row * ld : 0);

  v4f acc[RT > 0 ? RT : 1];
#pragma unroll
  for (int t = 0; t < (RT > 0 ? RT : 1); ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  for (int64_t p = wave; p < KP; p += nwaves) {
    v8h v[4];  // v[2j + h]: group j, k = 16c + 8h + [0,8)
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      if (valid) {
        const int64_t k = p * kKPair + (s >> 1) * kGroup + c * 16 + (s & 1) * 8;
        v[s] = *reinterpret_cast<const v8h*>(xrow + k);
      } else {
        v[s] = v8h{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
    uint32_t d[4];
    _Float16 sc[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      float am = absmax8(v[2 * j + 1], absmax8(v[2 * j], 0.0f));
      am = fmaxf(am, __shfl_xor(am, 16));
      am = fmaxf(am, __shfl_xor(am, 32));
      _Float16 s = group_scale(am);
      const float sf = (float)s;
      d[2 * j] = quantize8(v[2 * j], sf);
      d[2 * j + 1] = quantize8(v[2 * j + 1], sf);
      sc[j] = valid ? s : (_Float16)0.0f;
    }
    uint8_t* tile = codes + (size_t)(rt * KP + p) * kTileBytes;
    *reinterpret_cast<v4u*>(tile + lane * 16) = v4u{d[0], d[1], d[2], d[3]};
    if (c == 0) {
      _Float16* sp = reinterpret_cast<_Float16*>(scales) + ((size_t)(rt * KP + p) * 16 + r) * 2;
      sp[0] = sc[0];
      sp[1] = sc[1];
    }
    if constexpr (RT > 0) {
      const _Float16* lp = reinterpret_cast<const _Float16*>(ldown) + (size_t)p * RT * 4 * 64 * 8;
#pragma unroll
      for (int t = 0; t < RT; ++t) {
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          v8h b = *reinterpret_cast<const v8h*>(lp + ((size_t)(t * 4 + s) * 64 + lane) * 8);
          acc[t] = mfma_f16_16x16x32(v[s], b, acc[t]);
        }
      }
    }
  }

  if constexpr (RT > 0) {
    // red[w][t*4 + i][lane]: partial of rows 4c+i, rank 16t + (lane & 15)
    __shared__ float red[16][RT * 4][64];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][t * 4 + i][lane] = acc[t][i];
    __syncthreads();
    const int R = RT * 16;
    for (int e = threadIdx.x; e < RT * 4 * 64; e += blockDim.x) {
      const int ti = e >> 6, l = e & 63;
      float s = 0.0f;
      for (int w = 0; w < nwaves; ++w) s += red[w][ti][l];
      const int t = ti >> 2, i = ti & 3;
      const int64_t orow = rt * 16 + (l >> 4) * 4 + i;
      lora_act[orow * R + t * 16 + (l & 15)] = s;
    }
  }
}

hipError_t launch_quantize_rows(const uint16_t* src, int64_t ld, int64_t rows,
                                int64_t rows_padded, int64_t K, int R,
                                const uint16_t* ldown_packed, uint8_t* codes,
                                uint16_t* scales, float* lora_act,
                                hipStream_t stream) {
  const int64_t KP = K / kKPair;
  const int waves = (int)(KP < 16 ? KP : 16);
  dim3 grid((unsigned)(rows_padded / 16)), block(64 * waves);
  switch (R / 16) {
    case 0: quantize_rows_kernel<0><<<grid, block, 0, stream>>>(src, ld, rows, K, ldown_packed, codes, scales, lora_act); break;
    case 1: quantize_rows_kernel<1><<<grid, block, 0, stream>>>(src, ld, rows, K, ldown_packed, codes, scales, lora_act); break;
    case 2: quantize_rows_kernel<2><<<grid, block, 0, stream>>>(src, ld, rows, K, ldown_packed, codes, scales, lora_act); break;
    case 3: quantize_rows_kernel<3><<<grid, block, 0, stream>>>(src, ld, rows, K, ldown_packed, codes, scales, lora_act); break;
    case 4: quantize_rows_kernel<4><<<grid, block, 0, stream>>>(src, ld, rows, K, ldown_packed, codes, scales, lora_act); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Offline packers ("W4A4 CUDA Kernel for Voice Clone", sections 2.3 and 3.10)
// ---------------------------------------------------------------------------

// Checkpoint codes qweight [N][K/2] (byte j: k = 2j low nibble, 2j+1 high)
// and w_scales [N][K/64] -> W_q tiles and s_w.  A lane's 8 bytes of a group
// are the checkpoint's 8 bytes for k = 16c .. 16c+15, so this is a gather.
__global__ void repack_qweight_kernel(const uint8_t* __restrict__ qweight,
                                      const uint16_t* __restrict__ w_scales,
                                      int64_t K, uint8_t* __restrict__ codes,
                                      uint16_t* __restrict__ scales) {
  const int lane = threadIdx.x;
  const int r = lane & 15, c = lane >> 4;
  const int64_t nt = blockIdx.x, p = blockIdx.y;
  const int64_t KP = K / kKPair, G = K / kGroup;
  const int64_t n = nt * 16 + r;
  const uint8_t* rowp = qweight + n * (K / 2);
  uint8_t* tile = codes + (size_t)(nt * KP + p) * kTileBytes + lane * 16;
#pragma unroll
  for (int j = 0; j < 2; ++j)
#pragma unroll
    for (int b = 0; b < 8; ++b) tile[j * 8 + b] = rowp[p * 64 + j * 32 + c * 8 + b];
  if (c == 0) {
    uint16_t* sp = scales + ((size_t)(nt * KP + p) * 16 + r) * 2;
    sp[0] = w_scales[n * G + 2 * p];
    sp[1] = w_scales[n * G + 2 * p + 1];
  }
}

hipError_t launch_repack_qweight(const uint8_t* qweight, const uint16_t* w_scales,
                                 int64_t N, int64_t K, uint8_t* codes,
                                 uint16_t* scales, hipStream_t stream) {
  dim3 grid((unsigned)(N / 16), (unsigned)(K / kKPair));
  repack_qweight_kernel<<<grid, 64, 0, stream>>>(qweight, w_scales, K, codes, scales);
  return hipGetLastError();
}

// L_up [N][R] -> [N/16][R/16][64][4]:  (nt, t, l = i + 16c, j) = L_up[16nt+i][16t+4c+j]
__global__ void pack_lora_up_kernel(const uint16_t* __restrict__ lup, int R,
                                    uint16_t* __restrict__ out) {
  const int l = threadIdx.x, i = l & 15, c = l >> 4;
  const int64_t nt = blockIdx.x;
  const int t = blockIdx.y, RT = gridDim.y;
  uint16_t* o = out + (((size_t)nt * RT + t) * 64 + l) * 4;
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = lup[(nt * 16 + i) * R + t * 16 + c * 4 + j];
}

// L_down [K][R] -> [K/128][R/16][4][64][8]:
//   (p, t, s, l = n + 16c, j) = L_down[128p + 64(s/2) + 16c + 8(s%2) + j][16t + n]
__global__ void pack_lora_down_kernel(const uint16_t* __restrict__ ldn, int R,
                                      uint16_t* __restrict__ out) {
  const int l = threadIdx.x, n = l & 15, c = l >> 4;
  const int64_t p = blockIdx.x;
  const int t = blockIdx.y, s = blockIdx.z, RT = gridDim.y;
  uint16_t* o = out + ((((size_t)p * RT + t) * 4 + s) * 64 + l) * 8;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t k = p * kKPair + (s >> 1) * kGroup + c * 16 + (s & 1) * 8 + j;
    o[j] = ldn[k * R + t * 16 + n];
  }
}

hipError_t launch_pack_lora(const uint16_t* lora_down, const uint16_t* lora_up,
                            int64_t N, int64_t K, int R, uint16_t* ldown_packed,
                            uint16_t* lup_packed, hipStream_t stream) {
  if (R == 0) return hipSuccess;
  pack_lora_up_kernel<<<dim3((unsigned)(N / 16), R / 16), 64, 0, stream>>>(lora_up, R, lup_packed);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  pack_lora_down_kernel<<<dim3((unsigned)(K / kKPair), R / 16, 4), 64, 0, stream>>>(lora_down, R, ldown_packed);
  return hipGetLastError();
}

__global__ void pack_affine_kernel(const float* __restrict__ cs, const float* __restrict__ bs,
                                   int64_t N, float* __restrict__ a, float* __restrict__ b) {
  const int64_t n = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (n < N) {
    a[n] = cs ? cs[n] : 1.0f;
    b[n] = bs ? bs[n] : 0.0f;
  }
}

hipError_t launch_pack_affine(const float* col_scale, const float* bias, int64_t N,
                              float* a, float* b, hipStream_t stream) {
  pack_affine_kernel<<<(unsigned)((N + 255) / 256), 256, 0, stream>>>(col_scale, bias, N, a, b);
  return hipGetLastError();
}

}  // namespace w4a4
