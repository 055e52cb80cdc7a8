// W4A4 GEMM with per-group fp32 dequant, fused LoRA-up and column affine.
//
// Method: "W4A4 CUDA Kernel for Voice Clone", section 3.7 -- an integer main
// loop over K in 64-wide groups, each group's exact integer sum scaled by the
// activation and weight scales and accumulated; the LoRA-up product added to
// the same register accumulator; one store of Y.  The column-wise affine
// follows "High-Performance Kernel Design for W4A4 ... on Blackwell",
// section 1.
//
// gfx950 has no 4-bit integer MFMA, so every lane expands its nibbles to
// int8 (16*q per byte, see expand_group) in registers and issues
// v_mfma_i32_16x16x64_i8 once per (16x16 output tile, group) with a zero C,
// which yields 256*P exactly.  The fp32 epilogue per group folds the 1/256
// into the weight scale.  LoRA-up runs on v_mfma_f32_16x16x16_f16 with the
// fp32 lora_act split into fp16 hi + lo parts, accumulating straight into the
// main accumulator; the affine and the fp16 rounding follow in registers.
#include "device_common.hpp"
#include "w4a4_internal.hpp"

namespace w4a4 {

// ---------------------------------------------------------------------------
// Generic kernel: 4 waves in a 2 x 2 arrangement, each wave TM x TN tiles of
// 16 x 16.  Operand fragments come straight from global memory: the packed
// layouts are lane-ordered, so each 16 x 128 tile is one coalesced 1 KB read
// by a wave.  PSUM=true swaps the epilogue for a store of the integer group
// sums (diagnostic window [mt_base, mt_end) x [nt_base, nt_end) in tiles).
// ---------------------------------------------------------------------------
template <int TM, int TN, int RT, bool PSUM>
__global__ __launch_bounds__(256) void gemm_generic_kernel(
    GemmArgs g, int64_t mt_base, int64_t mt_end, int64_t nt_base, int64_t nt_end,
    int32_t* __restrict__ psum, int64_t psum_nc) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t mt0 = mt_base + ((int64_t)blockIdx.y * 2 + wm) * TM;
  const int64_t nt0 = nt_base + ((int64_t)blockIdx.x * 2 + wn) * TN;
  const int64_t KP = g.K / kKPair;
  const int64_t G = g.K / kGroup;
  const int c = lane >> 4, col_l = lane & 15;

  bool mv[TM], nv[TN];
#pragma unroll
  for (int i = 0; i < TM; ++i) mv[i] = (mt0 + i) < mt_end;
#pragma unroll
  for (int j = 0; j < TN; ++j) nv[j] = (nt0 + j) < nt_end;

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  const v4i zero = v4i{0, 0, 0, 0};
  for (int64_t p = 0; p < KP; ++p) {
    v4u araw[TM], braw[TN];
    v8h sxv[TM];
    uint32_t swv[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (mv[i]) {
        araw[i] = *reinterpret_cast<const v4u*>(g.xq + ((size_t)(mt0 + i) * KP + p) * kTileBytes + lane * 16);
        sxv[i] = *reinterpret_cast<const v8h*>(g.sx + ((size_t)(mt0 + i) * KP + p) * 32 + c * 8);
      } else {
        araw[i] = v4u{0, 0, 0, 0};
        sxv[i] = v8h{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      if (nv[j]) {
        braw[j] = *reinterpret_cast<const v4u*>(g.wq + ((size_t)(nt0 + j) * KP + p) * kTileBytes + lane * 16);
        swv[j] = *reinterpret_cast<const uint32_t*>(g.sw + ((size_t)(nt0 + j) * KP + p) * 32 + col_l * 2);
      } else {
        braw[j] = v4u{0, 0, 0, 0};
        swv[j] = 0;
      }
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      v4i A[TM], B[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) A[i] = expand_group(araw[i][2 * h], araw[i][2 * h + 1]);
#pragma unroll
      for (int j = 0; j < TN; ++j) B[j] = expand_group(braw[j][2 * h], braw[j][2 * h + 1]);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          v4i P = mfma_i8_16x16x64(A[i], B[j], zero);
          if constexpr (PSUM) {
            if (mv[i] && nv[j]) {
              const int64_t col = (nt0 + j) * 16 + col_l - nt_base * 16;
#pragma unroll
              for (int ii = 0; ii < 4; ++ii) {
                const int64_t row = (mt0 + i) * 16 + c * 4 + ii - mt_base * 16;
                psum[(row * psum_nc + col) * G + 2 * p + h] = P[ii] >> 8;
              }
            }
          } else {
            const float swf = half_bits_to_float((uint16_t)(swv[j] >> (16 * h))) * (1.0f / 256.0f);
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) {
              const float s = (float)sxv[i][ii * 2 + h] * swf;
              acc[i][j][ii] = fmaf((float)P[ii], s, acc[i][j][ii]);
            }
          }
        }
      }
    }
  }
  if constexpr (PSUM) return;

  // LoRA-up: acc += lora_act (hi + lo fp16) x L_up^T on f16 MFMA.
  if constexpr (RT > 0) {
    const int R = RT * 16;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      v4h ahi[TM], alo[TM], bl[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        v4f la = v4f{0.f, 0.f, 0.f, 0.f};
        if (mv[i]) la = *reinterpret_cast<const v4f*>(g.la + ((size_t)((mt0 + i) * 16 + col_l)) * R + t * 16 + c * 4);
        split_f16(la, ahi[i], alo[i]);
      }
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        bl[j] = v4h{0, 0, 0, 0};
        if (nv[j]) bl[j] = *reinterpret_cast<const v4h*>(g.lup + (((size_t)(nt0 + j) * RT + t) * 64 + lane) * 4);
      }
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          acc[i][j] = mfma_f16_16x16x16(ahi[i], bl[j], acc[i][j]);
          acc[i][j] = mfma_f16_16x16x16(alo[i], bl[j], acc[i][j]);
        }
    }
  }

  // Affine + fp16 store (rows >= M are padding and never written).
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    if (!nv[j]) continue;
    const int64_t col = (nt0 + j) * 16 + col_l;
    const float af = g.ca[col], bf = g.cb[col];
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      if (!mv[i]) continue;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int64_t row = (mt0 + i) * 16 + c * 4 + ii;
        if (row < g.M) {
          const _Float16 v = (_Float16)fmaf(af, acc[i][j][ii], bf);
          g.y[row * g.ldy + col] = __builtin_bit_cast(uint16_t, v);
        }
      }
    }
  }
}

template <int TM, int TN, bool PSUM>
static hipError_t launch_generic_rt(const GemmArgs& a, int64_t mt_base, int64_t mt_end,
                                    int64_t nt_base, int64_t nt_end, int32_t* psum,
                                    int64_t psum_nc, hipStream_t stream) {
  const int64_t mtiles = mt_end - mt_base, ntiles = nt_end - nt_base;
  dim3 grid((unsigned)((ntiles + 2 * TN - 1) / (2 * TN)), (unsigned)((mtiles + 2 * TM - 1) / (2 * TM)));
  switch (PSUM ? 0 : a.R / 16) {
    case 0: gemm_generic_kernel<TM, TN, 0, PSUM><<<grid, 256, 0, stream>>>(a, mt_base, mt_end, nt_base, nt_end, psum, psum_nc); break;
    case 1: gemm_generic_kernel<TM, TN, 1, PSUM><<<grid, 256, 0, stream>>>(a, mt_base, mt_end, nt_base, nt_end, psum, psum_nc); break;
    case 2: gemm_generic_kernel<TM, TN, 2, PSUM><<<grid, 256, 0, stream>>>(a, mt_base, mt_end, nt_base, nt_end, psum, psum_nc); break;
    case 3: gemm_generic_kernel<TM, TN, 3, PSUM><<<grid, 256, 0, stream>>>(a, mt_base, mt_end, nt_base, nt_end, psum, psum_nc); break;
    case 4: gemm_generic_kernel<TM, TN, 4, PSUM><<<grid, 256, 0, stream>>>(a, mt_base, mt_end, nt_base, nt_end, psum, psum_nc); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

int choose_variant(int64_t M, int64_t N, int64_t K, int R) {
  (void)M; (void)N; (void)K; (void)R;
  return kGeneric;
}

hipError_t launch_gemm(const GemmArgs& a, int variant, hipStream_t stream) {
  const int64_t mt = round_up16(a.M) / 16, nt = a.N / 16;
  switch (variant) {
    default:
      return launch_generic_rt<2, 2, false>(a, 0, mt, 0, nt, nullptr, 0, stream);
  }
}

hipError_t launch_group_psums(const GemmArgs& a, int64_t m0, int64_t mc, int64_t n0,
                              int64_t nc, int32_t* out, hipStream_t stream) {
  return launch_generic_rt<2, 2, true>(a, m0 / 16, (m0 + mc) / 16, n0 / 16, (n0 + nc) / 16, out, nc, stream);
}

}  // namespace w4a4
