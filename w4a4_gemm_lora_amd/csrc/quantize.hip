// Activation quantizer with fused LoRA-down, and the offline weight packers.
//
// Method: "W4A4 CUDA Kernel for Voice Clone", section 3.6 -- one read of X
// feeds both the int4 quantizer (per (row, 64-group) absmax, scale absmax/7,
// round to nearest, clamp to [-8, 7], 4-bit two's-complement codes) and the
// LoRA down-projection lora_act = X L_down on the fp16 values.  Section 2.3 /
// 3.10: weights are repacked once at load into the kernel's layout.
//
// gfx950 design: one workgroup of 2, 4, 8 or 16 waves per (16-row tile, k-pair
// range); a wave owns whole 16 x 128 k-pairs.  Lane l = r + 16c loads the 32 fp16 values
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
#include "quant_common.hpp"
#include "w4a4_internal.hpp"

namespace w4a4 {

// Grid (rows_padded/16 * 16/rh, ks) x NW waves.  Workgroup (x, j) handles
// rows [r0, r0 + rh) of the 16-row tile rt = x / (16/rh), r0 = (x % (16/rh)) *
// rh, and the k-pairs [j*KP/ks, (j+1)*KP/ks); its waves take every NW-th
// k-pair.  The wave works on whole tiles (lanes of other rows read zeros) but
// stores only its own rows' codes, scales and lora_act rows, so splitting a
// tile's rows over 2 workgroups doubles the parallelism of small M without
// partial sums (every such workgroup reads the whole L_down slice of its K
// range, which is why tiles are not split further).  NW (2, 4, 8 or 16)
// follows the number of k-pairs per workgroup so that few row tiles still
// give many waves.
//
// NORM: the rows are RMS-normalized first ("W4A4 CUDA Kernel for Voice
// Clone", sections 3.1 and 3.9: the RMSNorm ahead of the projections and its
// 1/sqrt(mean(x^2) + eps) over all of K).  Phase 1: every wave sums x^2 in
// fp64 over its share of the row's k-pairs -- all of K, also when K is split
// over workgroups -- and the sums meet in LDS in a fixed wave order; inv =
// 1/sqrt(sum/K + eps) in fp64.  Phase 2 quantizes and feeds LoRA-down with
// fp16(fp32((x * inv) * gamma[k])) (fp64 products, in that order) in place of
// x.  Phase 1's loads are re-read in phase 2 (from L2).
template <int RT, int NW, bool NORM>  // RT = R / 16 (0 = no LoRA)
__global__ __launch_bounds__(NW * 64) void quantize_rows_kernel(
    const uint16_t* __restrict__ src, int64_t ld, int64_t rows, int64_t rows_padded, int64_t K,
    const uint16_t* __restrict__ ldown, uint8_t* __restrict__ codes,
    uint16_t* __restrict__ scales, float* __restrict__ lora_part, int rh,
    const uint16_t* __restrict__ gamma, double eps) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // uniform: scalar loop control
  const int r = lane & 15, c = lane >> 4;
  const int64_t rt = blockIdx.x / (16 / rh);
  const int r0 = (int)(blockIdx.x % (16 / rh)) * rh;
  const int64_t row = rt * 16 + r;
  const bool mine = r >= r0 && r < r0 + rh;   // this workgroup stores row r
  const bool valid = mine && row < rows;
  const int64_t KP = K / kKPair;
  const int64_t ks = gridDim.y, j = blockIdx.y;
  const int64_t pbeg = j * KP / ks, pend = (j + 1) * KP / ks;
  const _Float16* xrow = reinterpret_cast<const _Float16*>(src) + (valid ? row * ld : 0);

  v4f acc[RT > 0 ? RT : 1];
#pragma unroll
  for (int t = 0; t < (RT > 0 ? RT : 1); ++t) acc[t] = v4f{0.f, 0.f, 0.f, 0.f};

  // Unconditional loads (lanes of rows this workgroup does not own, or past
  // M, read row 0 of X and are zeroed afterwards): no lane-divergent branch
  // around the loads, so the compiler's vmcnt waits stay exact.
  auto issue_x = [&](int64_t p, v8h* v) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int64_t k = p * kKPair + (s >> 1) * kGroup + c * 16 + (s & 1) * 8;
      v[s] = *reinterpret_cast<const v8h*>(xrow + k);   // (non-temporal loads measured 16% slower at 8192 x 4096)
    }
  };
  auto mask_x = [&](v8h* v) {
#pragma unroll
    for (int s = 0; s < 4; ++s) v[s] = valid ? v[s] : v8h{0, 0, 0, 0, 0, 0, 0, 0};
  };
  auto load_raw = [&](int64_t p, v8h* v) {
    issue_x(p, v);
    mask_x(v);
  };

  double inv = 1.0;   // 1/rms of row r (NORM)
  if constexpr (NORM) {
    __shared__ double ssq[NW][16];
    double ss = 0.0;
    for (int64_t p = wave; p < KP; p += NW) {
      v8h v[4];
      load_raw(p, v);
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double d = (double)(float)v[s][i];
          ss = __builtin_fma(d, d, ss);   // d * d is exact
        }
    }
    ss += __shfl_xor(ss, 16);   // the four lanes of row r
    ss += __shfl_xor(ss, 32);
    if (c == 0) ssq[wave][r] = ss;
    __syncthreads();
    double tot = ssq[0][r];
#pragma unroll
    for (int w = 1; w < NW; ++w) tot += ssq[w][r];
    inv = 1.0 / __builtin_sqrt(tot / (double)K + eps);
  }

  // the loaded k-pair of X as the quantizer takes it: masked, and
  // normalized under NORM (gm: gamma at the lane's 32 columns)
  auto finish_x = [&](const v8h* gm, v8h* v) {
    mask_x(v);
    if constexpr (NORM) {
      // No contraction here: under it the backend may merge the two
      // conversions fp64 -> fp32 -> fp16 into one rounding fp64 -> fp16,
      // which differs from the two-step rounding where the first lands on an
      // fp16 tie.
#pragma clang fp contract(off)
#pragma unroll
      for (int s = 0; s < 4; ++s)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const double t = ((double)(float)v[s][i] * inv) * (double)(float)gm[s][i];
          v[s][i] = (_Float16)(float)t;
        }
    }
  };

  // One k-pair.  Its L_down fragments (L2-resident, shared by every row
  // tile) and, under NORM, gamma are loaded first, then the next k-pair's X
  // into `nxt`, so that the LoRA MFMAs' wait for L_down leaves the next X in
  // flight while this one is quantized.  The next index is clamped to a
  // k-pair of the range, so the loads need no branch; on a wave's last
  // k-pair they re-read the current one, from cache.
  auto step = [&](int64_t p, v8h* cur, v8h* nxt) {
    constexpr int RTL = RT > 0 ? RT : 1;
    v8h lb[RTL][4];
    if constexpr (RT > 0) {
      const _Float16* lp = reinterpret_cast<const _Float16*>(ldown) + (size_t)p * RT * 4 * 64 * 8;
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s) lb[t][s] = *reinterpret_cast<const v8h*>(lp + ((size_t)(t * 4 + s) * 64 + lane) * 8);
    }
    v8h gm[NORM ? 4 : 1];
    if constexpr (NORM) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int64_t k = p * kKPair + (s >> 1) * kGroup + c * 16 + (s & 1) * 8;
        gm[s] = *reinterpret_cast<const v8h*>(reinterpret_cast<const _Float16*>(gamma) + k);
      }
    }
    // every L_down and gamma load ahead of the X loads, and those ahead of
    // this k-pair's arithmetic
    __builtin_amdgcn_sched_barrier(0);
    issue_x(p + NW < pend ? p + NW : p, nxt);
    __builtin_amdgcn_sched_barrier(0);
    finish_x(gm, cur);
    uint32_t d[4];
    _Float16 sc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const _Float16 s = quantize_group_row4(cur[2 * h], cur[2 * h + 1], d[2 * h], d[2 * h + 1]);
      sc[h] = valid ? s : (_Float16)0.0f;
    }
    uint8_t* tile = codes + (size_t)(rt * KP + p) * kTileBytes;
    if (mine) *reinterpret_cast<v4u*>(tile + lane * 16) = v4u{d[0], d[1], d[2], d[3]};
    if (c == 0 && mine) {
      _Float16* sp = reinterpret_cast<_Float16*>(scales) + ((size_t)(rt * KP + p) * 16 + r) * 2;
      *reinterpret_cast<uint32_t*>(sp) =
          uint32_t(__builtin_bit_cast(uint16_t, sc[0])) | (uint32_t(__builtin_bit_cast(uint16_t, sc[1])) << 16);
    }
    if constexpr (RT > 0) {
#pragma unroll
      for (int t = 0; t < RT; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[t] = mfma_f16_16x16x32(cur[s], lb[t][s], acc[t]);
    }
  };

  // The wave's k-pairs pbeg + wave, + NW, ... two per trip, the X buffers
  // alternating so that no register copy waits on a load in flight.  The
  // trip count is uniform and each trip straight-line, so every path into
  // the loop head has the same loads in flight (a break between the two
  // steps would add one with the other buffer still loading, and the
  // compiler would drain every load there).  pbeg < pend: the activation
  // layout never splits K into more ranges than k-pairs.
  v8h xa[4], xb[4];
  int64_t p = pbeg + wave;
  const int64_t n = p < pend ? (pend - p + NW - 1) / NW : 0;   // this wave's k-pairs
  issue_x(p < pend ? p : pbeg, xa);
  for (int64_t i = 0; i + 2 <= n; i += 2, p += 2 * NW) {
    step(p, xa, xb);
    step(p + NW, xb, xa);
  }
  if (n & 1) step(p, xa, xb);

  if constexpr (RT > 0) {
    // red[w][t*4 + i][lane]: partial of rows 4c+i, rank 16t + (lane & 15);
    // summed over the waves in order (deterministic)
    __shared__ float red[NW][RT * 4][64];
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[wave][t * 4 + i][lane] = acc[t][i];
    __syncthreads();
    const int R = RT * 16;
    float* out = lora_part + (size_t)j * rows_padded * R;
    for (int e = threadIdx.x; e < RT * 4 * 64; e += blockDim.x) {
      const int ti = e >> 6, l = e & 63;
      const int t = ti >> 2, i = ti & 3;
      const int lr = (l >> 4) * 4 + i;   // row within the tile
      if (lr < r0 || lr >= r0 + rh) continue;
      float s = 0.0f;
#pragma unroll
      for (int w = 0; w < NW; ++w) s += red[w][ti][l];
      out[(rt * 16 + lr) * R + t * 16 + (l & 15)] = s;
    }
  }
}

// Sixteen waves leave each lane 128 registers: enough for the plain pass up
// to rank 32 and for the RMSNorm pass (whose phase-1 fp64 state stays live)
// up to rank 16; beyond, the instances would spill, so they are not built.
constexpr int max_rank_16_waves(bool norm) { return norm ? 16 : 32; }

template <int RT, int NW, bool NORM>
static void launch_quantize_rt(dim3 grid, dim3 block, hipStream_t stream, const uint16_t* src, int64_t ld,
                               int64_t rows, int64_t rows_padded, int64_t K, const uint16_t* ldown_packed,
                               uint8_t* codes, uint16_t* scales, float* lora_part, int rh,
                               const uint16_t* gamma, double eps) {
  if constexpr (NW < 16 || 16 * RT <= max_rank_16_waves(NORM))
    quantize_rows_kernel<RT, NW, NORM><<<grid, block, 0, stream>>>(src, ld, rows, rows_padded, K, ldown_packed,
                                                                   codes, scales, lora_part, rh, gamma, eps);
}

template <int NW, bool NORM>
static hipError_t launch_quantize_nw(const uint16_t* src, int64_t ld, int64_t rows,
                                     int64_t rows_padded, int64_t K, int R, int ks,
                                     const uint16_t* ldown_packed, uint8_t* codes,
                                     uint16_t* scales, float* lora_part, const uint16_t* gamma,
                                     double eps, hipStream_t stream) {
  // rows per workgroup: 8 (tiles split in two) when there are < 256 workgroups
  int rh = 16;
  while (rh > 8 && rows_padded / 16 * (16 / rh) * ks < 256) rh /= 2;
  dim3 grid((unsigned)(rows_padded / 16 * (16 / rh)), (unsigned)ks), block(64 * NW);
  if (NW == 16 && R > max_rank_16_waves(NORM)) return hipErrorInvalidValue;   // not built (see above)
  switch (R / 16) {
    case 0: launch_quantize_rt<0, NW, NORM>(grid, block, stream, src, ld, rows, rows_padded, K, ldown_packed, codes, scales, lora_part, rh, gamma, eps); break;
    case 1: launch_quantize_rt<1, NW, NORM>(grid, block, stream, src, ld, rows, rows_padded, K, ldown_packed, codes, scales, lora_part, rh, gamma, eps); break;
    case 2: launch_quantize_rt<2, NW, NORM>(grid, block, stream, src, ld, rows, rows_padded, K, ldown_packed, codes, scales, lora_part, rh, gamma, eps); break;
    case 3: launch_quantize_rt<3, NW, NORM>(grid, block, stream, src, ld, rows, rows_padded, K, ldown_packed, codes, scales, lora_part, rh, gamma, eps); break;
    case 4: launch_quantize_rt<4, NW, NORM>(grid, block, stream, src, ld, rows, rows_padded, K, ldown_packed, codes, scales, lora_part, rh, gamma, eps); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool NORM>
static hipError_t launch_quantize_nwsel(const uint16_t* src, int64_t ld, int64_t rows,
                                        int64_t rows_padded, int64_t K, int R, int ks,
                                        const uint16_t* ldown_packed, uint8_t* codes,
                                        uint16_t* scales, float* lora_part, const uint16_t* gamma,
                                        double eps, int64_t wgs, int64_t kp_per_wg, hipStream_t stream) {
  // waves per workgroup: as many as the k-pairs of a workgroup allow (<= 16),
  // but 8 when there are enough row tiles to fill the GPU anyway, and at
  // ranks whose 16-wave instance would not fit its registers
  if (kp_per_wg >= 16 && wgs < 256 && R <= max_rank_16_waves(NORM))
    return launch_quantize_nw<16, NORM>(src, ld, rows, rows_padded, K, R, ks, ldown_packed, codes, scales, lora_part, gamma, eps, stream);
  if (kp_per_wg >= 8)
    return launch_quantize_nw<8, NORM>(src, ld, rows, rows_padded, K, R, ks, ldown_packed, codes, scales, lora_part, gamma, eps, stream);
  if (kp_per_wg >= 4)
    return launch_quantize_nw<4, NORM>(src, ld, rows, rows_padded, K, R, ks, ldown_packed, codes, scales, lora_part, gamma, eps, stream);
  return launch_quantize_nw<2, NORM>(src, ld, rows, rows_padded, K, R, ks, ldown_packed, codes, scales, lora_part, gamma, eps, stream);
}

hipError_t launch_quantize_rows(const uint16_t* src, int64_t ld, int64_t rows,
                                int64_t rows_padded, int64_t K, int R, int ks,
                                const uint16_t* ldown_packed, uint8_t* codes,
                                uint16_t* scales, float* lora_part, const uint16_t* gamma,
                                double eps, hipStream_t stream) {
  const int64_t wgs = rows_padded / 16 * ks;
  const int64_t kp_per_wg = (K / kKPair) / ks;
  if (gamma) return launch_quantize_nwsel<true>(src, ld, rows, rows_padded, K, R, ks, ldown_packed, codes, scales,
                                                lora_part, gamma, eps, wgs, kp_per_wg, stream);
  return launch_quantize_nwsel<false>(src, ld, rows, rows_padded, K, R, ks, ldown_packed, codes, scales,
                                      lora_part, gamma, eps, wgs, kp_per_wg, stream);
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

// lora_act partials of an activation blob from per-64-group LoRA-down
// partials (the gated GEMM's quantized output writes them): thread e owns one
// float of [Mp][R]; split j = blockIdx.y sums its groups in increasing order
// starting from 0, so the result does not depend on scheduling.  Up to 32
// loads are in flight at a time (one memory round trip per 32 groups: the
// pass is bound by latency, not bandwidth), and one thread per float (not
// per four) puts more of them in flight overall.
__global__ __launch_bounds__(256) void lora_group_sum_kernel(const float* __restrict__ part, int64_t n,
                                                             int64_t KP, int ks, float* __restrict__ la) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= n) return;
  const int64_t j = blockIdx.y;
  const int64_t g0 = 2 * (j * KP / ks), g1 = 2 * ((j + 1) * KP / ks);
  constexpr int B = 32;
  float s = 0.f;
  for (int64_t b = g0; b < g1; b += B) {
    float v[B];
#pragma unroll
    for (int q = 0; q < B; ++q) v[q] = b + q < g1 ? part[(b + q) * n + e] : 0.f;
#pragma unroll
    for (int q = 0; q < B; ++q) s += v[q];
  }
  la[j * n + e] = s;
}

hipError_t launch_lora_group_sum(const float* part, int64_t Mp, int R, int64_t K, int ks, float* la,
                                 hipStream_t stream) {
  const int64_t KP = K / kKPair, n = Mp * R;
  if (R <= 0 || R % 16 != 0 || Mp % 16 != 0 || ks < 1 || ks > KP || KP < 1) return hipErrorInvalidValue;
  dim3 grid((unsigned)((n + 255) / 256), (unsigned)ks), block(256);
  lora_group_sum_kernel<<<grid, block, 0, stream>>>(part, n, KP, ks, la);
  return hipGetLastError();
}

}  // namespace w4a4
