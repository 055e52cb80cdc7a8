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
// into the weight scale.  The tiled kernel (M > 16) instead starts the MFMA
// from the bits of 3.0f, so that its result read as fp32 is 3 + P 2^-14 and
// the conversion drops out of the per-group epilogue (kOffsetBits).  LoRA-up runs on v_mfma_f32_16x16x16_f16 with the
// fp32 lora_act (the in-order sum of its partials) split into fp16 hi + lo
// parts, accumulating straight into the main accumulator; the affine and the
// fp16 rounding follow in registers.
//
// Kernels: gemm_tiled_kernel (M > 16, nine tile shapes, lean and K-split
// variants), gemm_wide_kernel (M > 16 on large grids: 256 x 128 with the
// accumulators laid out for the 4-block f16 MFMA), gemm_decode_kernel (MFMA
// decode, M <= 16) and gemm_decode_dot_kernel (v_dot8 on the packed nibbles,
// M <= 4).  Each has a diagnostic instance (PSUM) that stores the exact group
// sums in place of the scale-accumulate.
//
// Gated variant (GLU template flag): for the MLP's gate and up projections
// packed as one layer with their rows interleaved by 16-row tiles (voice-
// clone article, section 3.1: the Qwen3 MLP computes SiLU(gate) * up), a
// wave or workgroup always holds a (gate, up) tile pair, rounds both to fp16
// as the two layers would store them, and writes fp16(SiLU(g) * u) to one
// output tile (glu_bits) -- or, with QOUT, quantizes it for the next layer.
//
// Cost model measured on MI355X: one v_mfma_i32_16x16x64_i8 occupies a SIMD
// for ~16.5 cycles and a wave64 fp32 VALU op for ~4.2-4.8 cycles (16 lanes
// per clock), and inside these loops the two barely overlap, so the
// per-group epilogue (scale product, fma on four accumulators per lane, and
// the nibble expansion) costs about as much as the integer MFMAs; the tiled
// kernel trades the four conversions for half of one more 4x4x4 MFMA.  Large-M
// kernels are therefore bound by issue of MFMA + VALU, not by HBM.
#include <cstdlib>

#include "device_common.hpp"
#include "quant_common.hpp"
#include "w4a4_internal.hpp"

namespace w4a4 {

// ---------------------------------------------------------------------------
// Shared epilogue pieces
// ---------------------------------------------------------------------------

// Diagnostic epilogue (GemmArgs::psum): the exact integer sums P of one
// 16 x 16 tile and group grp -- lane (c, r) holds rows 4c + ii of column r --
// stored where the tile meets the caller's window.
__device__ __forceinline__ void store_psum_tile(const GemmArgs& g, v4i P, int64_t row0, int64_t col0,
                                                int64_t grp, int lane) {
  const int64_t col = col0 + (lane & 15) - g.ps_n0;
  if (col < 0 || col >= g.ps_nc) return;
  const int64_t G = g.K / kGroup;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const int64_t row = row0 + (lane >> 4) * 4 + ii - g.ps_m0;
    if (row >= 0 && row < g.ps_mc) g.psum[(row * g.ps_nc + col) * G + grp] = P[ii];
  }
}

// The gated activation of one output value: the gate and up projections'
// fp16 outputs (their affine applied to the fp32 accumulators and rounded, as
// each layer on its own would store them), then fp16(SiLU(g) * u).  SiLU in
// fp32 from the hardware base-2 exponential and reciprocal (about 1 ulp
// each, plus the rounding of the exponent's argument), so SiLU(g) * u before
// the fp16 rounding is within about 1e-6 relative of its exact value for
// |g| <= 20 -- some 500 times finer than that rounding (2^-11); beyond, the
// value is g * u or far below fp16's range.  e = 2^(-g log2 e) overflows to
// +inf for g below about -88, and g * rcp(inf) = g * 0 is the signed zero.
__device__ __forceinline__ uint32_t glu_bits(float ag, float g_acc, float bg, float au, float u_acc,
                                             float bu) {
  const float g = (float)(_Float16)fmaf(ag, g_acc, bg);
  const float u = (float)(_Float16)fmaf(au, u_acc, bu);
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
  const float h = g * __builtin_amdgcn_rcpf(1.0f + e) * u;
  return __builtin_bit_cast(uint16_t, (_Float16)h);
}

// Y[row, col] = fp16(a * acc + b) for the MV leading rows of each lane's four
// (rows 4c + ii), column col0 + (lane & 15).
template <int MV>
__device__ __forceinline__ void store_tile(const GemmArgs& g, v4f acc, int64_t row0,
                                           int64_t col0, float af, float bf, int lane) {
  const int c = lane >> 4, r = lane & 15;
  const int64_t col = col0 + r;
#pragma unroll
  for (int ii = 0; ii < MV; ++ii) {
    const int64_t row = row0 + c * 4 + ii;
    if (row < g.M) {
      const _Float16 v = (_Float16)fmaf(af, acc[ii], bf);
      g.y[row * g.ldy + col] = __builtin_bit_cast(uint16_t, v);
    }
  }
}

template <int MV>
__device__ __forceinline__ void store_tile_glu(const GemmArgs& g, v4f gacc, v4f uacc, int64_t row0,
                                               int64_t col0, float ag, float bg, float au, float bu,
                                               int lane) {
  const int c = lane >> 4, r = lane & 15;
  const int64_t col = col0 + r;
#pragma unroll
  for (int ii = 0; ii < MV; ++ii) {
    const int64_t row = row0 + c * 4 + ii;
    if (row < g.M) g.y[row * g.ldy + col] = (uint16_t)glu_bits(ag, gacc[ii], bg, au, uacc[ii], bu);
  }
}

// Same for a tile known to start at a row < M: one 64-bit address per lane,
// then the four rows at a stride of ldy; only a ragged last tile pays a
// per-row check.

// Lane (c, r) holds rows 4c..4c+3 of column r as fp16 bits h[0..3].  A 4x4
// transpose inside each quad of lanes (columns 4q..4q+3, q = r / 4) -- two
// DPP exchanges and a byte permute -- leaves lane (c, 4q + s) with row
// 4c + s, columns 4q..4q+3: one 8-byte store per lane instead of four 2-byte
// ones (ldy % 8 == 0 and a 16-byte aligned y keep it aligned).
__device__ __forceinline__ void store_tile4_bits(const GemmArgs& g, const uint32_t (&h)[4], int64_t row0,
                                                 int64_t col0, int lane) {
  const int c = lane >> 4, r = lane & 15, s = lane & 3;
  uint32_t d0 = h[0] | (h[1] << 16), d1 = h[2] | (h[3] << 16);
  // 2x2 blocks across lane ^ 2: lanes 0,1 take the partner's low pair as
  // their high pair, lanes 2,3 the partner's high pair as their low pair
  const uint32_t p0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d0, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
  const uint32_t p1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d1, 0x4E, 0xF, 0xF, false);
  if (s & 2) d0 = p1; else d1 = p0;
  // 2x2 transposes of 16-bit values across lane ^ 1
  const uint32_t q0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d0, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
  const uint32_t q1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)d1, 0xB1, 0xF, 0xF, false);
  const uint32_t sel = (s & 1) ? 0x03020706u : 0x05040100u;   // odd: (hi partner, hi own); even: (lo own, lo partner)
  d0 = __builtin_amdgcn_perm(q0, d0, sel);
  d1 = __builtin_amdgcn_perm(q1, d1, sel);
  const int64_t row = row0 + c * 4 + s;
  if (row < g.M)
    *reinterpret_cast<v2u*>(g.y + row * g.ldy + col0 + (r & ~3)) = v2u{d0, d1};
}

__device__ __forceinline__ void store_tile4(const GemmArgs& g, v4f acc, int64_t row0, int64_t col0,
                                            float af, float bf, int lane) {
  uint32_t h[4];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii)
    h[ii] = __builtin_bit_cast(uint16_t, (_Float16)fmaf(af, acc[ii], bf));
  store_tile4_bits(g, h, row0, col0, lane);
}

// Gated pair: output tile col0 (in y's N/2 columns) from gate and up tiles.
__device__ __forceinline__ void store_tile4_glu(const GemmArgs& g, v4f gacc, v4f uacc, int64_t row0,
                                                int64_t col0, float ag, float bg, float au, float bu,
                                                int lane) {
  uint32_t h[4];
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) h[ii] = glu_bits(ag, gacc[ii], bg, au, uacc[ii], bu);
  store_tile4_bits(g, h, row0, col0, lane);
}

typedef __attribute__((address_space(3))) void lds_void;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits [3:0] and [15:14], expcnt [6:4] and lgkmcnt [11:8] left at
// their maxima).
#define W4A4_WAIT_VMCNT(n) \
  __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | (0x7 << 4) | (0xF << 8))

// Exact fp32 scale products of one 16 x 16 tile and group h in the MFMA
// accumulator layout, S[ii] = s_x[row 4c + ii] * s_w[col lane & 15], from one
// v_mfma_f32_4x4x4_16b_f16.  sx_pair: the fp16 s_x of both groups of row
// 4(lane / 16) + (lane & 3); sw_pair: the fp16 s_w of both groups of column
// lane & 15.  The product sums over k = 0..3: A carries (s_x g0, s_x g1, 0, 0)
// and B (s_w g0, 0, 0, 0) or (0, s_w g1, 0, 0), so only group h survives and
// the product of two fp16 values is exact in fp32.
__device__ __forceinline__ v4f scale_tile(uint32_t sx_pair, uint32_t sw_pair, int h) {
  const v4h a = __builtin_bit_cast(v4h, v2u{sx_pair, 0u});
  const v4h b = __builtin_bit_cast(v4h, v2u{sw_pair & (h ? 0xFFFF0000u : 0x0000FFFFu), 0u});
  return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, v4f{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
}

// Integer group sums as fp32 without a conversion.  The i8 MFMA adds 256 P
// (|256 P| <= 2^20) to its C operand; started from the bits of 3.0f (exponent
// 1, mantissa field 2^22) instead of zero, the result read as fp32 is exactly
// 3 + P * 2^-14.  The tiled loop keeps acc' = acc * 2^-14 and, per k-pair and
// tile, first subtracts 3 (S_0 + S_1) with one more 4x4x4 f16 MFMA whose C is
// acc' (offset_tile), then adds S_h * (3 + P_h 2^-14) for both groups with one
// fma each: every group's offset cancels within the k-pair, so acc' never
// carries more than 3 S of offset (rounding ~2^-24 * 3 S per step, against
// group terms of P S 2^-14).
constexpr int kOffsetBits = 0x40400000;   // 3.0f

// acc' - 3 (S_0 + S_1) for one 16 x 16 tile, S_h = s_x[row] s_w[col] of group
// h in the accumulator layout: A carries (s_x g0, s_x g1, 2 s_x g0, 2 s_x g1)
// (doubling an fp16 s_x <= 65504 / 7 is exact) and B (-s_w g0, -s_w g1,
// -s_w g0, -s_w g1); each product is exact in fp32.
__device__ __forceinline__ v4f offset_tile(uint32_t sx_pair, uint32_t sw_pair, v4f acc) {
  typedef _Float16 v2h __attribute__((ext_vector_type(2)));
  const uint32_t nsx = sx_pair ^ 0x80008000u;
  const v2h sx = __builtin_bit_cast(v2h, nsx);
  const v4h a = __builtin_bit_cast(v4h, v2u{nsx, __builtin_bit_cast(uint32_t, sx + sx)});
  const v4h b = __builtin_bit_cast(v4h, v2u{sw_pair, sw_pair});
  return __builtin_amdgcn_mfma_f32_4x4x4f16(a, b, acc, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// Decode kernel (M <= 16): weight-streaming, HBM-bound.
// One workgroup per 16-column tile; its DW waves split K into contiguous
// ranges, worked through in batches of KB k-pairs: a wave issues the whole
// batch of loads -- weight codes and scales (non-temporal: every weight byte
// is used once) and activation codes and scales (shared by every workgroup,
// served by L2) -- and then computes k-pair by k-pair as the data lands.  Everything
// the epilogue needs (LoRA partial sums, L_up, a, b) is loaded before the
// stream, so the tail costs no extra memory round trip.
// Partial accumulators are summed in LDS in wave order (deterministic).
// MV = accumulator rows per lane that hold valid output (for M <= 4 every
// valid row sits in lanes 0..15).
// ---------------------------------------------------------------------------
// Waves per decode workgroup (DW): 4, splitting K four ways; 8 where the
// grid has few workgroups (<= 256, e.g. 4096 columns) and K is long (>= 64
// k-pairs), which otherwise leaves one wave per SIMD: K = 14336, N = 4096
// measured 7.87 -> 7.19 us at M = 1 and 14.4 -> 9.6 us at M = 16, while at
// 448 workgroups or K = 4096 eight waves were no faster or slower.
// W4A4_DECODE_WAVES=4 / 8 and W4A4_DECODE_TILES=1 / 2 (column tiles per
// workgroup, where the shape allows two) force the decode kernels' shape
// (tuning and test aids, read at every launch like W4A4_TILED_*).
static int decode_env(const char* name) {
  const char* e = std::getenv(name);
  return (e && e[0]) ? std::atoi(e) : 0;
}

static int decode_waves(int64_t workgroups, int64_t K) {
  const int ov = decode_env("W4A4_DECODE_WAVES");
  if (ov == 4 || ov == 8) return ov;
  return (workgroups <= 256 && K / kKPair >= 64) ? 8 : 4;
}

// The LoRA operands of the decode epilogue: lora_act partials j = wave,
// wave + 4 (< ks) of rows < M as unconditional loads (clamped addresses:
// lanes of rows >= M read row 0, out-of-range j re-read a valid partial;
// both are zeroed when folded), and for wave 0 the L_up fragments of the
// workgroup's NTW column tiles.
template <int RT, int NTW, int LQ, int RTL, int DW>
__device__ __forceinline__ void decode_lora_loads(const GemmArgs& g, int64_t nt0, int wave, int lane,
                                                  v4f (&lpart)[LQ][RTL], v4h (&lup)[NTW][RTL]) {
  if constexpr (RT > 0) {
    const int c = lane >> 4, r = lane & 15;
    const int rr = r < g.M ? r : 0;
#pragma unroll
    for (int q = 0; q < LQ; ++q) {
      const int j0 = wave + q * DW;
      const int j = j0 < g.ks ? j0 : g.ks - 1;
#pragma unroll
      for (int t = 0; t < RT; ++t)
        lpart[q][t] = *reinterpret_cast<const v4f*>(g.la + ((size_t)j * 16 + rr) * g.R + t * 16 + c * 4);
    }
    if (wave == 0) {
#pragma unroll
      for (int n = 0; n < NTW; ++n)
#pragma unroll
        for (int t = 0; t < RT; ++t)
          lup[n][t] = *reinterpret_cast<const v4h*>(g.lup + (((size_t)(nt0 + n) * RT + t) * 64 + lane) * 4);
    }
  }
}

// PSUM: the diagnostic instance -- the same batches, loads, expansion and
// integer MFMAs, with the per-group scale-accumulate replaced by a store of
// each group's exact sums (GemmArgs::psum) and no LoRA, reduction or store
// of Y.
template <int MV, int RT, int KB, int NTW, bool GLU, int DW, bool PSUM = false>
__global__ __launch_bounds__(64 * DW, PSUM ? 1 : 16 / DW) void gemm_decode_kernel(GemmArgs g) {
  static_assert(!PSUM || (RT == 0 && !GLU), "the diagnostic instance has no epilogue");
  constexpr int RTL = RT > 0 ? RT : 1;
  __shared__ v4f red[NTW][DW][64];
  __shared__ v4f lred[RTL][DW][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nt0 = (int64_t)blockIdx.x * NTW;   // NTW column tiles per workgroup
  const int64_t KP = g.K / kKPair;
  const int64_t per = (KP + DW - 1) / DW;
  const int64_t p0 = wave * per;
  const int64_t p1 = p0 + per < KP ? p0 + per : KP;
  const int c = lane >> 4, r = lane & 15;

  // Epilogue operands, issued before the weight stream (unconditional loads,
  // so that no wait for them precedes the weight loads); wave 0 also takes
  // the affine of its columns.  At rank 64 with two column tiles the LoRA
  // operands would not fit the registers beside a weight batch of useful
  // size: that instance loads them after the stream instead (one more memory
  // round trip in the tail).
  constexpr bool kEarly = !(RT == 4 && NTW == 2);
  constexpr int LQ = (kMaxLoraSplits + DW - 1) / DW;
  v4f lpart[LQ][RTL];
  v4h lup[NTW][RTL];
  float af[NTW], bf[NTW];
  if constexpr (kEarly && RT > 0) {
    // decode_lora_loads written out: as a call, the rank-64 one-tile
    // instance no longer fits its registers (the allocator spills)
    const int rr = r < g.M ? r : 0;
#pragma unroll
    for (int q = 0; q < LQ; ++q) {
      const int j0 = wave + q * DW;
      const int j = j0 < g.ks ? j0 : g.ks - 1;
#pragma unroll
      for (int t = 0; t < RT; ++t)
        lpart[q][t] = *reinterpret_cast<const v4f*>(g.la + ((size_t)j * 16 + rr) * g.R + t * 16 + c * 4);
    }
    if (wave == 0) {
#pragma unroll
      for (int n = 0; n < NTW; ++n)
#pragma unroll
        for (int t = 0; t < RT; ++t)
          lup[n][t] = *reinterpret_cast<const v4h*>(g.lup + (((size_t)(nt0 + n) * RT + t) * 64 + lane) * 4);
    }
  }
#pragma unroll
  for (int n = 0; n < NTW; ++n) {
    af[n] = 0.f;
    bf[n] = 0.f;
    if (!PSUM && wave == 0) {
      af[n] = g.ca[(nt0 + n) * 16 + r];
      bf[n] = g.cb[(nt0 + n) * 16 + r];
    }
  }

  // LoRA-up while the first weight batch is in flight: every wave folds its
  // partials into LDS (the wait covers only the older partial loads), a bare
  // barrier (no vmcnt drain) publishes them, and wave 0 sums them in wave
  // order and runs the LoRA-up MFMAs into its own accumulators.
  v4f a_lora[NTW];
#pragma unroll
  for (int n = 0; n < NTW; ++n) a_lora[n] = v4f{0.f, 0.f, 0.f, 0.f};
  auto lora_early = [&]() {
    if constexpr (RT > 0) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        v4f l4 = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < LQ; ++q) {
          const bool use = r < g.M && wave + q * DW < g.ks;
          l4 += use ? lpart[q][t] : v4f{0.f, 0.f, 0.f, 0.f};
        }
        lred[t][wave][lane] = l4;
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes are done
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (wave == 0) {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          v4f l4 = lred[t][0][lane];
#pragma unroll
          for (int w = 1; w < DW; ++w) l4 += lred[t][w][lane];
          v4h hi, lo;
          split_f16(l4, hi, lo);
#pragma unroll
          for (int n = 0; n < NTW; ++n) {
            // gated pair (n = 0 gate, 1 up): skip the other half's zero blocks
            if (GLU && ((n & 1) ? t < g.glu_tlo : t >= g.glu_thi)) continue;
            a_lora[n] = mfma_f16_16x16x16(hi, lup[n][t], a_lora[n]);
            a_lora[n] = mfma_f16_16x16x16(lo, lup[n][t], a_lora[n]);
          }
        }
      }
    }
  };
  bool lora_done = false;

  v4f acc[NTW];
#pragma unroll
  for (int n = 0; n < NTW; ++n) acc[n] = v4f{0.f, 0.f, 0.f, 0.f};
  // Column tile nt0 + n's weights start KP k-pair tiles after tile nt0 +
  // n - 1's.  The activation tile is lane-ordered like the MFMA A operand, so
  // lane l loads its own 16 bytes; rows >= M are zero codes with zero scales.
  // One activation tile serves the NTW weight tiles.
  const uint8_t* wq = g.wq + (size_t)nt0 * KP * kTileBytes + lane * 16;
  const uint16_t* sw = g.sw + (size_t)nt0 * KP * 32 + r * 2;
  const uint8_t* xq = g.xq + lane * 16;
  const uint8_t* sxq = reinterpret_cast<const uint8_t*>(g.sx) + (4 * c + (lane & 3)) * 4;
  for (int64_t pb = p0; pb < p1; pb += KB) {
    // All loads of a batch are plain vector loads issued in k-pair order (one
    // kind of outstanding access keeps the compiler's vmcnt waits
    // incremental, so k-pair u starts as soon as its own data has landed).
    v4u braw[KB][NTW], araw[KB];
    uint32_t swv[KB][NTW], sxw[KB];
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      const int64_t p = pb + u < p1 ? pb + u : p1 - 1;   // clamped duplicates are skipped below
#pragma unroll
      for (int n = 0; n < NTW; ++n) {
        braw[u][n] = __builtin_nontemporal_load(
            reinterpret_cast<const v4u*>(wq + ((size_t)n * KP + p) * kTileBytes));
        swv[u][n] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(sw + ((size_t)n * KP + p) * 32));
      }
      araw[u] = *reinterpret_cast<const v4u*>(xq + (size_t)p * kTileBytes);
      sxw[u] = *reinterpret_cast<const uint32_t*>(sxq + (size_t)p * 64);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (!PSUM && kEarly && !lora_done) {
      lora_early();
      lora_done = true;
    }
#pragma unroll
    for (int u = 0; u < KB; ++u) {
      if (pb + u < p1) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const v4i Ae = expand_group(araw[u][2 * h], araw[u][2 * h + 1]);
          v4f S[NTW];
          v4i P[NTW];
          if constexpr (!PSUM) {
#pragma unroll
            for (int n = 0; n < NTW; ++n) S[n] = scale_tile(sxw[u], swv[u][n], h);
          }
#pragma unroll
          for (int n = 0; n < NTW; ++n)
            P[n] = mfma_i8_16x16x64(Ae, expand_group(braw[u][n][2 * h], braw[u][n][2 * h + 1]),
                                    v4i{0, 0, 0, 0});
          if constexpr (PSUM) {
            // the int8 operands carry 16 q each: the MFMA returns 256 P
#pragma unroll
            for (int n = 0; n < NTW; ++n) store_psum_tile(g, P[n] >> 8, 0, (nt0 + n) * 16, 2 * (pb + u) + h, lane);
          } else {
#pragma unroll
            for (int n = 0; n < NTW; ++n)
#pragma unroll
              for (int ii = 0; ii < MV; ++ii) acc[n][ii] = fmaf((float)P[n][ii], S[n][ii], acc[n][ii]);
          }
        }
      }
    }
  }
  if constexpr (PSUM) return;
  if constexpr (!kEarly) decode_lora_loads<RT, NTW, LQ, RTL, DW>(g, nt0, wave, lane, lpart, lup);
  if (!lora_done) lora_early();   // a wave with no k-pairs still meets the barrier

  // cross-wave sums in LDS, added by wave 0 in wave order
#pragma unroll
  for (int n = 0; n < NTW; ++n) red[n][wave][lane] = acc[n] * (1.0f / 256.0f);   // the int8 operands carry 16 q each
  __syncthreads();
  if (wave != 0) return;
  v4f av[NTW];
#pragma unroll
  for (int n = 0; n < NTW; ++n) {
    v4f a = red[n][0][lane];
#pragma unroll
    for (int w = 1; w < DW; ++w) a += red[n][w][lane];
    av[n] = a + a_lora[n];
  }
  if constexpr (!GLU) {
#pragma unroll
    for (int n = 0; n < NTW; ++n) store_tile<MV>(g, av[n], 0, (nt0 + n) * 16, af[n], bf[n], lane);
  } else {   // the workgroup's tiles are a (gate, up) pair
    static_assert(NTW == 2, "a gated output needs both tiles of its pair");
    store_tile_glu<MV>(g, av[0], av[1], 0, (nt0 / 2) * 16, af[0], bf[0], af[1], bf[1], lane);
  }
}

// ---------------------------------------------------------------------------
// Decode kernel for M <= 4: no nibble expansion and no MFMA in the K loop.
// v_dot8_i32_i4 multiplies the 8 signed nibbles of a weight dword with the
// 8 nibbles of the matching activation dword (the packed layouts pair the
// same k in the same nibble position), so lane (column r = lane & 15, k
// segment c = lane >> 4) forms the integer sum of its 16 k per group and row
// with two instructions and adds P * s_x * s_w to a per-lane fp32 partial.
// Per batch of KB k-pairs a wave issues plain vector loads only: first the
// activation codes of its k-pairs (rows < MR, 64 B per row and k-pair,
// served by L2), then the weight codes and scales k-pair by k-pair
// (non-temporal); s_x comes through scalar loads.  The activation codes are
// parked in a per-wave LDS slice (read back as 16-lane broadcasts), so the
// compiler's vmcnt waits stay incremental and k-pair u starts as soon as its
// own weights have landed.
// The four segment partials of a column are summed once after the K loop
// (shuffles), the four waves' partials in LDS in wave order, and the result
// is laid into the MFMA accumulator layout for the LoRA-up and the store.
// Workgroup and wave decomposition are those of gemm_decode_kernel.
// ---------------------------------------------------------------------------
template <int MR, int KB, int NT>
struct DotBatch {
  static constexpr int kChunks = KB * MR * 4;          // 16 B activation chunks
  static constexpr int kXLoads = (kChunks + 63) / 64;  // per-lane loads for them
  v4u w[KB][NT];      // weight codes of the NT column tiles, 16 B per lane per k-pair
  uint32_t sw[KB][NT];  // s_w of the lane's column, both groups
  uint32_t sx[KB][MR];
  v4u x[kXLoads];     // activation chunk(s) of this lane, before they go to LDS
};

// Bases and the k-pair index are wave-uniform, per-lane offsets 32-bit (one
// column tile of codes is at most 2^24 / 2 bytes).  TAIL batches clamp the
// k-pair to the last valid one (its contribution is skipped).  Chunk q of a
// batch is (k-pair q / (4 MR), row (q / 4) % MR, segment q % 4).  The
// activation chunks are issued first and s_x comes through scalar loads, so
// the wait that parks the chunks in LDS leaves the weight loads in flight.
// Column tile n of the workgroup starts n * KP k-pair tiles after the first.
template <int MR, int KB, int NT, bool TAIL>
__device__ __forceinline__ void dot_load(DotBatch<MR, KB, NT>& d, const uint8_t* wq, const uint8_t* sw,
                                         const uint8_t* xq, const uint8_t* sx, int lane, int pb, int p1,
                                         int KP) {
  using D = DotBatch<MR, KB, NT>;
  const uint32_t lane_w = lane * 16u, lane_sw = (lane & 15) * 4u;
  // batch bases are wave-uniform (scalar registers)
  const uint8_t* wb = wq + (size_t)pb * kTileBytes;
  const uint8_t* swb = sw + (size_t)pb * 64u;
  const uint8_t* xb = xq + (size_t)pb * kTileBytes;
  const uint8_t* sxb = sx + (size_t)pb * 64u;
#pragma unroll
  for (int i = 0; i < D::kXLoads; ++i) {
    const int q = lane + 64 * i;
    const int qc = q < D::kChunks ? q : D::kChunks - 1;
    const int u = qc / (4 * MR), m = (qc >> 2) % MR, cc = qc & 3;
    const uint32_t uq = (uint32_t)(TAIL && pb + u >= p1 ? p1 - 1 - pb : u);
    // row m of k segment cc sits at lane m + 16 cc of an activation tile
    d.x[i] = *reinterpret_cast<const v4u*>(xb + (uq * kTileBytes + (uint32_t)(m + 16 * cc) * 16u));
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int u = 0; u < KB; ++u) {
    const uint32_t uq = (uint32_t)(TAIL && pb + u >= p1 ? p1 - 1 - pb : u);
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const uint8_t* wn = wb + (size_t)n * KP * kTileBytes;
      const uint8_t* swn = swb + (size_t)n * KP * 64u;
      d.w[u][n] = __builtin_nontemporal_load(reinterpret_cast<const v4u*>(wn + (lane_w + uq * kTileBytes)));
      d.sw[u][n] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(swn + (lane_sw + uq * 64u)));
    }
#pragma unroll
    for (int m = 0; m < MR; ++m) d.sx[u][m] = *reinterpret_cast<const uint32_t*>(sxb + (uq * 64u + m * 4u));
    // issue in k-pair order, so that k-pair u waits only for its own loads
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Park the batch's activation chunks in the wave's LDS slice [KB][MR][4].
template <int MR, int KB, int NT>
__device__ __forceinline__ void dot_stage(const DotBatch<MR, KB, NT>& d, v4u* xs, int lane) {
  using D = DotBatch<MR, KB, NT>;
#pragma unroll
  for (int i = 0; i < D::kXLoads; ++i) {
    const int q = lane + 64 * i;
    if (D::kChunks % 64 == 0 || q < D::kChunks) xs[q] = d.x[i];
  }
}

// PSUM (diagnostic): instead of the scale-accumulate, the lane's integer
// partial (its 16 k of the group) is summed over the group's four k
// segments (lanes r, r + 16, r + 32, r + 48) and lanes of segment 0 store
// the group's exact sums for rows < MR of column tile nt0 + n (rows MR..15
// of the tile are padding, whose codes and sums are 0).
template <int MR, int KB, int NT, bool TAIL, bool PSUM>
__device__ __forceinline__ void dot_accumulate(const DotBatch<MR, KB, NT>& d, const v4u* xs,
                                               float (&acc)[NT][MR], int c, int pb, int p1,
                                               const GemmArgs& g, int64_t nt0, int lane) {
#pragma unroll
  for (int u = 0; u < KB; ++u) {
    if (TAIL && pb + u >= p1) break;   // wave-uniform
    v4u xv[MR];
#pragma unroll
    for (int m = 0; m < MR; ++m) xv[m] = xs[(u * MR + m) * 4 + c];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        const float swf = half_bits_to_float((uint16_t)(d.sw[u][n] >> (16 * h)));
        v4i Pt = v4i{0, 0, 0, 0};   // PSUM: rows 0..3 of the tile in the MFMA accumulator layout
#pragma unroll
        for (int m = 0; m < MR; ++m) {
          int P = __builtin_amdgcn_sdot8((int)d.w[u][n][2 * h], (int)xv[m][2 * h], 0, false);
          P = __builtin_amdgcn_sdot8((int)d.w[u][n][2 * h + 1], (int)xv[m][2 * h + 1], P, false);
          if constexpr (PSUM) {
            P += __shfl_xor(P, 16);
            P += __shfl_xor(P, 32);
            Pt[m] = P;
          } else {
            // s_x * s_w is exact in fp32; fma with +0 keeps it one mixed-precision op
            const float sc = __builtin_fmaf(half_bits_to_float((uint16_t)(d.sx[u][m] >> (16 * h))), swf, 0.f);
            acc[n][m] = fmaf((float)P, sc, acc[n][m]);
          }
        }
        if constexpr (PSUM) {
          // lanes of segment 0 hold rows 0..MR-1 (as lane (c = 0, r) of the
          // accumulator layout); the other lanes store the zero rows 4c..4c+3
          if (c != 0) Pt = v4i{0, 0, 0, 0};
          store_psum_tile(g, Pt, 0, (nt0 + n) * 16, 2 * (int64_t)(pb + u) + h, lane);
        }
      }
    }
  }
}

// PSUM: the diagnostic instance (dot_accumulate's PSUM path; no LoRA,
// reduction or store of Y).
template <int MR, int RT, int KB, int NT, bool GLU, int DW, bool PSUM = false>
__global__ __launch_bounds__(64 * DW, PSUM ? 1 : 16 / DW) void gemm_decode_dot_kernel(GemmArgs g) {
  static_assert(!PSUM || (RT == 0 && !GLU), "the diagnostic instance has no epilogue");
  static_assert(MR <= 4, "the dot kernel's rows sit in lanes 0..15 of the accumulator layout");
  constexpr int RTL = RT > 0 ? RT : 1;
  __shared__ float red[NT][DW][MR][16];
  __shared__ v4f lred[RTL][DW][64];
  __shared__ v4u xs_lds[DW][DotBatch<MR, KB, NT>::kXLoads * 64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t nt0 = (int64_t)blockIdx.x * NT;   // NT column tiles per workgroup
  const int KP = (int)(g.K / kKPair);
  const int per = (KP + DW - 1) / DW;
  const int p0 = wave * per;
  const int p1 = p0 + per < KP ? p0 + per : KP;
  const int c = lane >> 4, r = lane & 15;
  const uint8_t* wq = g.wq + (size_t)nt0 * KP * kTileBytes;
  const uint8_t* sw = reinterpret_cast<const uint8_t*>(g.sw + (size_t)nt0 * KP * 32);
  const uint8_t* sx = reinterpret_cast<const uint8_t*>(g.sx);
  v4u* xs = &xs_lds[wave][0];

  // LoRA-down partials j = wave, wave + 4 (< ks) of rows < M: unconditional
  // loads (clamped addresses: lanes of rows >= M read row 0, out-of-range j
  // re-read a valid partial; both are zeroed when folded), so no branch makes
  // the compiler's vmcnt waits conservative.
  constexpr int LQ = (kMaxLoraSplits + DW - 1) / DW;
  v4f lpart[LQ][RTL];
  v4h lup[NT][RTL];
  float af[NT], bf[NT];
  if constexpr (RT > 0) {
    const int rr = r < g.M ? r : 0;
#pragma unroll
    for (int q = 0; q < LQ; ++q) {
      const int j0 = wave + q * DW;
      const int j = j0 < g.ks ? j0 : g.ks - 1;
#pragma unroll
      for (int t = 0; t < RT; ++t)
        lpart[q][t] = *reinterpret_cast<const v4f*>(g.la + ((size_t)j * 16 + rr) * g.R + t * 16 + c * 4);
    }
    if (wave == 0) {
#pragma unroll
      for (int n = 0; n < NT; ++n)
#pragma unroll
        for (int t = 0; t < RT; ++t)
          lup[n][t] = *reinterpret_cast<const v4h*>(g.lup + (((size_t)(nt0 + n) * RT + t) * 64 + lane) * 4);
    }
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    af[n] = 0.f;
    bf[n] = 0.f;
    if (!PSUM && wave == 0) {
      af[n] = g.ca[(nt0 + n) * 16 + r];
      bf[n] = g.cb[(nt0 + n) * 16 + r];
    }
  }

  // LoRA-up early, while the first weight batch is in flight: every wave
  // folds its partials into LDS (the wait covers only the older partial
  // loads), a bare barrier (no vmcnt drain) publishes them, and wave 0 sums
  // them in wave order and runs the LoRA-up MFMAs into its own accumulators.
  v4f a_lora[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) a_lora[n] = v4f{0.f, 0.f, 0.f, 0.f};
  auto lora_early = [&]() {
    if constexpr (RT > 0) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        v4f l4 = v4f{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int q = 0; q < LQ; ++q) {
          const bool use = r < g.M && wave + q * DW < g.ks;
          l4 += use ? lpart[q][t] : v4f{0.f, 0.f, 0.f, 0.f};
        }
        lred[t][wave][lane] = l4;
      }
      asm volatile("" ::: "memory");
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes are done
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      if (wave == 0) {
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          v4f l4 = lred[t][0][lane];
#pragma unroll
          for (int w = 1; w < DW; ++w) l4 += lred[t][w][lane];
          v4h hi, lo;
          split_f16(l4, hi, lo);
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            // gated pair (n = 0 gate, 1 up): skip the other half's zero blocks
            if (GLU && ((n & 1) ? t < g.glu_tlo : t >= g.glu_thi)) continue;
            a_lora[n] = mfma_f16_16x16x16(hi, lup[n][t], a_lora[n]);
            a_lora[n] = mfma_f16_16x16x16(lo, lup[n][t], a_lora[n]);
          }
        }
      }
    }
  };

  float acc[NT][MR];
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[n][m] = 0.f;
  int pb = p0;
  bool lora_done = PSUM;   // the diagnostic instance has no LoRA (and no barrier)
  for (; pb + KB <= p1; pb += KB) {
    DotBatch<MR, KB, NT> d;
    dot_load<MR, KB, NT, false>(d, wq, sw, g.xq, sx, lane, pb, p1, KP);
    if (!lora_done) {
      lora_early();
      lora_done = true;
    }
    dot_stage(d, xs, lane);
    dot_accumulate<MR, KB, NT, false, PSUM>(d, xs, acc, c, pb, p1, g, nt0, lane);
  }
  if (pb < p1) {
    DotBatch<MR, KB, NT> d;
    dot_load<MR, KB, NT, true>(d, wq, sw, g.xq, sx, lane, pb, p1, KP);
    if (!lora_done) {
      lora_early();
      lora_done = true;
    }
    dot_stage(d, xs, lane);
    dot_accumulate<MR, KB, NT, true, PSUM>(d, xs, acc, c, pb, p1, g, nt0, lane);
  }
  if constexpr (PSUM) return;
  if (!lora_done) lora_early();   // a wave with no k-pairs still meets the barrier

  // sum the four k segments of each column (lanes r, r+16, r+32, r+48)
#pragma unroll
  for (int n = 0; n < NT; ++n)
#pragma unroll
    for (int m = 0; m < MR; ++m) {
      acc[n][m] += __shfl_xor(acc[n][m], 16);
      acc[n][m] += __shfl_xor(acc[n][m], 32);
    }
  if (c == 0) {
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int m = 0; m < MR; ++m) red[n][wave][m][r] = acc[n][m];
  }
  __syncthreads();
  if (wave != 0) return;
  // accumulator layout of a 16x16 tile: lane (c, r) holds rows 4c + ii of column r
  v4f av[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    v4f a = a_lora[n];
    if (c == 0) {
#pragma unroll
      for (int m = 0; m < MR; ++m) {
        float v = red[n][0][m][r];
#pragma unroll
        for (int w = 1; w < DW; ++w) v += red[n][w][m][r];
        a[m] += v;
      }
    }
    av[n] = a;
  }
  if constexpr (!GLU) {
#pragma unroll
    for (int n = 0; n < NT; ++n) store_tile<MR>(g, av[n], 0, (nt0 + n) * 16, af[n], bf[n], lane);
  } else {   // the workgroup's tiles are a (gate, up) pair
    static_assert(NT == 2, "a gated output needs both tiles of its pair");
    store_tile_glu<MR>(g, av[0], av[1], 0, (nt0 / 2) * 16, af[0], bf[0], af[1], bf[1], lane);
  }
}

// ---------------------------------------------------------------------------
// Tiled kernel (M > 16).  Workgroup tile (WM*TM*16) x (WN*TN*16); wave (wm,
// wn) owns TM x TN tiles of 16x16.  Per k-pair, the packed 16x128 operand
// tiles (1 KB each) and the scales of the workgroup's rows and columns (64 B
// per tile) are copied HBM -> LDS with global_load_lds_dwordx4 (each lane
// moves 16 bytes; no VGPRs involved) into an NS-deep ring: the copy of
// k-pair p+NS-1 is issued right after the barrier that publishes k-pair p
// and overlaps the arithmetic on p..p+NS-2.  Every wave issues the same
// number of copies per stage, so an exact vmcnt wait publishes stage p while
// later stages stay in flight.  Fragments are read back with conflict-free LDS
// reads (lane l reads bytes [16l, 16l+16) of a tile).  Workgroups are
// renumbered so that the workgroups of one XCD cover a contiguous range of
// a grouped tile order (groups of 8 row bands, column tiles outer), which
// keeps both operands' working set of an XCD inside its L2.
// Variants (template arguments): OCC = 3 -- the lean variant for large
// launches (3 workgroups per CU, 3-deep ring, epilogue operands after the
// loop); KS = 2 -- two sets of waves split K for launches that would give a
// SIMD fewer than two waves; GLU -- the gated (SiLU(gate) * up) epilogue.
// ---------------------------------------------------------------------------
constexpr int kTileGroupRows = 8;

// Workgroup -> (row band bm, column band bn) of an nbm x nbn grid of
// workgroup tiles (32-bit: the launchers keep nbm * nbn below 2^31).
// Dispatch places workgroup b on XCD b % 8; each XCD gets a contiguous range
// of a grouped order, in which kTileGroupRows row bands advance together and
// column bands are the outer index, so a B column band is reused by the
// whole group while the group's A bands stay in that XCD's L2.  (With nbm >
// kTileGroupRows, nbn < nblk / kTileGroupRows, so group_size fits.)
__device__ __forceinline__ void map_workgroup(uint32_t nbm, uint32_t nbn, uint32_t& bm, uint32_t& bn) {
  const uint32_t nblk = nbm * nbn;
  uint32_t b = blockIdx.x;
  {
    const uint32_t per_xcd = nblk >> 3, extra = nblk & 7;
    const uint32_t xcd = b & 7, local = b >> 3;
    b = xcd * per_xcd + (xcd < extra ? xcd : extra) + local;
  }
  uint32_t first_bm = 0, in_g = b, gm = nbm;
  if (nbm > (uint32_t)kTileGroupRows) {
    const uint32_t group_size = (uint32_t)kTileGroupRows * nbn;
    const uint32_t grp = b / group_size;
    first_bm = grp * kTileGroupRows;
    in_g = b - grp * group_size;
    gm = nbm - first_bm < (uint32_t)kTileGroupRows ? nbm - first_bm : (uint32_t)kTileGroupRows;
  }
  bn = in_g / gm;
  bm = first_bm + (in_g - bn * gm);
}

// PSUM: the diagnostic instance -- the same staging, waits, expansion and
// integer MFMAs, with the per-group scale-accumulate replaced by a store of
// each group's exact sums, read back from the MFMA's 3.0f-offset result as
// (bits - kOffsetBits) / 256 (GemmArgs::psum); no LoRA and no store of Y.
// (A diagnostic launch keeps no occupancy: its instances are built for one
// workgroup per CU, so the stores of its epilogue never spill.)
//
// QOUT: the gated layer's output quantized for the next layer (GemmArgs::
// qo_xq): the workgroup's 8 packed column tiles are one 64-column group of h,
// so the activation pass's per-group work -- absmax, scale, codes, and the
// group's share of LoRA-down -- runs in the epilogue and h never goes to
// memory in fp16 ("W4A4 CUDA Kernel for Voice Clone", section 3.1: SiLU(gate)
// * up feeds the W4A4 down projection; section 3.6: its quantizer).
template <int WM, int WN, int TM, int TN, int RT, int NS, int SPL, bool GLU, int OCC, int KS,
          bool PSUM = false, bool QOUT = false>
__global__ __launch_bounds__(WM * WN * KS * 64, PSUM ? 1 : OCC) void gemm_tiled_kernel(GemmArgs g, int64_t mt_count,
                                                                        int64_t nt_count) {
  static_assert(!PSUM || (RT == 0 && SPL == 1 && !GLU), "the diagnostic instance has no epilogue");
  static_assert(!QOUT || (GLU && WN * TN == 8 && KS == 1 && !PSUM), "one 64-column group of h per workgroup");
  // KS = 2 splits K between two sets of WM x WN waves over the same output
  // tiles (each with its own stage ring, in lockstep), and the second set's
  // accumulators are added to the first's in LDS after the loop: twice the
  // waves for launches too small to give every SIMD two (K % 256 == 0).
  constexpr int NW = WM * WN;
  constexpr int BMT = WM * TM, BNT = WN * TN;            // tiles per workgroup
  constexpr int CHUNKS = BMT + BNT;                      // 1 KB operand tiles per stage
  constexpr int CPW = (CHUNKS + NW - 1) / NW;            // operand copies per wave per stage
  constexpr int SLOTS = CPW * NW;                        // >= CHUNKS; extra slots take dummy copies
  static_assert(SLOTS <= 16, "the scale copy covers at most 16 tiles");
  constexpr int OPS = CPW + 1;                           // + one scale copy
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS][KS][SLOTS + 1][kTileBytes];

  const int lane = threadIdx.x & 63;
  const int wave_all = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform
  const int kh = wave_all / NW;      // K part of this wave (KS > 1)
  const int wave = wave_all % NW;    // the wave's tile role
  const int wm = wave / WN, wn = wave % WN;
  const int c = lane >> 4;
  const v4i kOffset = v4i{kOffsetBits, kOffsetBits, kOffsetBits, kOffsetBits};

  // 32-bit tile counts (the launcher keeps them below 2^31)
  const uint32_t mtc = (uint32_t)mt_count, ntc = (uint32_t)nt_count;
  uint32_t bm, bn;
  map_workgroup((mtc + BMT - 1) / BMT, (ntc + BNT - 1) / BNT, bm, bn);
  const uint32_t mt0 = bm * BMT, nt0 = bn * BNT;
  const int64_t KPT = g.K / kKPair;   // k-pairs of the whole K
  const int64_t KP = KPT / KS;        // k-pairs of this wave's part

  // operand tile q of a stage: q < BMT -> A tile mt0+q; else B tile nt0+q-BMT.
  // Tiles past the edge re-read the last valid tile (never stored); slots
  // q >= CHUNKS (padding so that every wave issues the same number of
  // copies) re-read tile CHUNKS-1.
  auto tile_index = [&](int q) -> int64_t {
    q = q < CHUNKS ? q : CHUNKS - 1;
    if (q < BMT) {
      const uint32_t t = mt0 + q;
      return t < mtc ? t : mtc - 1;
    }
    const uint32_t t = nt0 + (q - BMT);
    return t < ntc ? t : ntc - 1;
  };
  // Copy sources at k-pair 0: the wave's operand tiles (wave-uniform
  // pointers) and, for lanes l < 4*CPW, 16 B of the scales of tile
  // wave*CPW + l/4 (64 B per tile: 16 rows x 2 groups fp16).
  const uint8_t* src[CPW];
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int q = wave * CPW + u;
    const uint8_t* base = (q < CHUNKS ? q : CHUNKS - 1) < BMT ? g.xq : g.wq;
    src[u] = base + ((size_t)tile_index(q) * KPT + (size_t)kh * KP) * kTileBytes;
  }
  const uint8_t* ssrc;
  {
    const int q = wave * CPW + ((lane >> 2) < CPW ? (lane >> 2) : CPW - 1);
    const uint16_t* sbase = (q < CHUNKS ? q : CHUNKS - 1) < BMT ? g.sx : g.sw;
    ssrc = reinterpret_cast<const uint8_t*>(sbase) + ((size_t)tile_index(q) * KPT + (size_t)kh * KP) * 64 +
           (lane & 3) * 16;
  }
  const uint32_t lane_off = lane * 16u;
  auto issue_copy = [&](int stage, int64_t p) {
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      // (a local copy: clang's host pass drops the launch stub when the
      // captured array element feeds the builtin directly)
      const uint8_t* sp = src[u];
      __builtin_amdgcn_global_load_lds(sp + (size_t)p * kTileBytes + lane_off,
                                       (lds_void*)&lds[stage][kh][wave * CPW + u][0], 16, 0, 0);
    }
    if (lane < 4 * CPW)
      __builtin_amdgcn_global_load_lds(ssrc + (size_t)p * 64,
                                       (lds_void*)&lds[stage][kh][SLOTS][wave * CPW * 64], 16, 0, 0);
  };

  v4f acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] = v4f{0.f, 0.f, 0.f, 0.f};

  // OCC = waves per SIMD the instance is built for (the launch bound's
  // minimum, which the compiler turns into a budget of 512 / OCC registers
  // per lane).  A KS = 1 workgroup puts one wave on each SIMD, so there OCC is
  // also the workgroups per CU; a K-split workgroup (KS = 2) puts two, so its
  // OCC = 2 instances hold one workgroup per CU.  OCC = 3 (the lean
  // variant, 3 waves per SIMD, where the VALU work of the per-group epilogue
  // issues ~1.5x faster than at 2) keeps the loop's registers down: the
  // epilogue operands below are loaded after the loop, lora_act partials too,
  // the stage ring is 3 deep, and the loop body runs a few tiles at a time.
  constexpr bool kLean = OCC >= 3;
  // Epilogue operands, loaded during the first k-pair (after the first
  // stages' copies, so that those reach the memory pipeline first; the exact
  // vmcnt waits of later k-pairs then only wait a little more than needed):
  // L_up fragments and the affine of its columns (lora_act fragments of the
  // wave's row tiles follow).  Tiles past the edge read the last valid tile
  // (never stored).
  constexpr int RTL = RT > 0 ? RT : 1;
  v4h lu_f[TN][RTL];
  float af[TN], bf[TN];
  // Gated layer: the wave's column tiles alternate gate (even j), up (odd
  // j), and rank blocks wholly inside the other projection's half of the
  // block-diagonal L_up are zero: not multiplied (still loaded, so that the
  // number of epilogue loads stays fixed, see kEpiLoads).
  auto block_used = [&](int j, int t) -> bool {
    if constexpr (GLU) return (j & 1) ? t >= g.glu_tlo : t < g.glu_thi;
    return true;
  };
  auto load_epilogue_operands = [&]() {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t nt = tile_index(BMT + wn * TN + j);
      af[j] = g.ca[nt * 16 + (lane & 15)];
      bf[j] = g.cb[nt * 16 + (lane & 15)];
#pragma unroll
      for (int t = 0; t < RT; ++t)
        lu_f[j][t] = *reinterpret_cast<const v4h*>(g.lup + (((size_t)nt * RT + t) * 64 + lane) * 4);
    }
  };
  // lora_act comes as g.ks <= SPL K-range partials; all of them are loaded
  // with the operands above and summed in order in the epilogue --
  // unless they would take more than 64 registers through the loop, or 64
  // beside 4 x 4 accumulator tiles: then the epilogue loads them rank block
  // by rank block (one more memory round trip per workgroup).
  // (The quantizing gated epilogue needs more registers after the loop: its
  // instances load 64 registers' worth late as well.)
  constexpr bool kLateLora = kLean || TM * RT * SPL > 16 || TM * RT >= 16 || (QOUT && TM * RT * SPL >= 16);
  v4f la_p[kLateLora ? 1 : SPL][TM][RTL];
  auto load_lora_partials = [&]() {
    if constexpr (!kLateLora && RT > 0) {
      const size_t part = (size_t)round_up16(g.M) * g.R;   // floats per partial
#pragma unroll
      for (int j = 0; j < SPL; ++j) {
        if (j == 0 || j < g.ks) {   // uniform; partial 0 always exists (and kEpiLoads counts it)
#pragma unroll
          for (int i = 0; i < TM; ++i) {
            const int64_t mt = tile_index(wm * TM + i);
#pragma unroll
            for (int t = 0; t < RT; ++t)
              la_p[j][i][t] = *reinterpret_cast<const v4f*>(
                  g.la + j * part + (size_t)(mt * 16 + (lane & 15)) * g.R + t * 16 + c * 4);
          }
        }
      }
    }
  };
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < KP) issue_copy(s, s);


  // Loads of the epilogue operands issued at k-pair 0 right after that
  // iteration's copies (not lean): younger than the copies of stages 1 ..
  // NS-1, so the waits for those stages leave them in flight as well.  Loads
  // complete in issue order, so the count is what the wait may leave
  // outstanding; the conditional lora_act partials (split index >= 1) are
  // not counted -- more younger loads than counted only make a wait longer.
  constexpr int kEpiLoads = (kLean || PSUM) ? 0 : 2 * TN + TN * RT + ((!kLateLora && RT > 0) ? TM * RT : 0);
  static_assert(2 * OPS + kEpiLoads <= 63, "vmcnt counts to 63");
  int st = 0;                      // == p % NS
  int st_next = (NS - 1) % NS;     // == (p + NS - 1) % NS
  for (int64_t p = 0; p < KP; ++p) {
    // stages issued after p and still allowed in flight
    const int64_t after = (KP - 1 - p) < (NS - 2) ? (KP - 1 - p) : (NS - 2);
    asm volatile("" ::: "memory");
    if (kEpiLoads > 0 && p >= 1 && p <= NS - 1) {
      // the epilogue loads are younger than stage p
      if (after >= 2) W4A4_WAIT_VMCNT(2 * OPS + kEpiLoads);
      else if (after == 1) W4A4_WAIT_VMCNT(OPS + kEpiLoads);
      else W4A4_WAIT_VMCNT(kEpiLoads);
    } else if constexpr (NS >= 4) {
      if (after >= 2) W4A4_WAIT_VMCNT(2 * OPS);
      else if (after == 1) W4A4_WAIT_VMCNT(OPS);
      else W4A4_WAIT_VMCNT(0);
    } else if constexpr (NS == 3) {
      if (after >= 1) W4A4_WAIT_VMCNT(OPS);
      else W4A4_WAIT_VMCNT(0);
    } else {
      W4A4_WAIT_VMCNT(0);
    }
    // Every wave's copies of stage st have landed (each wave waited for its
    // own above); after this barrier stage (p-1)%NS is no longer read by
    // anyone.  A bare s_barrier is used: __syncthreads() would add a
    // vmcnt(0) wait and drain the copies of later stages.
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (p + NS - 1 < KP) issue_copy(st_next, p + NS - 1);
    if constexpr (!kLean && !PSUM) {
      // after every copy of stages <= NS-1 (the fence keeps the compiler
      // from moving these loads ahead of the copies: kEpiLoads relies on it)
      if (p == 0) {
        asm volatile("" ::: "memory");
        load_epilogue_operands();
        load_lora_partials();
      }
    }
    // Scales of this k-pair: lane l needs s_x of row 4(l/16) + l%4 of each of
    // its row tiles and s_w of column l%16 of each of its column tiles (both
    // groups in one dword).  The 4x4x4 f16 MFMA turns them into the exact
    // fp32 tile S[m][n] = s_x[m] * s_w[n] in the accumulator layout.
    const uint8_t* sl = &lds[st][kh][SLOTS][0];
    uint32_t sxw[TM], sww[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
      sxw[i] = *reinterpret_cast<const uint32_t*>(sl + (wm * TM + i) * 64 + (4 * c + (lane & 3)) * 4);
#pragma unroll
    for (int j = 0; j < TN; ++j)
      sww[j] = *reinterpret_cast<const uint32_t*>(sl + (BMT + wn * TN + j) * 64 + (lane & 15) * 4);
    // both groups' offsets leave the accumulators first (see kOffsetBits)
    if constexpr (!PSUM) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = offset_tile(sxw[i], sww[j], acc[i][j]);
    }
    // diagnostic epilogue: the group sums of tile (i, j), group h
    auto psum_tile = [&](int i, int j, int h, v4i P) {
      const uint32_t mt = mt0 + wm * TM + i, nt = nt0 + wn * TN + j;
      if (mt < mtc && nt < ntc)
        store_psum_tile(g, (P - kOffset) >> 8, (int64_t)mt * 16, (int64_t)nt * 16, 2 * ((int64_t)kh * KP + p) + h,
                        lane);
    };
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      // A codes stay packed until their row tile comes up (lean: fewer
      // registers live)
      v2u Ar[TM];
      v4i Be[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i) Ar[i] = *reinterpret_cast<const v2u*>(&lds[st][kh][wm * TM + i][lane * 16 + h * 8]);
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const v2u r2 = *reinterpret_cast<const v2u*>(&lds[st][kh][BMT + wn * TN + j][lane * 16 + h * 8]);
        Be[j] = expand_group(r2[0], r2[1]);
      }
      if constexpr (kLean) {
        // JP column tiles at a time (scale MFMAs, integer MFMAs, then the
        // fmas): fewer registers live than a whole row tile's, fewer MFMA
        // kind switches than tile by tile.  Pairs: a whole row of 4 x 4
        // tiles no longer fits 168 registers beside the offset operand.
        constexpr int JP = (TN % 2 == 0 ? 2 : 1);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const v4i Ae = expand_group(Ar[i][0], Ar[i][1]);
#pragma unroll
          for (int j0 = 0; j0 < TN; j0 += JP) {
            v4f S[JP];
            v4i P[JP];
            if constexpr (!PSUM) {
#pragma unroll
              for (int q = 0; q < JP; ++q) S[q] = scale_tile(sxw[i], sww[j0 + q], h);
            }
#pragma unroll
            for (int q = 0; q < JP; ++q) P[q] = mfma_i8_16x16x64(Ae, Be[j0 + q], kOffset);
#pragma unroll
            for (int q = 0; q < JP; ++q) {
              if constexpr (PSUM) {
                psum_tile(i, j0 + q, h, P[q]);
              } else {
                // (cast the whole vector: clang's bit_cast of one element of an
                // ext_vector reads element 0 whatever the index)
                const v4f Pf = __builtin_bit_cast(v4f, P[q]);
#pragma unroll
                for (int ii = 0; ii < 4; ++ii) acc[i][j0 + q][ii] = fmaf(S[q][ii], Pf[ii], acc[i][j0 + q][ii]);
              }
            }
          }
        }
      } else {
        // Per row tile: its TN scale MFMAs, then its TN integer MFMAs, then
        // the conversions and FMAs -- grouping MFMAs of one kind avoids the
        // pipeline's switch penalty between the two kinds, and the FMAs of a
        // tile no longer wait right behind the MFMA that feeds them.
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          const v4i Ae = expand_group(Ar[i][0], Ar[i][1]);
          v4f S[TN];
          v4i P[TN];
          if constexpr (!PSUM) {
#pragma unroll
            for (int j = 0; j < TN; ++j) S[j] = scale_tile(sxw[i], sww[j], h);
          }
#pragma unroll
          for (int j = 0; j < TN; ++j) P[j] = mfma_i8_16x16x64(Ae, Be[j], kOffset);
#pragma unroll
          for (int j = 0; j < TN; ++j) {
            if constexpr (PSUM) {
              psum_tile(i, j, h, P[j]);
            } else {
              const v4f Pf = __builtin_bit_cast(v4f, P[j]);   // whole-vector cast (see above)
#pragma unroll
              for (int ii = 0; ii < 4; ++ii) acc[i][j][ii] = fmaf(S[j][ii], Pf[ii], acc[i][j][ii]);
            }
          }
        }
      }
    }
    st = st + 1 == NS ? 0 : st + 1;
    st_next = st_next + 1 == NS ? 0 : st_next + 1;
  }
  if constexpr (PSUM) return;

  if constexpr (KS > 1) {
    // the second K part's accumulators join the first's, in that order
    static_assert(KS == 2, "two K parts");
    static_assert(NW * TM * TN * 64 * sizeof(v4f) <= sizeof(lds), "reduction fits the stage ring");
    v4f* red = reinterpret_cast<v4f*>(&lds[0][0][0][0]);
    __syncthreads();   // every wave is done with the ring
    if (kh == 1) {
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) red[((size_t)wave * TM * TN + i * TN + j) * 64 + lane] = acc[i][j];
    }
    __syncthreads();
    if (kh == 1) return;
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
      for (int j = 0; j < TN; ++j) acc[i][j] += red[((size_t)wave * TM * TN + i * TN + j) * 64 + lane];
  }

  if constexpr (kLean) load_epilogue_operands();

  // acc holds main * 2^-14 (see kOffsetBits)
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j) acc[i][j] *= 16384.0f;

  // LoRA-up of tile (i, j): lora_act rows of row tile i (partials summed in
  // order, split into fp16 hi + lo) times the L_up fragment of column tile j,
  // rank block by rank block
  if constexpr (kLateLora) {
    const size_t part = (size_t)round_up16(g.M) * g.R;
#pragma unroll
    for (int t = 0; t < RT; ++t)
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const float* lp = g.la + (size_t)(tile_index(wm * TM + i) * 16 + (lane & 15)) * g.R + t * 16 + c * 4;
        v4f l4 = *reinterpret_cast<const v4f*>(lp);
#pragma unroll
        for (int jj = 1; jj < SPL; ++jj)
          if (jj < g.ks) l4 += *reinterpret_cast<const v4f*>(lp + jj * part);
        v4h hi, lo;
        split_f16(l4, hi, lo);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if (!block_used(j, t)) continue;
          acc[i][j] = mfma_f16_16x16x16(hi, lu_f[j][t], acc[i][j]);
          acc[i][j] = mfma_f16_16x16x16(lo, lu_f[j][t], acc[i][j]);
        }
      }
  }
  auto lora_tile = [&](int i, int j) {
    v4f a = acc[i][j];
    if constexpr (!kLateLora) {
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        if (!block_used(j, t)) continue;
        v4f l4 = la_p[0][i][t];
#pragma unroll
        for (int jj = 1; jj < SPL; ++jj)
          if (jj < g.ks) l4 += la_p[jj][i][t];
        v4h hi, lo;
        split_f16(l4, hi, lo);
        a = mfma_f16_16x16x16(hi, lu_f[j][t], a);
        a = mfma_f16_16x16x16(lo, lu_f[j][t], a);
      }
    }
    return a;
  };
  if constexpr (!GLU) {
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const int64_t nt = nt0 + wn * TN + j;
      if (nt >= nt_count) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int64_t mt = mt0 + wm * TM + i;
        if (mt < mt_count) store_tile4(g, lora_tile(i, j), mt * 16, nt * 16, af[j], bf[j], lane);
      }
    }
  } else if constexpr (!QOUT) {
    // (gate, up) tile pairs: a wave's column tiles start on an even tile, so
    // pairs never straddle waves
    static_assert(TN % 2 == 0, "a gated output needs whole tile pairs per wave");
#pragma unroll
    for (int j = 0; j < TN; j += 2) {
      const int64_t nt = nt0 + wn * TN + j;
      if (nt >= nt_count) continue;
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int64_t mt = mt0 + wm * TM + i;
        if (mt < mt_count)
          store_tile4_glu(g, lora_tile(i, j), lora_tile(i, j + 1), mt * 16, (nt / 2) * 16, af[j], bf[j],
                          af[j + 1], bf[j + 1], lane);
      }
    }
  } else {
    // h of the workgroup's rows x its 64 columns (group gq = bn of h, all
    // inside N since N/2 % 128 == 0) is staged in LDS as fp16 bits -- the
    // values w4a4_linear_glu would store; rows >= M as 0, as the activation
    // pass zeroes them.  Then each wave takes whole 16-row tiles in the
    // activation pass's lane layout (lane r + 16c: row r, columns 16c ..
    // 16c + 15): group absmax and scale, codes, and those registers times the
    // group's L_down fragments on the f16 MFMA.
    constexpr int HST = 72;   // fp16 per staged row: 64 + 8 (rows stay 16-byte aligned, banks spread)
    static_assert(BMT * 16 * HST * 2 <= sizeof(lds), "the h tile fits the stage ring");
    uint16_t* hs = reinterpret_cast<uint16_t*>(&lds[0][0][0][0]);
    __syncthreads();   // every wave is done with the stage ring
#pragma unroll
    for (int j = 0; j < TN; j += 2) {
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const v4f ga = lora_tile(i, j), ua = lora_tile(i, j + 1);
        const int lr = (wm * TM + i) * 16 + c * 4;                      // row in the workgroup tile
        const int64_t row = (int64_t)(mt0 + wm * TM + i) * 16 + c * 4;  // row of h
        const int col = ((wn * TN + j) / 2) * 16 + (lane & 15);          // column in the group
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) {
          const uint32_t hb = glu_bits(af[j], ga[ii], bf[j], af[j + 1], ua[ii], bf[j + 1]);
          hs[(lr + ii) * HST + col] = row + ii < g.M ? (uint16_t)hb : (uint16_t)0;
        }
      }
    }
    const int64_t gq = bn, pq = gq >> 1;
    const int hq = (int)(gq & 1), r = lane & 15;
    const size_t Mp = (size_t)mtc * 16;
    const int rt_down = g.qo_R / 16;
    // the group's L_down fragments (fragments s = 2 hq, 2 hq + 1 of k-pair pq
    // in the packed L_down [KP][R/16][4][64][8]), issued before the barrier
    // so that their latency passes during it and the group arithmetic
    constexpr int RTD = kMaxRank / 16;
    v8h lb[RTD][2];
#pragma unroll
    for (int t = 0; t < RTD; ++t) {
      if (t < rt_down) {   // uniform
        const _Float16* lp = reinterpret_cast<const _Float16*>(g.qo_ldown) +
                             (((size_t)pq * rt_down + t) * 4 + 2 * hq) * 64 * 8 + lane * 8;
        lb[t][0] = *reinterpret_cast<const v8h*>(lp);
        lb[t][1] = *reinterpret_cast<const v8h*>(lp + 64 * 8);
      }
    }
    // a bare barrier after this wave's LDS writes (__syncthreads would also
    // wait for the loads just issued)
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's LDS writes are done
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    for (int q = wave; q < BMT; q += NW) {
      const uint32_t mt = mt0 + q;
      if (mt >= mtc) break;   // wave-uniform; later q lie further out
      const uint16_t* hr = hs + (q * 16 + r) * HST + c * 16;
      const v8h lo = *reinterpret_cast<const v8h*>(hr);
      const v8h hi = *reinterpret_cast<const v8h*>(hr + 8);
      uint32_t d0, d1;
      const _Float16 s = quantize_group_row4(lo, hi, d0, d1);
      const size_t tix = (size_t)mt * g.qo_kp + pq;   // code tile (row tile, k-pair)
      *reinterpret_cast<v2u*>(g.qo_xq + tix * kTileBytes + lane * 16 + hq * 8) = v2u{d0, d1};
      if (c == 0)
        g.qo_sx[(tix * 16 + r) * 2 + hq] = (int64_t)mt * 16 + r < g.M ? __builtin_bit_cast(uint16_t, s) : 0;
      // the group's share of LoRA-down: lo then hi
#pragma unroll
      for (int t = 0; t < RTD; ++t) {
        if (t >= rt_down) break;   // uniform
        v4f d = mfma_f16_16x16x32(lo, lb[t][0], v4f{0.f, 0.f, 0.f, 0.f});
        d = mfma_f16_16x16x32(hi, lb[t][1], d);
        float* out = g.qo_part + ((size_t)gq * Mp + (size_t)mt * 16 + c * 4) * g.qo_R + t * 16 + r;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) out[(size_t)ii * g.qo_R] = d[ii];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Wide kernel (large launches): 2 x 2 waves of 8 x 4 tiles of 16 x 16 (a
// 256 x 128 workgroup tile), staged like the tiled kernel: a 3-deep LDS ring
// of global_load_lds copies, exact vmcnt waits, bare barriers.  The four
// column tiles of one wave row tile i share one 16-register accumulator,
// laid out as the output of the 4-block v_mfma_f32_16x16x4_4b_f16 (block b
// = column tile b, each block in the 16 x 16 accumulator layout), so per
// k-pair and row tile one such MFMA removes both groups' offsets from all
// four tiles and, per group, one more forms the four tiles' exact scale
// products s_x * s_w: 3 MFMAs where the tiled kernel issues 12 of the 4x4x4
// kind (each 4-block MFMA costs what four 4x4x4 ones do, without their
// kind-switch stalls).  Eight row tiles per wave expand each B tile once per
// 8 row tiles: 2.25 expansion VALU ops per 16 x 16 x 64 product instead of 3.
// The epilogue operands (affine, L_up, lora_act partials) are loaded after
// the K loop.  PSUM: the diagnostic instance (see gemm_tiled_kernel).
// ---------------------------------------------------------------------------
__device__ __forceinline__ v4f tile4(const v16f& a, int j) {
  return v4f{a[4 * j], a[4 * j + 1], a[4 * j + 2], a[4 * j + 3]};
}

__device__ __forceinline__ void set_tile4(v16f& a, int j, v4f t) {
  a[4 * j] = t[0];
  a[4 * j + 1] = t[1];
  a[4 * j + 2] = t[2];
  a[4 * j + 3] = t[3];
}

__device__ __forceinline__ v16f mfma_4b_f16(v4h a, v4h b, v16f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f16(a, b, c, 0, 0, 0);
}

constexpr int kWideTM = 8, kWideTN = 4;
// The gated epilogue of the wide kernel fits its 256 registers up to rank 32
// (16 per projection); above, its instances would spill and are not built.
constexpr int kWideMaxGatedRank = 32;

template <int RT, int SPL, bool GLU, bool PSUM = false>
__global__ __launch_bounds__(256, PSUM ? 1 : 2) void gemm_wide_kernel(GemmArgs g, int64_t mt_count,
                                                                      int64_t nt_count) {
  static_assert(!PSUM || (RT == 0 && SPL == 1 && !GLU), "the diagnostic instance has no epilogue");
  constexpr int WN = 2, TM = kWideTM, TN = kWideTN, NW = 4, NS = 3;
  constexpr int BMT = 2 * TM, BNT = WN * TN;               // 16 row tiles, 8 column tiles
  constexpr int CHUNKS = BMT + BNT;                        // 1 KB operand tiles per stage
  constexpr int CPW = CHUNKS / NW;                         // operand copies per wave per stage
  static_assert(CPW * NW == CHUNKS, "every wave copies the same number of tiles");
  constexpr int OPS = CPW + 1;                             // + one scale copy
  constexpr int SCALE_SLOTS = (CHUNKS * 64 + kTileBytes - 1) / kTileBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t lds[NS][CHUNKS + SCALE_SLOTS][kTileBytes];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int c = lane >> 4;
  const v4i kOffset = v4i{kOffsetBits, kOffsetBits, kOffsetBits, kOffsetBits};
  const uint32_t mtc = (uint32_t)mt_count, ntc = (uint32_t)nt_count;
  uint32_t bm, bn;
  map_workgroup((mtc + BMT - 1) / BMT, (ntc + BNT - 1) / BNT, bm, bn);
  const uint32_t mt0 = bm * BMT, nt0 = bn * BNT;
  const int64_t KP = g.K / kKPair;

  // operand tile q of a stage: q < BMT -> A tile mt0 + q, else B tile nt0 +
  // q - BMT; tiles past the edge re-read the last valid tile (never stored)
  auto tile_index = [&](int q) -> int64_t {
    if (q < BMT) {
      const uint32_t t = mt0 + q;
      return t < mtc ? t : mtc - 1;
    }
    const uint32_t t = nt0 + (q - BMT);
    return t < ntc ? t : ntc - 1;
  };
  const uint8_t* src[CPW];
#pragma unroll
  for (int u = 0; u < CPW; ++u) {
    const int q = wave * CPW + u;
    src[u] = (q < BMT ? g.xq : g.wq) + (size_t)tile_index(q) * KP * kTileBytes;
  }
  // lanes l < 4 CPW copy 16 B of the scales of tile wave * CPW + l / 4
  const uint8_t* ssrc;
  {
    const int q = wave * CPW + ((lane >> 2) < CPW ? (lane >> 2) : CPW - 1);
    ssrc = reinterpret_cast<const uint8_t*>(q < BMT ? g.sx : g.sw) + (size_t)tile_index(q) * KP * 64 +
           (lane & 3) * 16;
  }
  const uint32_t lane_off = lane * 16u;
  auto issue_copy = [&](int stage, int64_t p) {
#pragma unroll
    for (int u = 0; u < CPW; ++u) {
      const uint8_t* sp = src[u];
      __builtin_amdgcn_global_load_lds(sp + (size_t)p * kTileBytes + lane_off,
                                       (lds_void*)&lds[stage][wave * CPW + u][0], 16, 0, 0);
    }
    if (lane < 4 * CPW)
      __builtin_amdgcn_global_load_lds(ssrc + (size_t)p * 64, (lds_void*)(&lds[stage][CHUNKS][0] + wave * CPW * 64),
                                       16, 0, 0);
  };

  v16f acc[TM];
#pragma unroll
  for (int i = 0; i < TM; ++i) acc[i] = v16f{};
#pragma unroll
  for (int s = 0; s < NS - 1; ++s)
    if (s < KP) issue_copy(s, s);

  int st = 0, st_next = NS - 1;
  for (int64_t p = 0; p < KP; ++p) {
    asm volatile("" ::: "memory");
    if (p + 1 < KP) W4A4_WAIT_VMCNT(OPS);   // stage p + 1 may stay in flight
    else W4A4_WAIT_VMCNT(0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
    if (p + NS - 1 < KP) issue_copy(st_next, p + NS - 1);

    const uint8_t* sl = &lds[st][CHUNKS][0];
    // the wave's column tiles, both groups, expanded once for its 8 row tiles
    v4i Be[TN][2];
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      const v4u r = *reinterpret_cast<const v4u*>(&lds[st][BMT + wn * TN + j][lane * 16]);
      Be[j][0] = expand_group(r[0], r[1]);
      Be[j][1] = expand_group(r[2], r[3]);
    }
    // B operands of the 4-block MFMAs: block b = the wave's column tile b,
    // lane l of block b = column l & 15 (s_w of both groups in one dword)
    const uint32_t swd = *reinterpret_cast<const uint32_t*>(sl + (BMT + wn * TN + c) * 64 + (lane & 15) * 4);
    const v4h sb[2] = {__builtin_bit_cast(v4h, v2u{swd & 0x0000FFFFu, 0u}),
                       __builtin_bit_cast(v4h, v2u{swd & 0xFFFF0000u, 0u})};
    const v4h ob = __builtin_bit_cast(v4h, v2u{swd, swd});
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const v4u ra = *reinterpret_cast<const v4u*>(&lds[st][wm * TM + i][lane * 16]);
      // s_x of row lane & 15 of row tile i, both groups (every block's A)
      const uint32_t sxd = *reinterpret_cast<const uint32_t*>(sl + (wm * TM + i) * 64 + (lane & 15) * 4);
      if constexpr (!PSUM) {
        // acc' -= 3 (S_0 + S_1) on the four tiles (see kOffsetBits, offset_tile)
        typedef _Float16 v2h __attribute__((ext_vector_type(2)));
        const uint32_t nsx = sxd ^ 0x80008000u;
        const v2h nsxh = __builtin_bit_cast(v2h, nsx);
        acc[i] = mfma_4b_f16(__builtin_bit_cast(v4h, v2u{nsx, __builtin_bit_cast(uint32_t, nsxh + nsxh)}), ob,
                             acc[i]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const v4i Ae = expand_group(ra[2 * h], ra[2 * h + 1]);
        v16f S;
        if constexpr (!PSUM) S = mfma_4b_f16(__builtin_bit_cast(v4h, v2u{sxd, 0u}), sb[h], v16f{});
        v4i P[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) P[j] = mfma_i8_16x16x64(Ae, Be[j][h], kOffset);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if constexpr (PSUM) {
            const uint32_t mt = mt0 + wm * TM + i, nt = nt0 + wn * TN + j;
            if (mt < mtc && nt < ntc)
              store_psum_tile(g, (P[j] - kOffset) >> 8, (int64_t)mt * 16, (int64_t)nt * 16, 2 * p + h, lane);
          } else {
            const v4f Pf = __builtin_bit_cast(v4f, P[j]);   // whole-vector cast
#pragma unroll
            for (int ii = 0; ii < 4; ++ii) acc[i][4 * j + ii] = fmaf(S[4 * j + ii], Pf[ii], acc[i][4 * j + ii]);
          }
        }
      }
    }
    st = st + 1 == NS ? 0 : st + 1;
    st_next = st_next + 1 == NS ? 0 : st_next + 1;
  }
  if constexpr (PSUM) return;

  // acc holds main * 2^-14 (see kOffsetBits)
#pragma unroll
  for (int i = 0; i < TM; ++i) acc[i] *= 16384.0f;
  // LoRA-up, one rank block at a time (its L_up fragments of the wave's
  // column tiles, then per row tile the lora_act rows -- partials summed in
  // order, split fp16 hi + lo -- times each fragment); gated layers skip the
  // other half's zero blocks
  if constexpr (RT > 0) {
    const size_t part = (size_t)round_up16(g.M) * g.R;
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      v4h lu_f[TN];
#pragma unroll
      for (int j = 0; j < TN; ++j)
        lu_f[j] = *reinterpret_cast<const v4h*>(g.lup + (((size_t)tile_index(BMT + wn * TN + j) * RT + t) * 64 +
                                                         lane) * 4);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const float* lp = g.la + (size_t)(tile_index(wm * TM + i) * 16 + (lane & 15)) * g.R + t * 16 + c * 4;
        v4f l4 = *reinterpret_cast<const v4f*>(lp);
#pragma unroll
        for (int jj = 1; jj < SPL; ++jj)
          if (jj < g.ks) l4 += *reinterpret_cast<const v4f*>(lp + jj * part);
        v4h hi, lo;
        split_f16(l4, hi, lo);
#pragma unroll
        for (int j = 0; j < TN; ++j) {
          if (GLU && ((j & 1) ? t < g.glu_tlo : t >= g.glu_thi)) continue;
          v4f a4 = tile4(acc[i], j);
          a4 = mfma_f16_16x16x16(hi, lu_f[j], a4);
          a4 = mfma_f16_16x16x16(lo, lu_f[j], a4);
          set_tile4(acc[i], j, a4);
        }
      }
    }
  }
  // affine of the wave's column tiles
  float af[TN], bf[TN];
#pragma unroll
  for (int j = 0; j < TN; ++j) {
    const int64_t nt = tile_index(BMT + wn * TN + j);
    af[j] = g.ca[nt * 16 + (lane & 15)];
    bf[j] = g.cb[nt * 16 + (lane & 15)];
  }
  // stores row tile by row tile: a row's 4 column tiles (128 contiguous
  // bytes of Y) go out back to back, so the L2 writes whole lines
  if constexpr (!GLU) {
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const uint32_t mt = mt0 + wm * TM + i;
      if (mt >= mtc) continue;
#pragma unroll
      for (int j = 0; j < TN; ++j) {
        const uint32_t nt = nt0 + wn * TN + j;
        if (nt < ntc) store_tile4(g, tile4(acc[i], j), (int64_t)mt * 16, (int64_t)nt * 16, af[j], bf[j], lane);
      }
    }
  } else {   // (gate, up) pairs: the wave's column tiles start on an even tile
#pragma unroll
    for (int i = 0; i < TM; ++i) {
      const uint32_t mt = mt0 + wm * TM + i;
      if (mt >= mtc) continue;
#pragma unroll
      for (int j = 0; j < TN; j += 2) {
        const uint32_t nt = nt0 + wn * TN + j;
        if (nt < ntc)
          store_tile4_glu(g, tile4(acc[i], j), tile4(acc[i], j + 1), (int64_t)mt * 16, (int64_t)(nt / 2) * 16,
                          af[j], bf[j], af[j + 1], bf[j + 1], lane);
      }
    }
  }
}

template <bool GLU>
static hipError_t launch_wide(const GemmArgs& a, hipStream_t stream) {
  const int64_t mt = round_up16(a.M) / 16, nt = a.N / 16;
  const int64_t nblk = ((mt + 2 * kWideTM - 1) / (2 * kWideTM)) * ((nt + 2 * kWideTN - 1) / (2 * kWideTN));
  if (nblk >= ((int64_t)1 << 31)) return hipErrorInvalidValue;   // 32-bit tile arithmetic
  const dim3 grid((unsigned)nblk), block(256);
  if (a.psum) {
    gemm_wide_kernel<0, 1, false, true><<<grid, block, 0, stream>>>(a, mt, nt);
    return hipGetLastError();
  }
  const bool split = a.ks > 1;
  switch (a.R / 16) {
#define W4A4_WIDE_CASE(rt)                                                                              \
  case rt:                                                                                              \
    if constexpr (GLU && rt > kWideMaxGatedRank / 16) return hipErrorInvalidValue;                     \
    else if (split) gemm_wide_kernel<rt, kMaxTiledLoraSplits, GLU><<<grid, block, 0, stream>>>(a, mt, nt); \
    else gemm_wide_kernel<rt, 1, GLU><<<grid, block, 0, stream>>>(a, mt, nt);                           \
    break;
    W4A4_WIDE_CASE(0)
    W4A4_WIDE_CASE(1)
    W4A4_WIDE_CASE(2)
    W4A4_WIDE_CASE(3)
    W4A4_WIDE_CASE(4)
#undef W4A4_WIDE_CASE
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Weight k-pairs per batch of the MFMA decode kernel, by R / 16.  Within the
// 128-VGPR budget (with the LoRA-down partials held across the first batch)
// small batches measured best: the per-k-pair arithmetic here is heavy enough
// that starting it early beats keeping more bytes in flight per wave.
constexpr int mv_kb(int rt, int ntw) {
  constexpr int kTable[2][5] = {{4, 4, 2, 2, 2}, {4, 2, 2, 2, 4}};
  return kTable[ntw - 1][rt];
}

// The layer's instance, or (a.psum set) the diagnostic instance with the
// same batch size, column tiles per workgroup and waves.
template <int MV, int RT, int NTW, bool GLU, int DW>
static void launch_mv_rt(const GemmArgs& a, dim3 grid, dim3 block, hipStream_t stream) {
  constexpr int KB = mv_kb(RT, NTW);
  if (a.psum)
    gemm_decode_kernel<MV, 0, KB, NTW, false, DW, true><<<grid, block, 0, stream>>>(a);
  else
    gemm_decode_kernel<MV, RT, KB, NTW, GLU, DW><<<grid, block, 0, stream>>>(a);
}

template <int MV, int NTW, bool GLU, int DW>
static hipError_t launch_decode_mv_dw(const GemmArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)(a.N / 16 / NTW)), block(64 * DW);
  switch (a.R / 16) {
    case 0: launch_mv_rt<MV, 0, NTW, GLU, DW>(a, grid, block, stream); break;
    case 1: launch_mv_rt<MV, 1, NTW, GLU, DW>(a, grid, block, stream); break;
    case 2: launch_mv_rt<MV, 2, NTW, GLU, DW>(a, grid, block, stream); break;
    case 3: launch_mv_rt<MV, 3, NTW, GLU, DW>(a, grid, block, stream); break;
    case 4: launch_mv_rt<MV, 4, NTW, GLU, DW>(a, grid, block, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MV, int NTW, bool GLU>
static hipError_t launch_decode_mv_n(const GemmArgs& a, hipStream_t stream) {
  if (decode_waves(a.N / 16 / NTW, a.K) == 8) return launch_decode_mv_dw<MV, NTW, GLU, 8>(a, stream);
  return launch_decode_mv_dw<MV, NTW, GLU, 4>(a, stream);
}

// Two column tiles per workgroup (one activation tile serves both) when the
// column tiles pair up, there are still >= 256 workgroups and the rank leaves
// room in 128 VGPRs (R <= 48); else one.  A gated output always takes two
// (its (gate, up) pair).
template <int MV>
static hipError_t launch_decode_mv(const GemmArgs& a, hipStream_t stream) {
  const int64_t ntiles = a.N / 16;
  if (a.glu) return launch_decode_mv_n<MV, 2, true>(a, stream);
  const int ov = decode_env("W4A4_DECODE_TILES");
  const bool two = ntiles % 2 == 0 && a.R <= 48 && (ov ? ov == 2 : ntiles / 2 >= 256);
  if (two) return launch_decode_mv_n<MV, 2, false>(a, stream);
  return launch_decode_mv_n<MV, 1, false>(a, stream);
}


// Weight k-pairs per batch of the dot decode kernel ([column tiles per
// workgroup - 1][M - 1][R / 16]): as many as fit the 128-VGPR budget,
// together with the LoRA-down partials held across the first batch, without
// spills.
constexpr int dot_kb(int mr, int rt, int nt) {
  constexpr int kTable[2][4][5] = {{{8, 8, 8, 8, 4}, {8, 8, 8, 4, 4}, {8, 4, 4, 2, 4}, {8, 4, 4, 4, 2}},
                                   {{4, 4, 4, 2, 1}, {4, 4, 4, 2, 1}, {4, 2, 2, 1, 1}, {4, 2, 2, 1, 1}}};
  return kTable[nt - 1][mr - 1][rt];
}

// A wave whose k range is shorter than one batch would run only the
// bounds-checked tail batch, whose conditional loads make every wait a full
// drain; a 4-pair batch keeps such short ranges on the unchecked path.
template <int MR, int RT, int NT, bool GLU, int DW>
static void launch_dot_rt_dw(const GemmArgs& a, hipStream_t stream) {
  constexpr int KB = dot_kb(MR, RT, NT);
  constexpr int KBS = KB < 4 ? KB : 4;
  const dim3 grid((unsigned)(a.N / 16 / NT)), block(64 * DW);
  const int64_t per = (a.K / kKPair + DW - 1) / DW;
  const bool short_range = KBS < KB && per < KB;
  if (a.psum) {   // the diagnostic instance of the same batch size
    if (short_range)
      gemm_decode_dot_kernel<MR, 0, KBS, NT, false, DW, true><<<grid, block, 0, stream>>>(a);
    else
      gemm_decode_dot_kernel<MR, 0, KB, NT, false, DW, true><<<grid, block, 0, stream>>>(a);
  } else if (short_range) {
    gemm_decode_dot_kernel<MR, RT, KBS, NT, GLU, DW><<<grid, block, 0, stream>>>(a);
  } else {
    gemm_decode_dot_kernel<MR, RT, KB, NT, GLU, DW><<<grid, block, 0, stream>>>(a);
  }
}

template <int MR, int RT, int NT, bool GLU>
static void launch_dot_rt(const GemmArgs& a, hipStream_t stream) {
  if (decode_waves(a.N / 16 / NT, a.K) == 8)
    launch_dot_rt_dw<MR, RT, NT, GLU, 8>(a, stream);
  else
    launch_dot_rt_dw<MR, RT, NT, GLU, 4>(a, stream);
}

template <int MR, int NT, bool GLU>
static hipError_t launch_decode_dot_n(const GemmArgs& a, hipStream_t stream) {
  switch (a.R / 16) {
    case 0: launch_dot_rt<MR, 0, NT, GLU>(a, stream); break;
    case 1: launch_dot_rt<MR, 1, NT, GLU>(a, stream); break;
    case 2: launch_dot_rt<MR, 2, NT, GLU>(a, stream); break;
    case 3: launch_dot_rt<MR, 3, NT, GLU>(a, stream); break;
    case 4: launch_dot_rt<MR, 4, NT, GLU>(a, stream); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Two column tiles per workgroup (sharing the activation chunks, the
// LoRA-down fold and the cross-wave reduction) when they pair up and at
// least 256 workgroups remain; else one.  A gated output always takes two
// (its (gate, up) pair).
template <int MR>
static hipError_t launch_decode_dot(const GemmArgs& a, hipStream_t stream) {
  const int64_t ntiles = a.N / 16;
  if (a.glu) return launch_decode_dot_n<MR, 2, true>(a, stream);
  const int ov = decode_env("W4A4_DECODE_TILES");
  if (ntiles % 2 == 0 && (ov ? ov == 2 : ntiles / 2 >= 256)) return launch_decode_dot_n<MR, 2, false>(a, stream);
  return launch_decode_dot_n<MR, 1, false>(a, stream);
}

// M <= 4: nibble dot products (about 10 VALU per row and k-pair); larger M:
// int8 MFMA on expanded nibbles (a fixed ~50 VALU + 4 MFMA per k-pair).  At
// M = 4 the two cost about the same per k-pair; where two column tiles per
// workgroup still leave >= 256 workgroups the MFMA kernel shares one
// activation tile between them and measured 6% faster (4096 x 14336: 8.5
// against 9.05 us), elsewhere the dot kernel wins (4096 x 4096: 5.0 against
// 5.7 us).
static hipError_t launch_decode(const GemmArgs& a, hipStream_t stream) {
  const int64_t ntiles = a.N / 16;
  switch (a.M) {
    case 1: return launch_decode_dot<1>(a, stream);
    case 2: return launch_decode_dot<2>(a, stream);
    case 3: return launch_decode_dot<3>(a, stream);
    case 4:
      if (ntiles % 2 == 0 && ntiles / 2 >= 256) return launch_decode_mv<4>(a, stream);
      return launch_decode_dot<4>(a, stream);
    default: return launch_decode_mv<4>(a, stream);
  }
}

// LDS stage ring depth: 4, or 3 for the lean (3 workgroups per CU) variant,
// whose 128 x 128 tile shape then fits three 51 KB rings in a CU's 160 KB.
template <int WM, int WN, int TM, int TN, int SPL, bool GLU, int OCC, int KS>
static hipError_t launch_tiled_spl(const GemmArgs& a, int64_t mt, int64_t nt, dim3 grid, dim3 block,
                                   hipStream_t stream) {
  constexpr int NS = OCC >= 3 ? 3 : 4;
  if (a.psum) {   // the diagnostic instance of this tile shape and variant
    gemm_tiled_kernel<WM, WN, TM, TN, 0, NS, 1, false, OCC, KS, true><<<grid, block, 0, stream>>>(a, mt, nt);
    return hipGetLastError();
  }
  if (a.qo_xq) {   // the gated output quantized for the next layer
    if constexpr (GLU && WN * TN == 8 && KS == 1) {
      switch (a.R / 16) {
        case 0: gemm_tiled_kernel<WM, WN, TM, TN, 0, NS, SPL, true, OCC, 1, false, true><<<grid, block, 0, stream>>>(a, mt, nt); break;
        case 1: gemm_tiled_kernel<WM, WN, TM, TN, 1, NS, SPL, true, OCC, 1, false, true><<<grid, block, 0, stream>>>(a, mt, nt); break;
        case 2: gemm_tiled_kernel<WM, WN, TM, TN, 2, NS, SPL, true, OCC, 1, false, true><<<grid, block, 0, stream>>>(a, mt, nt); break;
        case 3: gemm_tiled_kernel<WM, WN, TM, TN, 3, NS, SPL, true, OCC, 1, false, true><<<grid, block, 0, stream>>>(a, mt, nt); break;
        case 4: gemm_tiled_kernel<WM, WN, TM, TN, 4, NS, SPL, true, OCC, 1, false, true><<<grid, block, 0, stream>>>(a, mt, nt); break;
        default: return hipErrorInvalidValue;
      }
      return hipGetLastError();
    }
    return hipErrorInvalidValue;   // this tile shape does not hold whole groups of h
  }
  switch (a.R / 16) {
    case 0: gemm_tiled_kernel<WM, WN, TM, TN, 0, NS, SPL, GLU, OCC, KS><<<grid, block, 0, stream>>>(a, mt, nt); break;
    case 1: gemm_tiled_kernel<WM, WN, TM, TN, 1, NS, SPL, GLU, OCC, KS><<<grid, block, 0, stream>>>(a, mt, nt); break;
    case 2: gemm_tiled_kernel<WM, WN, TM, TN, 2, NS, SPL, GLU, OCC, KS><<<grid, block, 0, stream>>>(a, mt, nt); break;
    case 3: gemm_tiled_kernel<WM, WN, TM, TN, 3, NS, SPL, GLU, OCC, KS><<<grid, block, 0, stream>>>(a, mt, nt); break;
    case 4: gemm_tiled_kernel<WM, WN, TM, TN, 4, NS, SPL, GLU, OCC, KS><<<grid, block, 0, stream>>>(a, mt, nt); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// SPL = number of lora_act partials a wave sums: 1, or up to
// kMaxTiledLoraSplits.
template <int WM, int WN, int TM, int TN, bool GLU, int OCC, int KS = 1>
static hipError_t launch_tiled_cfg(const GemmArgs& a, hipStream_t stream) {
  const int64_t mt = round_up16(a.M) / 16, nt = a.N / 16;
  const int64_t nblk = ((mt + WM * TM - 1) / (WM * TM)) * ((nt + WN * TN - 1) / (WN * TN));
  if (nblk >= ((int64_t)1 << 31)) return hipErrorInvalidValue;   // the kernel's tile math is 32-bit
  if (KS > 1 && (a.K / kKPair) % KS != 0) return hipErrorInvalidValue;
  dim3 grid((unsigned)nblk), block(64 * WM * WN * KS);
  if (a.ks == 1) return launch_tiled_spl<WM, WN, TM, TN, 1, GLU, OCC, KS>(a, mt, nt, grid, block, stream);
  return launch_tiled_spl<WM, WN, TM, TN, kMaxTiledLoraSplits, GLU, OCC, KS>(a, mt, nt, grid, block, stream);
}

// Tile shapes for M > 16: a workgroup of WM x WN waves, each wave TM x TN
// tiles of 16 x 16.  occ = workgroups one CU holds at once (from the VGPR and
// LDS use of the instance).
struct TiledCfg {
  int wm, wn, tm, tn, occ;
};
constexpr TiledCfg kTiledCfgs[] = {
    {2, 2, 4, 4, 2},   // 128 x 128
    {2, 2, 2, 4, 3},   //  64 x 128
    {2, 2, 4, 2, 3},   // 128 x  64
    {2, 2, 2, 2, 4},   //  64 x  64
    {2, 2, 1, 2, 4},   //  32 x  64
    {4, 1, 1, 3, 4},   //  64 x  48
    {1, 4, 3, 1, 4},   //  48 x  64
    {4, 1, 1, 2, 4},   //  64 x  32
    {4, 1, 1, 4, 4},   //  64 x  64, one row tile per wave
    {2, 2, 8, 4, 2},   // 256 x 128, the wide kernel (gemm_wide_kernel)
};
constexpr int kWideCfg = 9;
constexpr int kNumTiledCfgs = (int)(sizeof(kTiledCfgs) / sizeof(kTiledCfgs[0]));

// W4A4_TILED_CFG=<index into kTiledCfgs> forces a tile shape (tuning and
// test aid; read at every launch so that one process can cover every shape).
static int tiled_override() {
  const char* e = std::getenv("W4A4_TILED_CFG");
  if (!e || !e[0]) return -1;
  const int i = std::atoi(e);
  return (i >= 0 && i < kNumTiledCfgs) ? i : -1;
}

// Makespan model of a launch on 256 CUs x 4 SIMDs.  Workgroups spread evenly
// over the CUs, so the busiest SIMD runs ceil(ceil(nblk / 256) * waves / 4)
// waves one after another or interleaved (the kernel is bound by instruction
// issue); a wave's cost is its tiles times the per-tile cost of its shape
// (integer MFMA, scale MFMA and the per-group epilogue are fixed per tile;
// the nibble expansion is shared by a wave's row and column tiles), plus a
// fixed prologue / epilogue share.  Units: SIMD cycles per k-pair.  The
// constants were fitted when the epilogue still converted each group sum
// (4 converts + 4 fmas); with the conversion-free loop a sweep of 38 shapes
// x 9 forced tile shapes x both variants put the picks within 0.7% of the
// per-shape best in total, so they stay.
static double tiled_cost(const TiledCfg& c, int64_t mt, int64_t nt, int64_t kp) {
  const int64_t bmt = c.wm * c.tm, bnt = c.wn * c.tn;
  const int64_t nblk = ((mt + bmt - 1) / bmt) * ((nt + bnt - 1) / bnt);
  const int64_t per_cu = (nblk + 255) / 256;
  const int64_t waves_per_simd = (per_cu * c.wm * c.wn + 3) / 4;
  const double tiles = (double)(c.tm * c.tn);
  const double per_tile = 2.0 * (16.5 + 8.6 + 8 * 2.8 + 5 * 2.8) +
                          2.0 * 6 * 2.8 * (double)(c.tm + c.tn) / tiles;
  const double fixed = 900.0 + 150.0 * tiles;   // prologue, LoRA-up and store per wave
  return (double)waves_per_simd * (tiles * per_tile * (double)kp + fixed);
}

// Per-tile cost of the wide kernel relative to the model's figure for its
// shape: measured 192.6 against 209.3 us for the 128 x 128 lean kernel at
// M = 8192, K = N = 4096, where the model puts the two within 3% of each
// other.
constexpr double kWideCostScale = 0.95;

static int pick_tiled(int64_t M, int64_t N, int64_t K, int R, int ks, bool glu) {
  // gated output: a wave's column tiles must hold whole (gate, up) pairs
  (void)ks;
  auto ok = [&](int i) {
    return (!glu || kTiledCfgs[i].tn % 2 == 0) && !(glu && i == kWideCfg && R > kWideMaxGatedRank);
  };
  const int ov = tiled_override();
  if (ov >= 0 && ok(ov)) return ov;
  const int64_t mt = round_up16(M) / 16, nt = N / 16, kp = K / kKPair;
  int best = -1;
  double best_c = 0;
  for (int i = 0; i < kNumTiledCfgs; ++i) {
    if (!ok(i)) continue;
    double c = tiled_cost(kTiledCfgs[i], mt, nt, kp);
    if (i == kWideCfg) {
      // the wide kernel keeps two workgroups per CU; with fewer a SIMD runs
      // one wave at a time, which this loop cannot keep busy
      const TiledCfg& w = kTiledCfgs[i];
      const int64_t nblk = ((mt + w.wm * w.tm - 1) / (w.wm * w.tm)) * ((nt + w.wn * w.tn - 1) / (w.wn * w.tn));
      if (nblk < 512) continue;
      c *= kWideCostScale;
    }
    if (best < 0 || c < best_c) {
      best_c = c;
      best = i;
    }
  }
  return best;
}

// The lean variant (3 workgroups per CU, epilogue operands loaded after the
// K loop) wins once every SIMD has enough tile-k-pairs of work to amortize
// the extra memory round trip at its end: over a grid of prefill shapes
// (M 300..8192, N x K from 1024 x 3072 to 14336 x 4096) the rule "at least
// 150 16x16x128 tile-k-pairs per SIMD" came within 0.2% of the per-shape
// better of the two (M=8192 K=N=4096: 241 -> 224 us; M=700 N=14336 K=4096:
// 106 -> 86 us; the M=700 MLP shapes keep the 4-stage variant).  Built for
// the shapes that carry large launches.
// W4A4_TILED_LEAN=0 / 1 forces the choice where the shape has both (tuning
// and test aid, read at every launch like W4A4_TILED_CFG).
constexpr bool kLeanCfg[kNumTiledCfgs] = {true, true, true, true, false, true, false, false, true, false};
static bool tiled_lean(int cfg, int64_t M, int64_t N, int64_t K) {
  if (cfg < 0 || cfg >= kNumTiledCfgs || !kLeanCfg[cfg]) return false;
  const char* e = std::getenv("W4A4_TILED_LEAN");
  if (e && (e[0] == '0' || e[0] == '1')) return e[0] == '1';
  const double tkp = (double)(round_up16(M) / 16) * (double)(N / 16) * (double)(K / kKPair);
  return tkp >= 150.0 * 1024;
}

// Split K inside the workgroup (KS = 2) for launches that would leave a
// SIMD fewer than two waves, on the small tile shapes such launches pick,
// when K has >= 16 k-pairs in an even count.  W4A4_TILED_KSPLIT=0 / 1
// forces the choice where both exist (tuning and test aid).
constexpr bool kKSplitCfg[kNumTiledCfgs] = {false, false, false, true, true, true, false, true, true, false};
static bool tiled_ksplit(int cfg, int64_t M, int64_t N, int64_t K) {
  if (cfg < 0 || cfg >= kNumTiledCfgs || !kKSplitCfg[cfg]) return false;
  const int64_t kp = K / kKPair;
  if (kp % 2 != 0) return false;
  const char* e = std::getenv("W4A4_TILED_KSPLIT");
  if (e && (e[0] == '0' || e[0] == '1')) return e[0] == '1';
  const TiledCfg& c = kTiledCfgs[cfg];
  const int64_t bmt = c.wm * c.tm, bnt = c.wn * c.tn;
  const int64_t nblk = ((round_up16(M) / 16 + bmt - 1) / bmt) * ((N / 16 + bnt - 1) / bnt);
  return kp >= 16 && nblk * c.wm * c.wn < 2048;
}

template <bool GLU>
static hipError_t launch_tiled_pick(const GemmArgs& a, int cfg, bool lean, hipStream_t stream) {
  if (cfg == kWideCfg) return launch_wide<GLU>(a, stream);
  if constexpr (!GLU) {
    if (!lean && tiled_ksplit(cfg, a.M, a.N, a.K)) {
      switch (cfg) {
        case 3: return launch_tiled_cfg<2, 2, 2, 2, false, 2, 2>(a, stream);
        case 4: return launch_tiled_cfg<2, 2, 1, 2, false, 2, 2>(a, stream);
        case 5: return launch_tiled_cfg<4, 1, 1, 3, false, 2, 2>(a, stream);
        case 7: return launch_tiled_cfg<4, 1, 1, 2, false, 2, 2>(a, stream);
        case 8: return launch_tiled_cfg<4, 1, 1, 4, false, 2, 2>(a, stream);
        default: break;
      }
    }
  }
  if (lean) {
    switch (cfg) {
      case 0: return launch_tiled_cfg<2, 2, 4, 4, GLU, 3>(a, stream);
      case 1: return launch_tiled_cfg<2, 2, 2, 4, GLU, 3>(a, stream);
      case 2: return launch_tiled_cfg<2, 2, 4, 2, GLU, 3>(a, stream);
      case 3: return launch_tiled_cfg<2, 2, 2, 2, GLU, 3>(a, stream);
      case 5:
        if constexpr (!GLU) return launch_tiled_cfg<4, 1, 1, 3, GLU, 3>(a, stream);
        break;
      case 8: return launch_tiled_cfg<4, 1, 1, 4, GLU, 3>(a, stream);
      default: break;
    }
    return hipErrorInvalidValue;
  }
  switch (cfg) {
    case 0: return launch_tiled_cfg<2, 2, 4, 4, GLU, 2>(a, stream);
    case 1: return launch_tiled_cfg<2, 2, 2, 4, GLU, 2>(a, stream);
    case 2: return launch_tiled_cfg<2, 2, 4, 2, GLU, 2>(a, stream);
    case 3: return launch_tiled_cfg<2, 2, 2, 2, GLU, 2>(a, stream);
    case 4: return launch_tiled_cfg<2, 2, 1, 2, GLU, 2>(a, stream);
    case 5:
      if constexpr (!GLU) return launch_tiled_cfg<4, 1, 1, 3, GLU, 2>(a, stream);
      break;
    case 6:
      if constexpr (!GLU) return launch_tiled_cfg<1, 4, 3, 1, GLU, 2>(a, stream);
      break;
    case 7: return launch_tiled_cfg<4, 1, 1, 2, GLU, 2>(a, stream);
    case 8: return launch_tiled_cfg<4, 1, 1, 4, GLU, 2>(a, stream);
    default: break;
  }
  return hipErrorInvalidValue;   // no tile shape fits, or one that cannot pair (gate, up) tiles
}

// The quantized gated output needs workgroups of 8 packed column tiles (one
// 64-column group of h): the 128 x 128 and 64 x 128 shapes, chosen by the
// same cost model (W4A4_TILED_CFG forces one of the two).  The lean variant
// is also taken once the grid exceeds two workgroups per CU: its epilogue
// then costs less than a second round of workgroups (measured over the MLP
// shapes at M = 64 .. 8192: 24.0 against 26.6 us at M = 700, 15.5 against
// 13.9 us at M = 64, where the grid is 48 workgroups).
constexpr int kQuantOutCfgs[] = {0, 1};

hipError_t launch_gemm_glu_quant(const GemmArgs& a, hipStream_t stream) {
  if (!a.glu || !a.qo_xq || a.M <= 16 || a.ks < 1 || a.ks > kMaxTiledLoraSplits || (a.N / 2) % kKPair != 0)
    return hipErrorInvalidValue;
  const int64_t mt = round_up16(a.M) / 16, nt = a.N / 16, kp = a.K / kKPair;
  int cfg = -1;
  const int ov = tiled_override();
  for (int i : kQuantOutCfgs)
    if (i == ov) cfg = ov;
  if (cfg < 0) {
    double best_c = 0;
    for (int i : kQuantOutCfgs) {
      const double c = tiled_cost(kTiledCfgs[i], mt, nt, kp);
      if (cfg < 0 || c < best_c) {
        best_c = c;
        cfg = i;
      }
    }
  }
  const TiledCfg& c = kTiledCfgs[cfg];
  const int64_t nblk = ((mt + c.wm * c.tm - 1) / (c.wm * c.tm)) * ((nt + c.wn * c.tn - 1) / (c.wn * c.tn));
  const char* e = std::getenv("W4A4_TILED_LEAN");
  const bool forced = e && (e[0] == '0' || e[0] == '1');
  const bool lean = tiled_lean(cfg, a.M, a.N, a.K) || (!forced && nblk > 2 * 256);
  return launch_tiled_pick<true>(a, cfg, lean, stream);
}

int choose_variant(int64_t M, int64_t N, int64_t K, int R) {
  (void)N; (void)K; (void)R;
  return M <= 16 ? kDecode : kPrefill;
}

hipError_t launch_gemm(const GemmArgs& a, int variant, hipStream_t stream) {
  switch (variant) {
    case kDecode:
      return launch_decode(a, stream);
    case kPrefill:
      if (a.ks < 1 || a.ks > kMaxTiledLoraSplits) return hipErrorInvalidValue;   // lora_splits() for M > 16
      {
        const int cfg = pick_tiled(a.M, a.N, a.K, a.R, a.ks, a.glu != 0);
        bool lean = tiled_lean(cfg, a.M, a.N, a.K);
        if (a.glu && !lean && kLeanCfg[cfg]) {
          // a gated grid beyond one round of resident workgroups takes the
          // lean variant (M=700, 6144 packed columns, K=1024: 1056 workgroups
          // of 64 x 64 for 1024 slots, 18.7 -> 17.3 us; its extra epilogue
          // round trip costs less than the second round)
          const TiledCfg& c = kTiledCfgs[cfg];
          const int64_t nblk = ((round_up16(a.M) / 16 + c.wm * c.tm - 1) / (c.wm * c.tm)) *
                               ((a.N / 16 + c.wn * c.tn - 1) / (c.wn * c.tn));
          const char* e = std::getenv("W4A4_TILED_LEAN");
          if (!(e && (e[0] == '0' || e[0] == '1')) && nblk > (int64_t)c.occ * 256) lean = true;
        }
        return a.glu ? launch_tiled_pick<true>(a, cfg, lean, stream) : launch_tiled_pick<false>(a, cfg, lean, stream);
      }
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace w4a4
