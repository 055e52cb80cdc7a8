// Internal definitions of libw4a4: blob geometry and kernel launchers.
// The packed formats themselves are specified in include/w4a4.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace w4a4 {

constexpr int kGroup = 64;        // quantization group along K
constexpr int kKPair = 128;       // two groups: the unit of one 128-bit lane load
constexpr int kTileRows = 16;     // rows per MFMA tile
constexpr int kTileBytes = 1024;  // 16 rows x 128 k nibbles
constexpr int kMaxRank = 64;

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
__host__ __device__ inline int64_t round_up16(int64_t x) { return (x + 15) / 16 * 16; }

struct WeightGeom {
  int64_t N, K;
  int R;
  size_t off_ldown, off_wq, off_sw, off_lup, off_a, off_b, total;
};

struct ActGeom {
  int64_t M, Mp, K;
  int R, ks;
  size_t off_xq, off_sx, off_la, total;
};

// The activation pass splits K into `ks` contiguous ranges of k-pairs when M
// fits one 16-row tile (decode): each range writes its own LoRA-down partial
// sum and the GEMM adds the partials.  For M > 16 there is one range.
constexpr int kMaxLoraSplits = 8;
constexpr int kMaxTiledLoraSplits = 4;
// Number S of K-range partials of lora_act the quantizer writes (each its own
// workgroup column).  M <= 16: clamp(KP/4, 1, 8), summed by the decode GEMM.
// M > 16: enough K splits for >= 256 quantizer workgroups (a power of two,
// at most 4, each split keeping >= 8 k-pairs), 1 once there are >= 256 row
// tiles; the tiled GEMM loads every partial and sums them in its epilogue
// (each extra partial costs start-up loads there, so short K is not split).
inline int lora_splits(int64_t M, int64_t K) {
  const int64_t kp = K / kKPair;
  if (M <= 16) {
    const int64_t ks = kp / 4;
    return ks < 1 ? 1 : (ks > kMaxLoraSplits ? kMaxLoraSplits : (int)ks);
  }
  const int64_t mt = (M + 15) / 16;
  int s = 1;
  while (s < kMaxTiledLoraSplits && mt * s < 256 && 16 * s <= kp) s *= 2;
  return s;
}

inline WeightGeom weight_geom(int64_t N, int64_t K, int R) {
  WeightGeom g{};
  g.N = N;
  g.K = K;
  g.R = R;
  size_t o = 0;
  g.off_ldown = o; o = align256(o + size_t(K) * R * 2);
  g.off_wq = o;    o = align256(o + size_t(N) * K / 2);
  g.off_sw = o;    o = align256(o + size_t(N) * (K / kGroup) * 2);
  g.off_lup = o;   o = align256(o + size_t(N) * R * 2);
  g.off_a = o;     o = align256(o + size_t(N) * 4);
  g.off_b = o;     o = align256(o + size_t(N) * 4);
  g.total = o;
  return g;
}

inline ActGeom act_geom(int64_t M, int64_t K, int R) {
  ActGeom g{};
  g.M = M;
  g.Mp = round_up16(M);
  g.K = K;
  g.R = R;
  g.ks = lora_splits(M, K);
  size_t o = 0;
  g.off_xq = o; o = align256(o + size_t(g.Mp) * K / 2);
  g.off_sx = o; o = align256(o + size_t(g.Mp) * (K / kGroup) * 2);
  g.off_la = o; o = align256(o + size_t(g.ks) * g.Mp * R * 4);
  g.total = o;
  return g;
}

// ---- launchers (defined in the .hip files; return hipError_t of the launch)
// Quantize `rows` rows (padded up to a multiple of 16 with q=0, s=0) of an
// fp16 matrix into codes/scales tiles.  With R > 0 also the LoRA-down partial sums lora_part[ks][rows_padded][R]
// over `ks` k-pair ranges (ks = 1: the full sum).
// gamma != nullptr: RMS-normalize each row first (fp16 gamma [K], eps > 0).
hipError_t launch_quantize_rows(const uint16_t* src, int64_t ld, int64_t rows,
                                int64_t rows_padded, int64_t K, int R, int ks,
                                const uint16_t* ldown_packed, uint8_t* codes,
                                uint16_t* scales, float* lora_part, const uint16_t* gamma,
                                double eps, hipStream_t stream);

hipError_t launch_repack_qweight(const uint8_t* qweight, const uint16_t* w_scales,
                                 int64_t N, int64_t K, uint8_t* codes,
                                 uint16_t* scales, hipStream_t stream);

hipError_t launch_pack_lora(const uint16_t* lora_down, const uint16_t* lora_up,
                            int64_t N, int64_t K, int R, uint16_t* ldown_packed,
                            uint16_t* lup_packed, hipStream_t stream);

hipError_t launch_pack_affine(const float* col_scale, const float* bias, int64_t N,
                              float* a, float* b, hipStream_t stream);

struct GemmArgs {
  const uint8_t* xq;
  const uint16_t* sx;
  const float* la;
  const uint8_t* wq;
  const uint16_t* sw;
  const uint16_t* lup;
  const float* ca;
  const float* cb;
  uint16_t* y;
  int64_t ldy;
  int64_t M, N, K;
  int R;
  int ks;   // LoRA-down partials in la: [ks][Mp][R]
  // Gated output (MLP): column tiles come in (gate, up) pairs -- tile 2j is
  // gate columns 16j.., tile 2j+1 the up columns 16j.. -- and y gets
  // h = fp16(SiLU(gate) * up) with N/2 columns instead of the N columns.
  int glu = 0;
  // gated layer: rank blocks [0, glu_thi) can carry the gate projection's
  // L_up and [glu_tlo, R/16) the up projection's (blocks wholly inside the
  // other half are zero by the packing and are skipped)
  int glu_tlo = 0, glu_thi = 0;
  // Diagnostic group sums (psum != nullptr): the launch runs the kernel and
  // tile shape w4a4_linear would run for this shape, with the per-group
  // epilogue swapped for a store of the exact integer sums P of every 16 x 16
  // tile inside the window rows [ps_m0, ps_m0 + ps_mc) x columns [ps_n0,
  // ps_n0 + ps_nc) into psum[(row - ps_m0) * ps_nc + (col - ps_n0)][K / 64];
  // nothing else is written (y is not touched).
  int32_t* psum = nullptr;
  int64_t ps_m0 = 0, ps_mc = 0, ps_n0 = 0, ps_nc = 0;
  // Quantized gated output (qo_xq != nullptr; gated layers with M > 16, a
  // tile shape of 8 packed column tiles per workgroup): in place of h the
  // epilogue writes the next layer's activation blob pieces for h (K' = N/2
  // columns, qo_kp = K'/128 k-pairs, Mp/16 row tiles) -- codes qo_xq and
  // scales qo_sx, as the activation pass would write them -- and the
  // LoRA-down partial of every 64-column group of h, qo_part[g][Mp][qo_R]
  // (fp32), from the next layer's packed L_down qo_ldown (rank qo_R).
  uint8_t* qo_xq = nullptr;
  uint16_t* qo_sx = nullptr;
  float* qo_part = nullptr;
  const uint16_t* qo_ldown = nullptr;
  int qo_R = 0;
  int64_t qo_kp = 0;
};

enum Variant { kDecode = 1, kPrefill = 2 };

int choose_variant(int64_t M, int64_t N, int64_t K, int R);

// Y (a.psum == nullptr) or the diagnostic group sums (a.psum set) of one
// layer; the kernel, its tile shape and variant depend only on the shape (and
// the W4A4_TILED_* tuning overrides), never on which of the two is asked.
hipError_t launch_gemm(const GemmArgs& a, int variant, hipStream_t stream);

// The gated GEMM with the quantized output (a.qo_xq set, a.glu = 1, M > 16),
// on the tile shapes whose workgroups hold one 64-column group of h.
hipError_t launch_gemm_glu_quant(const GemmArgs& a, hipStream_t stream);

// lora_act of an activation blob from per-64-group LoRA-down partials
// part[g][Mp][R] (G = K/64 groups): partial j of the blob's ks K-range
// splits (k-pairs [j*KP/ks, (j+1)*KP/ks)) is the sum of its groups' partials
// taken in increasing g.
// w4a4_linear_glu_quant's body; with validate_only, its host-side argument
// checks alone (nothing is enqueued; the workspace is not checked).
int glu_quant_call(int64_t M, int64_t N, int64_t K, int32_t R, int32_t r_gate, const void* act,
                   const void* wblob, int32_t R_down, const void* down_wblob, void* act_out,
                   void* workspace, void* stream, bool validate_only);

hipError_t launch_lora_group_sum(const float* part, int64_t Mp, int R, int64_t K, int ks, float* la,
                                 hipStream_t stream);

}  // namespace w4a4
