// C ABI of libw4a4 (declared in include/w4a4.h): argument validation on the
// host, blob geometry, kernel selection and launches on the caller's stream.
// Validation runs before any HIP call, so every error path is testable
// without a GPU, and nothing is enqueued when a call fails.
#include "w4a4.h"

#include <cstdio>
#include <cstdlib>

#include "w4a4_internal.hpp"

using namespace w4a4;

namespace {

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int check_nkr(int64_t N, int64_t K, int32_t R) {
  if (K < kKPair || K % kKPair != 0) return W4A4_ERR_SHAPE;
  if (N < 16 || N % 16 != 0) return W4A4_ERR_SHAPE;
  if (R < 0 || R > kMaxRank || R % 16 != 0) return W4A4_ERR_SHAPE;
  // 32-bit grid dimensions and code tile counts
  if (N / 16 > (int64_t)1 << 30 || K > (int64_t)1 << 24) return W4A4_ERR_SHAPE;
  return W4A4_OK;
}

int check_m(int64_t M) {
  if (M < 0 || M > ((int64_t)1 << 30)) return W4A4_ERR_SHAPE;
  return W4A4_OK;
}

bool log_enabled() {
  static const bool on = [] {
    const char* v = std::getenv("W4A4_LOG");
    return v && v[0] && v[0] != '0';
  }();
  return on;
}

int hip_status(hipError_t e) {
  if (e == hipSuccess) return W4A4_OK;
  if (log_enabled()) std::fprintf(stderr, "w4a4: HIP error %d (%s)\n", (int)e, hipGetErrorName(e));
  return W4A4_ERR_HIP;
}

const char* variant_name(int v) {
  switch (v) {
    case kDecode: return "decode";
    case kPrefill: return "prefill";
    default: return "?";
  }
}

}  // namespace

extern "C" {

const char* w4a4_status_string(int status) {
  switch (status) {
    case W4A4_OK: return "W4A4_OK";
    case W4A4_ERR_NULL: return "W4A4_ERR_NULL: a required pointer is NULL";
    case W4A4_ERR_SHAPE: return "W4A4_ERR_SHAPE: unsupported shape";
    case W4A4_ERR_ALIGN: return "W4A4_ERR_ALIGN: misaligned pointer or leading dimension";
    case W4A4_ERR_ARG: return "W4A4_ERR_ARG: inconsistent arguments";
    case W4A4_ERR_HIP: return "W4A4_ERR_HIP: HIP runtime error";
    default: return "W4A4: unknown status";
  }
}

int w4a4_weight_layout(int64_t N, int64_t K, int32_t R, size_t* total_bytes, size_t* offsets) {
  if (!total_bytes) return W4A4_ERR_NULL;
  int st = check_nkr(N, K, R);
  if (st) return st;
  WeightGeom g = weight_geom(N, K, R);
  *total_bytes = g.total;
  if (offsets) {
    offsets[0] = g.off_ldown;
    offsets[1] = g.off_wq;
    offsets[2] = g.off_sw;
    offsets[3] = g.off_lup;
    offsets[4] = g.off_a;
    offsets[5] = g.off_b;
  }
  return W4A4_OK;
}

int w4a4_act_layout(int64_t M, int64_t K, int32_t R, size_t* total_bytes, size_t* offsets,
                    int32_t* lora_splits) {
  if (!total_bytes) return W4A4_ERR_NULL;
  int st = check_nkr(16, K, R);
  if (st) return st;
  if ((st = check_m(M))) return st;
  ActGeom g = act_geom(M, K, R);
  *total_bytes = g.total;
  if (offsets) {
    offsets[0] = g.off_xq;
    offsets[1] = g.off_sx;
    offsets[2] = g.off_la;
  }
  if (lora_splits) *lora_splits = g.ks;
  return W4A4_OK;
}

int w4a4_pack_weights(int64_t N, int64_t K, int32_t R, const uint16_t* w_fp16,
                      const uint8_t* qweight, const uint16_t* w_scales,
                      const uint16_t* lora_down, const uint16_t* lora_up,
                      const float* col_scale, const float* bias, void* wblob,
                      void* stream) {
  int st = check_nkr(N, K, R);
  if (st) return st;
  if (!wblob) return W4A4_ERR_NULL;
  const bool have_w = w_fp16 != nullptr;
  const bool have_q = qweight != nullptr || w_scales != nullptr;
  if (have_w == have_q) return W4A4_ERR_ARG;
  if (have_q && (!qweight || !w_scales)) return W4A4_ERR_NULL;
  if (R > 0 && (!lora_down || !lora_up)) return W4A4_ERR_NULL;
  if (!aligned(wblob, 256)) return W4A4_ERR_ALIGN;
  if (have_w && !aligned(w_fp16, 16)) return W4A4_ERR_ALIGN;
  if (have_q && !aligned(w_scales, 2)) return W4A4_ERR_ALIGN;
  if (R > 0 && (!aligned(lora_down, 2) || !aligned(lora_up, 2))) return W4A4_ERR_ALIGN;
  if ((col_scale && !aligned(col_scale, 4)) || (bias && !aligned(bias, 4))) return W4A4_ERR_ALIGN;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  WeightGeom g = weight_geom(N, K, R);
  uint8_t* base = static_cast<uint8_t*>(wblob);
  uint8_t* wq = base + g.off_wq;
  uint16_t* sw = reinterpret_cast<uint16_t*>(base + g.off_sw);
  hipError_t e;
  if (have_w)
    e = launch_quantize_rows(w_fp16, K, N, N, K, 0, 1, nullptr, wq, sw, nullptr, nullptr, 0.0, s);
  else
    e = launch_repack_qweight(qweight, w_scales, N, K, wq, sw, s);
  if (e != hipSuccess) return hip_status(e);
  e = launch_pack_lora(lora_down, lora_up, N, K, R,
                       reinterpret_cast<uint16_t*>(base + g.off_ldown),
                       reinterpret_cast<uint16_t*>(base + g.off_lup), s);
  if (e != hipSuccess) return hip_status(e);
  e = launch_pack_affine(col_scale, bias, N, reinterpret_cast<float*>(base + g.off_a),
                         reinterpret_cast<float*>(base + g.off_b), s);
  return hip_status(e);
}

static int quantize_act_impl(int64_t M, int64_t K, int32_t R, const uint16_t* x, int64_t ldx,
                             const uint16_t* gamma, double eps, const void* wblob, void* act,
                             void* stream) {
  int st = check_nkr(16, K, R);
  if (st) return st;
  if ((st = check_m(M))) return st;
  if (M == 0) return W4A4_OK;
  if (!x || !act || (R > 0 && !wblob)) return W4A4_ERR_NULL;
  if (ldx < K) return W4A4_ERR_SHAPE;
  if (ldx % 8 != 0 || !aligned(x, 16) || !aligned(act, 256) || (wblob && !aligned(wblob, 256)) ||
      (gamma && !aligned(gamma, 16)))
    return W4A4_ERR_ALIGN;
  ActGeom g = act_geom(M, K, R);
  uint8_t* base = static_cast<uint8_t*>(act);
  const uint16_t* ldown = R > 0 ? reinterpret_cast<const uint16_t*>(
                                      static_cast<const uint8_t*>(wblob) + weight_geom(16, K, R).off_ldown)
                                : nullptr;
  hipError_t e = launch_quantize_rows(x, ldx, M, g.Mp, K, R, g.ks, ldown, base + g.off_xq,
                                      reinterpret_cast<uint16_t*>(base + g.off_sx),
                                      reinterpret_cast<float*>(base + g.off_la), gamma, eps,
                                      reinterpret_cast<hipStream_t>(stream));
  return hip_status(e);
}

int w4a4_quantize_act(int64_t M, int64_t K, int32_t R, const uint16_t* x, int64_t ldx,
                      const void* wblob, void* act, void* stream) {
  return quantize_act_impl(M, K, R, x, ldx, nullptr, 0.0, wblob, act, stream);
}

int w4a4_quantize_act_rmsnorm(int64_t M, int64_t K, int32_t R, const uint16_t* x, int64_t ldx,
                              const uint16_t* gamma, double eps, const void* wblob, void* act,
                              void* stream) {
  if (!gamma) return W4A4_ERR_NULL;
  if (!(eps > 0.0) || !(eps < 1e300)) return W4A4_ERR_ARG;   // also rejects NaN and inf
  return quantize_act_impl(M, K, R, x, ldx, gamma, eps, wblob, act, stream);
}

static int make_gemm_args(int64_t M, int64_t N, int64_t K, int32_t R, const void* act,
                          const void* wblob, uint16_t* y, int64_t ldy, GemmArgs* a,
                          int64_t ycols = -1) {
  if (ycols < 0) ycols = N;
  int st = check_nkr(N, K, R);
  if (st) return st;
  if ((st = check_m(M))) return st;
  if (!act || !wblob) return W4A4_ERR_NULL;
  if (!aligned(act, 256) || !aligned(wblob, 256)) return W4A4_ERR_ALIGN;
  ActGeom ag = act_geom(M, K, R);
  WeightGeom wg = weight_geom(N, K, R);
  const uint8_t* ab = static_cast<const uint8_t*>(act);
  const uint8_t* wb = static_cast<const uint8_t*>(wblob);
  a->xq = ab + ag.off_xq;
  a->sx = reinterpret_cast<const uint16_t*>(ab + ag.off_sx);
  a->la = reinterpret_cast<const float*>(ab + ag.off_la);
  a->wq = wb + wg.off_wq;
  a->sw = reinterpret_cast<const uint16_t*>(wb + wg.off_sw);
  a->lup = reinterpret_cast<const uint16_t*>(wb + wg.off_lup);
  a->ca = reinterpret_cast<const float*>(wb + wg.off_a);
  a->cb = reinterpret_cast<const float*>(wb + wg.off_b);
  a->y = y;
  a->ldy = ldy;
  a->M = M;
  a->N = N;
  a->K = K;
  a->R = R;
  a->ks = ag.ks;
  // y must not overlap either blob
  if (y) {
    const uint8_t* yb = reinterpret_cast<const uint8_t*>(y);
    const uint8_t* ye = yb + (size_t)(M > 0 ? (M - 1) * ldy + ycols : 0) * 2;
    if ((yb < ab + ag.total && ab < ye) || (yb < wb + wg.total && wb < ye)) return W4A4_ERR_ARG;
  }
  return W4A4_OK;
}

// y holds N columns, or N/2 for the gated output (one per (gate, up) pair).
static int linear_impl(int64_t M, int64_t N, int64_t K, int32_t R, const void* act,
                       const void* wblob, uint16_t* y, int64_t ldy, void* stream, bool glu,
                       int32_t r_gate = 0) {
  int st = check_nkr(N, K, R);
  if (st) return st;
  if (glu && N % 32 != 0) return W4A4_ERR_SHAPE;   // whole (gate, up) tile pairs
  if (glu && (r_gate < 0 || r_gate > R)) return W4A4_ERR_SHAPE;
  if ((st = check_m(M))) return st;
  if (M == 0) return W4A4_OK;
  if (!y) return W4A4_ERR_NULL;
  const int64_t ycols = glu ? N / 2 : N;
  if (ldy < ycols) return W4A4_ERR_SHAPE;
  if (ldy % 8 != 0 || !aligned(y, 16)) return W4A4_ERR_ALIGN;
  GemmArgs a;
  if ((st = make_gemm_args(M, N, K, R, act, wblob, y, ldy, &a, ycols))) return st;
  a.glu = glu ? 1 : 0;
  a.glu_tlo = r_gate / 16;          // up tiles: blocks wholly at or past r_gate
  a.glu_thi = (r_gate + 15) / 16;   // gate tiles: blocks that reach below r_gate
  const int v = choose_variant(M, N, K, R);
  if (log_enabled())
    std::fprintf(stderr, "%s M=%lld N=%lld K=%lld R=%d -> %s\n", glu ? "w4a4_linear_glu" : "w4a4_linear",
                 (long long)M, (long long)N, (long long)K, R, variant_name(v));
  return hip_status(launch_gemm(a, v, reinterpret_cast<hipStream_t>(stream)));
}

int w4a4_linear(int64_t M, int64_t N, int64_t K, int32_t R, const void* act,
                const void* wblob, uint16_t* y, int64_t ldy, void* stream) {
  return linear_impl(M, N, K, R, act, wblob, y, ldy, stream, false);
}

int w4a4_linear_glu(int64_t M, int64_t N, int64_t K, int32_t R, int32_t r_gate, const void* act,
                    const void* wblob, uint16_t* y, int64_t ldy, void* stream) {
  return linear_impl(M, N, K, R, act, wblob, y, ldy, stream, true, r_gate);
}

// Workspace of w4a4_linear_glu_quant: room for either route -- the
// per-group LoRA-down partials [H/64][Mp][R_down] fp32 of the quantizing
// epilogue, or h itself [M][H] fp16 on the way through the activation pass.
static size_t glu_quant_workspace(int64_t M, int64_t N, int32_t R_down) {
  const int64_t H = N / 2;
  if (M <= 0) return 0;
  const size_t parts = (size_t)(H / kGroup) * round_up16(M) * R_down * 4, h = (size_t)M * H * 2;
  return align256(parts > h ? parts : h);
}

// The quantizing epilogue needs workgroups that each hold a 64-column group
// of h: ceil(M/64) x H/64 of them at 64 rows.  Below 128 such workgroups (M
// <= 128 at H = 3072) the chip is too empty for it to pay: h goes through
// the workspace and the activation pass instead (measured at H = 3072, K =
// 1024: M = 64, 13.5 against 10.8 us; M = 256, 14.4 against 15.2 us).  M <=
// 16 always takes that route (the decode kernels' workgroups hold 16 or 32
// columns of h).  W4A4_GLU_QUANT_EPILOGUE=0 / 1 forces the route for M > 16
// (tuning and test aid, read at every call like the W4A4_TILED_* overrides).
static bool glu_quant_in_epilogue(int64_t M, int64_t H) {
  if (M <= 16) return false;
  const char* e = std::getenv("W4A4_GLU_QUANT_EPILOGUE");
  if (e && (e[0] == '0' || e[0] == '1')) return e[0] == '1';
  return ((M + 63) / 64) * (H / kGroup) >= 128;
}

// [a, a + na) and [b, b + nb) share a byte (a NULL pointer covers nothing)
static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uint8_t* pa = static_cast<const uint8_t*>(a);
  const uint8_t* pb = static_cast<const uint8_t*>(b);
  return pa && pb && na > 0 && nb > 0 && pa < pb + nb && pb < pa + na;
}

static int check_glu_quant(int64_t M, int64_t N, int64_t K, int32_t R, int32_t r_gate, int32_t R_down) {
  int st = check_nkr(N, K, R);
  if (st) return st;
  if (N % 32 != 0 || r_gate < 0 || r_gate > R) return W4A4_ERR_SHAPE;
  if ((N / 2) % kKPair != 0) return W4A4_ERR_SHAPE;   // h is the next layer's K
  if ((st = check_nkr(16, N / 2, R_down))) return st;
  return check_m(M);
}

int w4a4_glu_quant_workspace(int64_t M, int64_t N, int32_t R_down, size_t* bytes) {
  if (!bytes) return W4A4_ERR_NULL;
  *bytes = 0;
  if (N < 256 || N % 256 != 0 || R_down < 0 || R_down > kMaxRank || R_down % 16 != 0) return W4A4_ERR_SHAPE;
  int st = check_m(M);
  if (st) return st;
  *bytes = glu_quant_workspace(M, N, R_down);
  return W4A4_OK;
}

}  // extern "C"

// w4a4_linear_glu_quant, or with validate_only its argument checks alone
// (the workspace may then be NULL: it is not checked).
int w4a4::glu_quant_call(int64_t M, int64_t N, int64_t K, int32_t R, int32_t r_gate, const void* act,
                         const void* wblob, int32_t R_down, const void* down_wblob, void* act_out,
                         void* workspace, void* stream, bool validate_only) {
  int st = check_glu_quant(M, N, K, R, r_gate, R_down);
  if (st) return st;
  if (M == 0) return W4A4_OK;
  const int64_t H = N / 2;
  const size_t ws = glu_quant_workspace(M, N, R_down);
  if (!act || !wblob || !act_out || (R_down > 0 && !down_wblob) || (ws > 0 && !workspace && !validate_only))
    return W4A4_ERR_NULL;
  if (!aligned(act, 256) || !aligned(wblob, 256) || !aligned(act_out, 256) ||
      (down_wblob && !aligned(down_wblob, 256)) || (workspace && !aligned(workspace, 256)))
    return W4A4_ERR_ALIGN;
  const ActGeom og = act_geom(M, H, R_down);
  const size_t at = act_geom(M, K, R).total, wt = weight_geom(N, K, R).total;
  // the down layer's blob is read only for L_down, its first section
  const size_t dt = R_down > 0 ? (size_t)H * R_down * 2 : 0;
  if (overlaps(act_out, og.total, act, at) || overlaps(act_out, og.total, wblob, wt) ||
      overlaps(act_out, og.total, down_wblob, dt) || overlaps(act_out, og.total, workspace, ws) ||
      overlaps(workspace, ws, act, at) || overlaps(workspace, ws, wblob, wt) || overlaps(workspace, ws, down_wblob, dt))
    return W4A4_ERR_ARG;
  if (validate_only) return W4A4_OK;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const bool in_epilogue = glu_quant_in_epilogue(M, H);
  if (log_enabled())
    std::fprintf(stderr, "w4a4_linear_glu_quant M=%lld N=%lld K=%lld R=%d R_down=%d -> %s\n", (long long)M,
                 (long long)N, (long long)K, R, R_down,
                 in_epilogue ? "prefill, quantized in the epilogue" : "gated GEMM + activation pass");
  if (!in_epilogue) {
    uint16_t* h = static_cast<uint16_t*>(workspace);
    if ((st = linear_impl(M, N, K, R, act, wblob, h, H, stream, true, r_gate))) return st;
    return quantize_act_impl(M, H, R_down, h, H, nullptr, 0.0, down_wblob, act_out, stream);
  }
  GemmArgs a;
  if ((st = make_gemm_args(M, N, K, R, act, wblob, nullptr, N, &a))) return st;
  a.glu = 1;
  a.glu_tlo = r_gate / 16;
  a.glu_thi = (r_gate + 15) / 16;
  uint8_t* ob = static_cast<uint8_t*>(act_out);
  a.qo_xq = ob + og.off_xq;
  a.qo_sx = reinterpret_cast<uint16_t*>(ob + og.off_sx);
  a.qo_part = static_cast<float*>(workspace);
  a.qo_ldown = R_down > 0 ? reinterpret_cast<const uint16_t*>(static_cast<const uint8_t*>(down_wblob) +
                                                              weight_geom(16, H, R_down).off_ldown)
                          : nullptr;
  a.qo_R = R_down;
  a.qo_kp = H / kKPair;
  hipError_t e = launch_gemm_glu_quant(a, s);
  if (e == hipSuccess && R_down > 0)
    e = launch_lora_group_sum(static_cast<const float*>(workspace), og.Mp, R_down, H, og.ks,
                              reinterpret_cast<float*>(ob + og.off_la), s);
  return hip_status(e);
}

extern "C" {

int w4a4_linear_glu_quant(int64_t M, int64_t N, int64_t K, int32_t R, int32_t r_gate, const void* act,
                          const void* wblob, int32_t R_down, const void* down_wblob, void* act_out,
                          void* workspace, void* stream) {
  return glu_quant_call(M, N, K, R, r_gate, act, wblob, R_down, down_wblob, act_out, workspace, stream, false);
}

int w4a4_query_variant(int64_t M, int64_t N, int64_t K, int32_t R) {
  if (check_nkr(N, K, R) || check_m(M)) return -W4A4_ERR_SHAPE;
  return choose_variant(M, N, K, R);
}

// The exact group sums of a window, from the instance of the kernel and tile
// shape that w4a4_linear (glu = false) or w4a4_linear_glu (glu = true) runs
// for this shape, with only its per-group epilogue swapped for the store.
static int group_psums_impl(int64_t M, int64_t N, int64_t K, int32_t R, const void* act,
                            const void* wblob, int64_t m0, int64_t mc, int64_t n0, int64_t nc,
                            int32_t* out, void* stream, bool glu) {
  int st = check_nkr(N, K, R);
  if (st) return st;
  if (glu && N % 32 != 0) return W4A4_ERR_SHAPE;
  if ((st = check_m(M))) return st;
  if (!out) return W4A4_ERR_NULL;
  const int64_t Mp = round_up16(M);
  if (m0 < 0 || n0 < 0 || mc <= 0 || nc <= 0 || m0 % 16 || n0 % 16 || mc % 16 || nc % 16 ||
      m0 + mc > Mp || n0 + nc > N)
    return W4A4_ERR_SHAPE;
  if (!aligned(out, 4)) return W4A4_ERR_ALIGN;
  GemmArgs a;
  if ((st = make_gemm_args(M, N, K, R, act, wblob, nullptr, N, &a))) return st;
  // out must not overlap either blob
  {
    const uint8_t* ob = reinterpret_cast<const uint8_t*>(out);
    const uint8_t* oe = ob + (size_t)mc * nc * (K / kGroup) * 4;
    const uint8_t* ab = static_cast<const uint8_t*>(act);
    const uint8_t* wb = static_cast<const uint8_t*>(wblob);
    const size_t at = act_geom(M, K, R).total, wt = weight_geom(N, K, R).total;
    if ((ob < ab + at && ab < oe) || (ob < wb + wt && wb < oe)) return W4A4_ERR_ARG;
  }
  a.glu = glu ? 1 : 0;
  a.psum = out;
  a.ps_m0 = m0;
  a.ps_mc = mc;
  a.ps_n0 = n0;
  a.ps_nc = nc;
  const int v = choose_variant(M, N, K, R);
  if (log_enabled())
    std::fprintf(stderr, "%s M=%lld N=%lld K=%lld R=%d -> %s\n",
                 glu ? "w4a4_debug_group_psums_glu" : "w4a4_debug_group_psums", (long long)M, (long long)N,
                 (long long)K, R, variant_name(v));
  return hip_status(launch_gemm(a, v, reinterpret_cast<hipStream_t>(stream)));
}

int w4a4_debug_group_psums(int64_t M, int64_t N, int64_t K, int32_t R, const void* act,
                           const void* wblob, int64_t m0, int64_t mc, int64_t n0,
                           int64_t nc, int32_t* out, void* stream) {
  return group_psums_impl(M, N, K, R, act, wblob, m0, mc, n0, nc, out, stream, false);
}

int w4a4_debug_group_psums_glu(int64_t M, int64_t N, int64_t K, int32_t R, const void* act,
                               const void* wblob, int64_t m0, int64_t mc, int64_t n0,
                               int64_t nc, int32_t* out, void* stream) {
  return group_psums_impl(M, N, K, R, act, wblob, m0, mc, n0, nc, out, stream, true);
}

}  // extern "C"
