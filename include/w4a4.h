/*
 * w4a4.h -- C ABI of libw4a4.so: a W4A4 linear layer with a fused low-rank
 * (LoRA / SVDQuant) correction and a column-wise affine, for AMD MI355X
 * (gfx950).
 *
 *   Y[m,n] = a[n] * ( sum_g s_x[m,g] s_w[n,g] P[m,n,g]
 *                     + sum_r lora_act[m,r] L_up[n,r] ) + b[n]
 *   P[m,n,g]      = sum over the 64 k of group g of q_x[m,k] q_w[n,k]
 *   lora_act[m,r] = sum_k X[m,k] L_down[k,r]
 *
 * Sources: "W4A4 CUDA Kernel for Voice Clone: From Profiling to 2.6x Faster
 * Than FP16" (section 2.1 low-rank correction; 2.3 checkpoint tensors; 3.4
 * the three-kernel forward; 3.6 fused quantize + LoRA-down; 3.7 GEMM +
 * per-group dequant + LoRA-up), and "High-Performance Kernel Design for W4A4
 * Quantized Matrix Multiplication on Blackwell Architecture" (section 1:
 * scaled low-bit matmul + low-rank residual + column-wise affine).
 *
 * Conventions shared by every call
 * --------------------------------
 * - Every pointer argument is a DEVICE pointer unless stated otherwise; fp16
 *   tensors are passed as uint16_t bit patterns.  `stream` is a hipStream_t
 *   (NULL = the legacy default stream).  Every call only enqueues work on
 *   `stream` and returns; nothing is synchronized.
 * - The library allocates no memory and keeps no per-call state: the caller
 *   owns every buffer (sizes come from w4a4_weight_layout / w4a4_act_layout).
 * - Arguments are validated on the host before anything is enqueued; on error
 *   nothing is launched and a non-zero w4a4_status is returned.  Shapes the
 *   kernels do not support return W4A4_ERR_SHAPE; there is no fallback path.
 * - Shape rules: K % 128 == 0 (two 64-wide quantization groups per 128),
 *   N % 16 == 0, R % 16 == 0 with 0 <= R <= 64, M >= 0 (M == 0 is a no-op).
 *   Mp = M rounded up to a multiple of 16 (padding rows of the activation
 *   blob hold q = 0 and scale 0).
 * - Inputs must be finite.
 * - Calls that write the same buffer must not overlap on different streams.
 *
 * Packed layouts (the one definition of both blobs)
 * -------------------------------------------------
 * Codes: q in [-8, 7] stored as the low 4 bits of q (two's complement).
 * A "16 x 128 tile" of codes (16 rows of X, or 16 rows n of W, times 128
 * consecutive k = two 64-groups) is 1024 bytes: lane l = r + 16*c
 * (r = row in tile 0..15, c = 0..3) owns bytes [16*l, 16*l + 16):
 * bytes 0..7 hold group 0 of the tile and bytes 8..15 group 1; within a
 * group's 8 bytes, byte b holds k = 16*c + 2*b (low nibble) and 16*c + 2*b + 1
 * (high nibble), k counted from the start of that group.
 *
 * Weight blob (w4a4_pack_weights writes it; offsets from w4a4_weight_layout;
 * every section starts on a 256-byte boundary), KP = K/128, G = K/64:
 *   [0] L_down: fp16, [KP][R/16][4][64][8]: entry (p, t, s, l = n + 16c, j)
 *       = L_down[128p + 64*(s/2) + 16c + 8*(s%2) + j][16t + n]
 *   [1] W_q:    [N/16][KP] tiles of 1024 bytes (layout above, rows = n)
 *   [2] s_w:    fp16, [N/16][KP][16][2]: entry (nt, p, i, h) = s_w[16nt+i][2p+h]
 *   [3] L_up:   fp16, [N/16][R/16][64][4]: entry (nt, t, l = i + 16c, j)
 *       = L_up[16nt + i][16t + 4c + j]
 *   [4] a:      fp32 [N]   (column scale)
 *   [5] b:      fp32 [N]   (bias)
 * Activation blob (w4a4_quantize_act writes it; offsets from w4a4_act_layout):
 *   [0] X_q:      [Mp/16][KP] tiles of 1024 bytes (rows = m)
 *   [1] s_x:      fp16, [Mp/16][KP][16][2]: entry (mt, p, i, h) = s_x[16mt+i][2p+h]
 *   [2] lora_act: fp32 [S][Mp][R] row-major partial sums: partial j covers the
 *       k-pairs [j*KP/S, (j+1)*KP/S) (integer division) and lora_act is their
 *       sum taken in order j = 0..S-1.  S ("lora splits") depends only on
 *       (M, K) and is reported by w4a4_act_layout: for M <= 16,
 *       S = clamp(KP / 4, 1, 8); for M > 16, S is the smallest power of two
 *       with ceil(M/16) * S >= 256, capped at 4 and at KP / 8 (every split
 *       keeps at least 8 k-pairs; S = 1 when KP < 16 or ceil(M/16) >= 256).
 */
#ifndef W4A4_H_
#define W4A4_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Return codes of every call below. */
typedef enum {
  W4A4_OK = 0,
  W4A4_ERR_NULL = 1,   /* a required pointer is NULL                       */
  W4A4_ERR_SHAPE = 2,  /* a shape rule above is violated (no fallback)     */
  W4A4_ERR_ALIGN = 3,  /* a pointer or leading dimension is misaligned     */
  W4A4_ERR_ARG = 4,    /* inconsistent optional arguments                  */
  W4A4_ERR_HIP = 5     /* the HIP runtime reported an error at launch      */
} w4a4_status;

/* Static, NUL-terminated name of a status code (host only, never NULL). */
const char* w4a4_status_string(int status);

/* Sizes of the weight blob (host-only, no GPU needed).  total_bytes and
 * offsets[6] (section order as above) are HOST pointers; offsets may be NULL.
 * Errors: W4A4_ERR_NULL if total_bytes is NULL, W4A4_ERR_SHAPE on bad shapes. */
int w4a4_weight_layout(int64_t N, int64_t K, int32_t R,
                       size_t* total_bytes, size_t* offsets);

/* Sizes of the activation blob for M rows (host-only).  offsets[3] as above
 * and the number S of LoRA-down partial sums; offsets and lora_splits may be
 * NULL.  Errors as for w4a4_weight_layout. */
int w4a4_act_layout(int64_t M, int64_t K, int32_t R,
                    size_t* total_bytes, size_t* offsets, int32_t* lora_splits);

/* Offline weight preparation, once per layer ("W4A4 CUDA Kernel for Voice
 * Clone", section 2.3: repack the checkpoint into the kernel's layout once at
 * load).  Exactly one source of codes is given:
 *   w_fp16 [N][K] fp16 row-major: quantized here with the activation rule
 *     (per (n, 64-group) absmax, scale fp16(absmax/7), round-half-even);
 *   or qweight [N][K/2] uint8 (byte j: k=2j low nibble, k=2j+1 high nibble,
 *     two's complement) together with w_scales [N][K/64] fp16.
 * lora_down [K][R] and lora_up [N][R] fp16 row-major (both ignored if R==0,
 * required otherwise).  col_scale, bias fp32 [N] (NULL -> 1 and 0).
 * wblob: device buffer of w4a4_weight_layout's total_bytes, 256-byte aligned.
 * Pointers must be 16-byte aligned, except qweight / w_scales / col_scale /
 * bias / lora_* which need only their element alignment. */
int w4a4_pack_weights(int64_t N, int64_t K, int32_t R,
                      const uint16_t* w_fp16, const uint8_t* qweight,
                      const uint16_t* w_scales, const uint16_t* lora_down,
                      const uint16_t* lora_up, const float* col_scale,
                      const float* bias, void* wblob, void* stream);

/* Per forward, kernel 1 ("W4A4 CUDA Kernel for Voice Clone", section 3.6):
 * reads X once and writes the activation blob: int4 codes and fp16 scales per
 * (row, 64-group) -- scale = fp16(fp32(absmax/7)), a zero scale replaced by
 * 2^-24, q = clamp(rint(x / scale), -8, 7) with an IEEE fp32 division -- and
 * lora_act = X L_down (fp32, from the fp16 X, not the codes).
 * x: fp16 [M][ldx], ldx >= K, ldx % 8 == 0, 16-byte aligned.
 * wblob: a blob packed for this (K, R) (any N).  act: device buffer of
 * w4a4_act_layout's total_bytes, 256-byte aligned. */
int w4a4_quantize_act(int64_t M, int64_t K, int32_t R, const uint16_t* x,
                      int64_t ldx, const void* wblob, void* act, void* stream);

/* Per forward, the RMSNorm in front of a projection fused into kernel 1
 * ("W4A4 CUDA Kernel for Voice Clone", section 3.1: an RMSNorm precedes the
 * q/k/v and gate/up projections; section 3.9: the norm's 1/sqrt(mean(x^2) +
 * eps) runs over all K columns of a row): the activation blob is exactly what
 * w4a4_quantize_act writes for the normalized rows
 *     xn[m][k] = fp16(fp32((x[m][k] * inv[m]) * gamma[k])),
 *     inv[m]   = 1 / sqrt((sum_k x[m][k]^2) / K + eps),
 * with inv, the sum and both products in fp64 (the sum's order is the
 * kernel's; everything after it is fixed).  The normalized rows themselves
 * are not written out.
 * gamma: fp16 [K], 16-byte aligned.  eps: > 0 and finite (else
 * W4A4_ERR_ARG).  Other arguments, layouts and errors as w4a4_quantize_act. */
int w4a4_quantize_act_rmsnorm(int64_t M, int64_t K, int32_t R, const uint16_t* x,
                              int64_t ldx, const uint16_t* gamma, double eps,
                              const void* wblob, void* act, void* stream);

/* Per forward, kernel 2 ("W4A4 CUDA Kernel for Voice Clone", section 3.7;
 * affine: Blackwell article, section 1): Y = a * (int4 GEMM with per-group
 * fp32 dequant + lora_act L_up^T) + b, rounded to fp16.
 * act from w4a4_quantize_act with the same (M, K, R); wblob from
 * w4a4_pack_weights with the same (N, K, R).
 * y: fp16 [M][ldy], ldy >= N, ldy % 8 == 0, 16-byte aligned, not aliasing
 * act or wblob.  Rows m >= M are never written. */
int w4a4_linear(int64_t M, int64_t N, int64_t K, int32_t R, const void* act,
                const void* wblob, uint16_t* y, int64_t ldy, void* stream);

/* The gate and up projections of a gated MLP as one layer, and its gated
 * activation in the GEMM's epilogue ("W4A4 CUDA Kernel for Voice Clone",
 * section 3.1: the Qwen3 MLP computes SiLU(gate_proj(x)) * up_proj(x); gate
 * and up read the same X, so one w4a4_quantize_act serves both).
 * wblob: packed (w4a4_pack_weights) from the two layers interleaved by
 * 16-row tiles -- rows [32j, 32j+16) are gate rows [16j, 16j+16), rows
 * [32j+16, 32j+32) up rows [16j, 16j+16) -- with L_down = [L_down_gate |
 * L_down_up] ([K][Rg + Ru]) and the L_up rows of a gate row being
 * [L_up_gate row, 0], of an up row [0, L_up_up row] (so the low-rank term of
 * each half is exactly its own layer's); a and b interleaved the same way.
 * N = 2 * (columns of each layer), N % 32 == 0; R = Rg + Ru; r_gate = Rg,
 * 0 <= r_gate <= R: the kernel skips the 16-wide rank blocks of L_up that the
 * block-diagonal packing makes zero for a half (a wrong r_gate drops LoRA
 * terms; r_gate only steers that skip, it is not checked against wblob).
 * y: fp16 [M][ldy], ldy >= N/2, ldy % 8 == 0, 16-byte aligned:
 *     y[m][c] = fp16(SiLU(g) * u),  g = gate layer's fp16 output (m, c),
 *                                   u = up layer's fp16 output (m, c),
 * SiLU in fp32 with the hardware exponential and reciprocal (relative error
 * about 1e-6 before the fp16 rounding).  Other arguments and errors as w4a4_linear
 * (W4A4_ERR_SHAPE also if N % 32 != 0 or r_gate is outside [0, R]). */
int w4a4_linear_glu(int64_t M, int64_t N, int64_t K, int32_t R, int32_t r_gate, const void* act,
                    const void* wblob, uint16_t* y, int64_t ldy, void* stream);

/* The gated layer whose output goes straight into the next layer's
 * activation blob ("W4A4 CUDA Kernel for Voice Clone", section 3.1: the MLP
 * computes SiLU(gate) * up and feeds it to the W4A4 down projection; section
 * 3.6: that projection's activation pass).  h = fp16(SiLU(g) * u) is
 * exactly what w4a4_linear_glu(M, N, K, R, r_gate, act, wblob, ...) would
 * store, and act_out becomes what w4a4_quantize_act(M, N/2, R_down, h, N/2,
 * down_wblob, act_out) would write from it: codes and scales bit for bit,
 * lora_act equal up to the order of its fp32 sums.  Where the grid is large
 * enough (M > 16 and ceil(M/64) * N/128 >= 128) h never goes to memory in
 * fp16: the GEMM's epilogue quantizes each 64-column group of h and computes
 * that group's share of LoRA-down (into workspace), and a second kernel sums
 * the shares in group order into lora_act (deterministic).  Otherwise
 * (decode sizes, small grids) the call runs w4a4_linear_glu into workspace,
 * then the activation pass.
 * N: packed gate/up columns as for w4a4_linear_glu, with N/2 % 128 == 0 (N/2
 * is the next layer's K).  R_down: the next layer's LoRA rank (0..64, % 16);
 * down_wblob: its weight blob (w4a4_weight_layout(N_down, N/2, R_down));
 * only its L_down section is read, NULL allowed when R_down == 0.
 * act_out: activation blob of w4a4_act_layout(M, N/2, R_down), 256-byte
 * aligned.  workspace: device buffer of w4a4_glu_quant_workspace bytes,
 * 256-byte aligned (NULL allowed when that is 0); its contents are scratch.
 * act_out and workspace must not overlap each other or any input
 * (W4A4_ERR_ARG).  Other arguments and errors as w4a4_linear_glu
 * (W4A4_ERR_SHAPE also when N/2 % 128 != 0 or R_down is invalid). */
int w4a4_linear_glu_quant(int64_t M, int64_t N, int64_t K, int32_t R, int32_t r_gate,
                          const void* act, const void* wblob, int32_t R_down,
                          const void* down_wblob, void* act_out, void* workspace,
                          void* stream);

/* Bytes of workspace w4a4_linear_glu_quant needs for (M, N, R_down)
 * (host-only): the larger of 4 * (N/128) * Mp * R_down (the LoRA-down
 * shares) and 2 * M * N/2 (h), rounded up to 256; 0 for M = 0.
 * W4A4_ERR_SHAPE for N not a positive multiple of 256, an invalid R_down or
 * M out of range. */
int w4a4_glu_quant_workspace(int64_t M, int64_t N, int32_t R_down, size_t* bytes);

/* w4a4_linear_glu_quant for callers that cannot allocate (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same call and results, with the workspace taken from a library-owned
 * device array of W4A4_NOALLOC_SCRATCH_BYTES bytes per GPU (file-scope
 * device memory, held by every GPU the library runs on until the process
 * ends) instead of an argument.  Allocates nothing.  The array keeps the
 * last call's contents (no call needs them cleared); calls that overlap on
 * one GPU -- on different streams or from different host threads -- share
 * it and race.  W4A4_ERR_SHAPE when w4a4_glu_quant_workspace(M, N, R_down)
 * exceeds the array (use w4a4_linear_glu_quant with a workspace of its own
 * then); W4A4_ERR_HIP if the array's device address cannot be obtained.
 * Other arguments and errors as w4a4_linear_glu_quant. */
#define W4A4_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int w4a4_linear_glu_quant_noalloc(int64_t M, int64_t N, int64_t K, int32_t R, int32_t r_gate,
                                  const void* act, const void* wblob, int32_t R_down,
                                  const void* down_wblob, void* act_out, void* stream);

/* Which GEMM kernel w4a4_linear runs for a shape (host-only):
 * 1 = decode (M <= 16), 2 = prefill (tiled); -W4A4_ERR_SHAPE if the
 * shape is unsupported.  Lets a caller log the kernel chosen per layer
 * ("INT4 Kernel Architecture, in depth", section "Failure modes"). */
int w4a4_query_variant(int64_t M, int64_t N, int64_t K, int32_t R);

/* Diagnostic: the exact per-group integer sums P[m,n,g] ("W4A4 CUDA Kernel
 * for Voice Clone", section 3.7: the int32 sum of each 64-group before the
 * per-group dequant) of a window of the output.  The launch runs the same
 * kernel, tile shape and variant that w4a4_linear runs for (M, N, K, R) --
 * its loads, nibble expansion and integer products unchanged -- with only
 * the per-group scale-accumulate swapped for a store of P, and no LoRA, affine
 * or output (the LoRA rank only steers which kernel is chosen).  Rows of the
 * window at or past M are padding and read 0.
 * act, wblob: as for w4a4_linear.  out: int32 device buffer [mc][nc][K/64]
 * (row-major), not overlapping act or wblob (else W4A4_ERR_ARG).  m0, mc,
 * n0, nc must be multiples of 16 with m0 + mc <= Mp and n0 + nc <= N (else
 * W4A4_ERR_SHAPE). */
int w4a4_debug_group_psums(int64_t M, int64_t N, int64_t K, int32_t R,
                           const void* act, const void* wblob, int64_t m0,
                           int64_t mc, int64_t n0, int64_t nc, int32_t* out,
                           void* stream);

/* The same for the kernel and tile shape w4a4_linear_glu runs for a gated
 * layer of N packed columns (N % 32 == 0): P of the packed (interleaved gate
 * / up) columns, before the gated activation. */
int w4a4_debug_group_psums_glu(int64_t M, int64_t N, int64_t K, int32_t R,
                               const void* act, const void* wblob, int64_t m0,
                               int64_t mc, int64_t n0, int64_t nc, int32_t* out,
                               void* stream);

/* Captured forward passes ("W4A4 CUDA Kernel for Voice Clone", section 4:
 * launch overhead dominates decode-size calls, so the forward step is
 * replayed from graphs, one pre-captured per bucket of the row count).
 * A graph bakes in every argument of the calls it holds: the shapes, the
 * weight blobs and the x / act / y buffers.  The caller writes each
 * request's rows into the captured x buffers (rows past the request's own
 * should hold finite values, zeros say), replays, and reads the rows it
 * needs; every replay recomputes all captured rows.  Buffers must stay
 * valid while the graph exists; replays of one graph must not overlap (they
 * share its buffers).  None of the library's kernels uses a memset or an
 * allocation, so a graph holds kernel nodes only. */
typedef struct w4a4_graph w4a4_graph;

/* Capture every library call enqueued on stream (not NULL: the legacy
 * default stream cannot be captured) from w4a4_graph_begin to
 * w4a4_graph_end -- a whole step of many layers, say.  Calls made in between
 * are recorded, not run; their own argument errors are returned by them as
 * usual.  w4a4_graph_end ends the capture in every case and returns
 * W4A4_ERR_HIP if it or the instantiation fails (*out = NULL then). */
int w4a4_graph_begin(void* stream);
int w4a4_graph_end(void* stream, w4a4_graph** out);

/* One layer captured on a private stream: the activation pass
 * (w4a4_quantize_act, or w4a4_quantize_act_rmsnorm when gamma is not NULL)
 * followed by w4a4_linear, for exactly these arguments (M > 0 is the
 * bucket).  The calls' shape and argument errors are returned and nothing is
 * kept; W4A4_ERR_HIP if capture or instantiation fails. */
int w4a4_layer_graph_create(int64_t M, int64_t N, int64_t K, int32_t R,
                            const uint16_t* x, int64_t ldx, const uint16_t* gamma,
                            double eps, const void* wblob, void* act, uint16_t* y,
                            int64_t ldy, w4a4_graph** out);

/* Enqueue one replay on stream (asynchronous). */
int w4a4_graph_launch(w4a4_graph* graph, void* stream);
/* Free the graph (NULL is a no-op).  Replays already enqueued must have
 * completed. */
int w4a4_graph_destroy(w4a4_graph* graph);

#ifdef __cplusplus
}
#endif

#endif /* W4A4_H_ */
