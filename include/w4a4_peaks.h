/*
 * w4a4_peaks.h -- C ABI of libw4a4_peaks.so: microbenchmarks that measure the
 * attainable peak of the resources the W4A4 + LoRA linear layer is bound by
 * on MI355X (gfx950) -- dense int8 MFMA issue for large row counts (with the
 * fp32 VALU work of its per-group epilogue beside it), HBM read bandwidth
 * for decode-sized ones ("W4A4 CUDA Kernel for Voice Clone",
 * section 1.2: a kernel is judged against the roofline of the resource that
 * bounds it; "INT4 Kernel Architecture, in depth", "Why INT4 kernels exist":
 * small batches stream weights, large ones are compute-bound).  They stand
 * beside the published peaks in the benchmark; nothing on the layer's path
 * calls them.
 *
 * Pointers are device pointers; every call only enqueues one kernel on
 * `stream` (a hipStream_t, NULL = legacy default) and returns; the caller
 * times it.  Return: 0 on success, 4 on bad arguments (nothing launched),
 * 5 if the launch failed.
 */
#ifndef W4A4_PEAKS_H_
#define W4A4_PEAKS_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* int8 MFMA: 512 workgroups (two per CU, two waves per SIMD), every wave
 * iters x 8 independent v_mfma_i32_16x16x64_i8.  out: int32 device buffer
 * of w4a4_peak_i8_mfma_out_ints() entries (one per thread, written).
 * Integer operations launched = w4a4_peak_i8_mfma_ops(iters). */
int w4a4_peak_i8_mfma(int32_t iters, int32_t* out, void* stream);
int64_t w4a4_peak_i8_mfma_ops(int32_t iters);
int64_t w4a4_peak_i8_mfma_out_ints(void);

/* HBM read: every byte of src[0, bytes) read once with 16-byte non-temporal
 * loads (bytes % 16 == 0, src 16-byte aligned; use a buffer well beyond the
 * 256 MB last-level cache).  out: uint32 device buffer of
 * w4a4_peak_hbm_read_out_ints() entries (written). */
int w4a4_peak_hbm_read(const void* src, uint64_t bytes, uint32_t* out, void* stream);
int64_t w4a4_peak_hbm_read_out_ints(void);

/* Two kinds of work on the same SIMDs ("W4A4 CUDA Kernel for Voice Clone",
 * section 3.7: each group's integer sum is followed by its fp32 dequant on
 * the vector ALUs): one workgroup of 8 waves per CU, waves 0..3 (one per
 * SIMD) doing role_a for iters_a iterations and waves 4..7 role_b for
 * iters_b.  Roles: 0 nothing, 1 = 8 independent v_mfma_i32_16x16x64_i8 per
 * iteration, 2 = 32 independent wave64 v_fma_f32 per iteration.  Timing one
 * role alone and both together gives the unpacked fp32 VALU rate and how
 * far the two overlap.  Roles 3..5 time the GEMM loop's per-tile mix within
 * one wave, 8 tiles per iteration: 3 = per tile one int8 MFMA and, on the
 * tile before's sums, 4 v_fma_f32 and 2 integer ops; 4 = its MFMAs alone;
 * 5 = its VALU ops alone.  Roles 6 and 7 = 8 independent
 * v_mfma_f32_16x16x4_4b_f16 or v_mfma_f32_16x16x32_f16 per iteration (their
 * issue cost).  out: int32 device buffer of
 * w4a4_peak_roles_out_ints() entries.  w4a4_peak_roles_ops(role, iters):
 * int8 operations (role 1) or fp32 FMA lane operations (role 2) of the
 * four waves of one role on every CU. */
int w4a4_peak_roles(int32_t role_a, int32_t role_b, int32_t iters_a, int32_t iters_b,
                    int32_t* out, void* stream);
int64_t w4a4_peak_roles_ops(int32_t role, int32_t iters);
int64_t w4a4_peak_roles_out_ints(void);

#ifdef __cplusplus
}
#endif

#endif /* W4A4_PEAKS_H_ */
