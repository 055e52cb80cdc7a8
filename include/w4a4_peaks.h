/*
 * w4a4_peaks.h -- C ABI of libw4a4_peaks.so: microbenchmarks that measure the
 * attainable peak of the two resources the W4A4 + LoRA linear layer is bound
 * by on MI355X (gfx950) -- dense int8 MFMA issue for large row counts, HBM
 * read bandwidth for decode-sized ones ("W4A4 CUDA Kernel for Voice Clone",
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

#ifdef __cplusplus
}
#endif

#endif /* W4A4_PEAKS_H_ */
