/*
 * fp4q_peaks.h -- C ABI of libfp4q_peaks: microbenchmarks of the attainable
 * MI355X (gfx950) matrix-core and HBM peaks.  These are measurement
 * infrastructure for reporting the quantized GEMM and quantizer against
 * what the chip delivers in practice, next to its published peaks (dense
 * FP4 MFMA 10.1 PFLOP/s, f16 2.5 PFLOP/s, HBM3E 8 TB/s).  They compute
 * nothing of the quantization method.
 *
 * Conventions: device pointers owned by the caller; every call is
 * asynchronous on the caller's HIP stream (void*, NULL = default stream);
 * time a call with HIP events on that stream.  Return 0, -1 for an invalid
 * argument (checked before any HIP call), -4 for a HIP launch error
 * (fp4q_peaks_last_hip_error() then holds the hipError_t, thread-local).
 */
#ifndef FP4Q_PEAKS_H
#define FP4Q_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* hipError_t of the last -4 on the calling thread (0 if none). */
int fp4q_peaks_last_hip_error(void);

/* Floats of `out` that fp4q_peak_mfma writes for `blocks` workgroups. */
int64_t fp4q_peak_mfma_out_floats(int32_t blocks);

/* Matrix-core throughput: `blocks` workgroups of 4 waves, each wave running
 * `iters` rounds of 8 independent accumulator chains.
 *   kind 0: v_mfma_f32_32x32x16_f16 (32,768 flops each);
 *   kind 1: v_mfma_scale_f32_32x32x64_f8f6f4 on random FP4 codes with unit
 *           E8M0 scales (131,072 flops each).
 *   out    device f32 [fp4q_peak_mfma_out_floats(blocks)], one sum per lane
 *          (keeps the work observable)
 *   flops  host double: receives the flops the launch performs */
int fp4q_peak_mfma(int32_t kind, int32_t blocks, int32_t iters, float* out, double* flops,
                   void* stream);

/* HBM streaming read of `bytes` (a multiple of 16, buf 16-byte aligned) by
 * `blocks` workgroups of 256 lanes, 16 bytes per lane per load;
 * out: device u32 [blocks * 256], one XOR per lane. */
int fp4q_peak_read(const void* buf, uint64_t bytes, int32_t blocks, uint32_t* out, void* stream);

/* HBM streaming copy of `bytes` from src to dst (both 16-byte aligned,
 * non-overlapping): `bytes` read plus `bytes` written. */
int fp4q_peak_copy(const void* src, void* dst, uint64_t bytes, int32_t blocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FP4Q_PEAKS_H */
