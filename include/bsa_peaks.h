/*
 * bsa_peaks.h -- attainable-peak microbenchmarks of libbsa_peaks.so (gfx950).
 *
 * They give the measured denominators that roofline fractions are also
 * reported against, next to the vendor figures (HBM3E 8 TB/s, dense bf16
 * MFMA 2.5 PFLOP/s).  Not part of the attention path.  Pointers are HIP
 * device pointers; stream is a hipStream_t (NULL = legacy default stream);
 * work is enqueued asynchronously; nothing is allocated.  Return 0 on
 * success, 1 for a bad argument, 5 for a failed launch.
 */
#ifndef BSA_PEAKS_H
#define BSA_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Streaming read of `bytes` (a multiple of 16, buffer 16-byte aligned) by
 * `workgroups` workgroups of 256 threads with 16-byte non-temporal loads.
 * sink: one device word, written only if the data hash hits a fixed pattern. */
int32_t bsa_peak_hbm_read(const void* buf, size_t bytes, int32_t workgroups, uint32_t* sink, void* stream);

/* `workgroups` workgroups of 4 waves, each wave issuing `iters` rounds of
 * four independent v_mfma_f32_32x32x16_bf16 on register operands.
 * bsa_peak_mfma_flops gives the flops of such a launch. */
int32_t bsa_peak_mfma_bf16(int32_t iters, int32_t workgroups, float* sink, void* stream);
double bsa_peak_mfma_flops(int32_t iters, int32_t workgroups);

#ifdef __cplusplus
}
#endif

#endif /* BSA_PEAKS_H */
