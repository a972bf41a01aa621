/*
 * moe_peaks.h -- measurement kernels (libmoe_peaks.so), not part of the
 * layer: the ceilings that the benchmark reports beside the vendor peaks of
 * the MI355X (HBM 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s).
 *
 * All pointers are device pointers owned by the caller; every call only
 * enqueues one kernel on `stream` (a hipStream_t, NULL = default) and returns
 * 0, -1 for an invalid argument, or a negative value below -1000 for a launch
 * failure (-1000 - hipError_t - 1).
 */
#ifndef MOE_PEAKS_H
#define MOE_PEAKS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* dst = src over `bytes` (a multiple of 16): reads and writes `bytes` each. */
int moe_peak_copy(const void *src, void *dst, size_t bytes, int workgroups, void *stream);

/* Reads `bytes` (a multiple of 16) of src; writes one word per workgroup to
 * sink [workgroups]. */
int moe_peak_read(const void *src, size_t bytes, uint32_t *sink, int workgroups, void *stream);

/* bf16 MFMA 16x16x32 issue rate: `workgroups` workgroups of 4 wavefronts,
 * each running `iters` x 8 independent MFMAs on register operands; writes
 * out [workgroups * 256] floats. moe_peak_mfma_bf16_flops gives the flops
 * of one such launch. */
int moe_peak_mfma_bf16(float *out, int workgroups, int iters, void *stream);
double moe_peak_mfma_bf16_flops(int workgroups, int iters);

#ifdef __cplusplus
}
#endif

#endif
