/*
 * moe_peak.h -- measured peaks of the GPU (libmoe_peak_gfx950.so), reported
 * next to the published MI355X figures by the benchmark.  Not part of the MoE
 * path: measurement only.
 *
 * Status: 0 ok, 1 invalid argument, 4 launch failed (the MoE library's codes).
 * All pointers are device pointers owned by the caller; each call enqueues
 * one kernel on `stream` (hipStream_t as void*) and returns.
 */
#ifndef MOE_PEAK_H_
#define MOE_PEAK_H_

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Floating-point operations one moe_peak_mfma(workgroups, iters) launch
 * performs (-1 for invalid sizes). */
long long moe_peak_mfma_flops(int workgroups, int iters);

/* MFMA-only loop: `workgroups` workgroups of 4 wavefronts, each wavefront
 * issuing iters * 8 independent bf16 v_mfma_f32_32x32x16 with fp32
 * accumulation.  sink: workgroups * 256 floats, written only in a case that
 * never happens (it keeps the loop alive). */
int moe_peak_mfma(int workgroups, int iters, float *sink, void *stream);

/* Read-only stream of `bytes` (16-byte aligned buffer; the last bytes % 16
 * are not read) by `workgroups` workgroups of 256 threads, each reading its
 * own contiguous part with 16-byte loads.  sink: `workgroups` unsigned,
 * written only in a case that never happens. */
int moe_peak_read(const void *buf, size_t bytes, int workgroups, unsigned *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_PEAK_H_ */
