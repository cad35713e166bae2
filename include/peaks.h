/* libpeaks: device peak probes used to state roofline fractions against what
 * the device in hand sustains, next to the datasheet peaks.  Measurement
 * infrastructure only; the loss itself is in librece (rece.h).
 *
 * Every call enqueues one kernel on `stream` (a hipStream_t, NULL = the null
 * stream) and returns at once; the caller times it with events on that stream.
 * Return value: 0 on success, else a hipError_t code (hipErrorInvalidValue for
 * bad arguments, nothing enqueued).  Nothing is allocated.
 */
#ifndef RECE_PEAKS_H
#define RECE_PEAKS_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Floating-point operations one rece_peak_mfma_bf16(blocks, iters) launch performs. */
double rece_peak_mfma_flops(int blocks, int iters);

/* bf16 matrix-core loop: `blocks` workgroups of 256 threads, each wave issuing
 * `iters` x 8 independent v_mfma_f32_16x16x32_bf16 with no memory traffic.
 * sink: device float[blocks * 256], written once per thread (keeps the work live). */
int rece_peak_mfma_bf16(void* stream, int blocks, int iters, float* sink);

/* Device copy of `bytes` (a multiple of 16; both pointers 16-byte aligned, device
 * memory, not overlapping) with 16-byte loads and stores: moves 2 * bytes of HBM. */
int rece_peak_copy(void* stream, const void* src, void* dst, size_t bytes);

#ifdef __cplusplus
}
#endif

#endif
