/*
 * hypic_probe.h -- C ABI of libhypic_probe: a matrix-core rate probe for MI355X
 * (gfx950), kept apart from libhypic.
 *
 * It answers one measurement question: how many dense f16 matrix-core flops per
 * second (and per clock cycle) this GPU sustains when nothing but
 * v_mfma_f32_32x32x16_f16 products run, so that the segment build's rate can be
 * stated against the achievable rate as well as against the 2.5 PFLOP/s
 * specification.  It computes nothing of the method.
 */
#ifndef HYPIC_PROBE_H
#define HYPIC_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* hypic_probe_stream_t; /* a hipStream_t */

/* Flops of one probe launch: n_groups * 8 waves * iters * 4 products * 32768. */
double hypic_probe_mfma_f16_flops(int n_groups, int iters);

/*
 * Enqueues one probe launch on `stream` and returns without waiting: n_groups
 * workgroups of 8 waves (2 per SIMD); each wave keeps 4 independent
 * 32x32x16 f16 products in flight on register operands for `iters` rounds, with
 * no memory traffic until it writes its sums.
 *   sink    device float[n_groups * 512]: the waves' accumulator sums (written so
 *           that the products are not removed; their values carry no meaning).
 *   clocks  device int64[n_groups * 2]: per workgroup, the core-clock cycles
 *           (s_memtime) and the 100 MHz real-time ticks (s_memrealtime) wave 0
 *           measured between its first and last product; cycles / (ticks * 10 ns)
 *           is the clock in that interval.
 * Both buffers are caller-owned device memory.  Returns 0 on success, -1 for
 * n_groups < 1, iters < 1 or a NULL buffer (nothing enqueued), or the hipError_t
 * of the launch.
 */
int hypic_probe_mfma_f16(int n_groups, int iters, float* sink, int64_t* clocks, hypic_probe_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* HYPIC_PROBE_H */
