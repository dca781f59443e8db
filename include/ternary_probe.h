/*
 * Measurement probes (libternary_probe.so, a library apart from the layer's): the
 * device's achievable HBM stream and bf16 MFMA rates, measured with kernels of
 * known traffic and flop counts.
 *
 * They are not part of the layer.  A roofline fraction is the layer's rate
 * over a published peak; these kernels measure how much of that peak plain
 * code reaches on this device (a streaming read, a streaming copy, a loop of
 * independent MFMAs), so that a kernel's result can also be read against what
 * is achievable.  They also calibrate hardware counters: the copy moves a known
 * number of bytes, the MFMA loop issues a known number of MFMAs and keeps the
 * matrix cores busy for its whole duration.
 *
 * All pointers are device pointers owned by the caller; every call is
 * asynchronous on `stream` and returns a ternary_status (include/ternary.h).
 * Validation is on the host and launches nothing on error.
 */
#ifndef TERNARY_PROBE_H
#define TERNARY_PROBE_H

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "ternary.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Largest `workgroups` any probe takes. */
#define TERNARY_PROBE_MAX_WORKGROUPS 65536

/*
 * ternary_probe_read - read `bytes` bytes of `src` once, with 16-byte loads,
 * four in flight per lane (a grid-stride loop over `workgroups` workgroups of
 * 256 threads).  Nothing is written except, with vanishing probability, one
 * word of `sink` (a data-dependent store that keeps the loads live).
 *   src         16-byte aligned, bytes % 16 == 0, bytes >= 0 (0 is a no-op).
 *   workgroups  1 .. TERNARY_PROBE_MAX_WORKGROUPS.
 *   sink        one uint32 of device memory.
 */
int ternary_probe_read(const void *src, int64_t bytes, int32_t workgroups, uint32_t *sink,
                       hipStream_t stream);

/*
 * ternary_probe_read_nt - ternary_probe_read with non-temporal loads (the `nt`
 * cache-policy bit, the policy the decode kernels give their code loads);
 * same arguments, errors and traffic.
 */
int ternary_probe_read_nt(const void *src, int64_t bytes, int32_t workgroups, uint32_t *sink,
                          hipStream_t stream);

/*
 * ternary_probe_copy - copy `bytes` bytes from src to dst with 16-byte loads
 * and stores (grid-stride, four in flight per lane); it reads and writes
 * `bytes` bytes each.
 *   src, dst    16-byte aligned, not overlapping, bytes % 16 == 0.
 *   workgroups  1 .. TERNARY_PROBE_MAX_WORKGROUPS.
 */
int ternary_probe_copy(const void *src, void *dst, int64_t bytes, int32_t workgroups,
                       hipStream_t stream);

/*
 * ternary_probe_mfma - every wave of `workgroups` workgroups of 4 waves runs
 * `iters` iterations of four independent v_mfma_f32_16x16x32_bf16 (16384
 * flops each), on register operands, and stores its accumulators' sum: the
 * launch performs workgroups * 4 * iters * 4 * 16384 flops and touches no
 * memory but `out`.
 *   workgroups  1 .. TERNARY_PROBE_MAX_WORKGROUPS.
 *   iters       1 .. 1 << 20.
 *   out         float [workgroups * 256], 4-byte aligned.
 */
int ternary_probe_mfma(int32_t workgroups, int32_t iters, float *out, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* TERNARY_PROBE_H */
