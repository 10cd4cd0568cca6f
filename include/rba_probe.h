/*
 * rba_probe.h — measurement probes used by the benchmark (librba_probe.so).
 *
 * Not part of the ring-step library: these two kernels measure what the
 * chip sustains, so that the step kernels' rates can be quoted against
 * measured ceilings as well as the datasheet's (dense bf16 MFMA
 * 2.5 PFLOP/s, HBM3E 8 TB/s).
 *
 * Conventions as in rba.h: device pointers of the current HIP device,
 * 16-byte aligned; launches are asynchronous on `stream` (a hipStream_t,
 * NULL = legacy default stream); arguments are checked before any launch and
 * a negative status (RBA_ERR_* values of rba.h) means nothing was launched.
 */
#ifndef RBA_PROBE_H
#define RBA_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * rba_probe_mfma_bf16 — a dense loop of v_mfma_f32_32x32x16_bf16 on register
 * operands (nonzero, lane-varying values): `workgroups` workgroups of 4 waves
 * (launch bounds: 2 workgroups per compute unit, the occupancy of the step
 * kernels), each wave running `iters` iterations of 4 independent
 * accumulator chains.  No memory traffic except one float per thread written
 * at the end into out[workgroups * 256] (device, fp32).
 * *flops_per_launch (host) receives workgroups * 4 * iters * 4 * 32768.
 * Requires 1 <= workgroups, 1 <= iters.
 */
int rba_probe_mfma_bf16(int32_t workgroups, int32_t iters, float* out, double* flops_per_launch, void* stream);

/*
 * rba_probe_copy — dst[0, bytes) = src[0, bytes) with 16-byte vector loads
 * and stores in a grid-stride loop (`workgroups` workgroups of 256 threads).
 * Moves 2 * bytes through HBM when both buffers are far larger than the
 * last-level cache.  bytes must be a positive multiple of 16; src and dst
 * must not overlap.
 */
int rba_probe_copy(const void* src, void* dst, int64_t bytes, int32_t workgroups, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* RBA_PROBE_H */
