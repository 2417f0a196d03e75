/*
 * ceilings.h -- C ABI of libbqceil.so: two microbenchmarks that measure, on
 * the machine at hand, the ceilings of the rooflines the MoE layer's kernels
 * are reported against (an HBM read stream for decode, dense bf16
 * matrix-core work for prefill).  Only the benchmark uses them.
 *
 * Conventions as in moe.h: device pointers, a hipStream_t (NULL = null
 * stream), calls enqueue and return; 0 = success, 1 = bad argument, other
 * values are HIP error codes of the launch.
 */
#ifndef BQMOE_CEILINGS_H
#define BQMOE_CEILINGS_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* One launch that reads `bytes` (a multiple of 16) of device memory `src`
 * with `blocks` workgroups of 256 lanes, each lane keeping `unroll` (1, 2 or
 * 4) 16-byte loads in flight.  `sink` (device, >= blocks * 4 bytes) is
 * written only in a case that does not occur; it keeps the loads live. */
int bqc_read_stream(const void* src, size_t bytes, int blocks, int unroll, uint32_t* sink,
                    void* stream);

/* One launch of `blocks` workgroups of 4 waves, each wave issuing `iters`
 * rounds of four independent 32x32x16 bf16 matrix-core ops on register
 * operands (no memory traffic).  `sink` as above (>= blocks * 4 bytes). */
int bqc_mfma_bf16(int blocks, int iters, float* sink, void* stream);

/* Floating-point operations of one bqc_mfma_bf16 launch. */
double bqc_mfma_bf16_flops(int blocks, int iters);

#ifdef __cplusplus
}
#endif

#endif
