// Measured ceilings of the two rooflines the MoE layer is reported against,
// for reporting kernel results beside the chip's spec peaks:
//   - a plain HBM read stream (what a launch of a given size can read), and
//   - dense bf16 matrix-core work with no memory traffic.
// Built as its own library (libbqceil.so); only the benchmark loads it.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"

namespace bqceil {

using bqmoe::f32x16;
using bqmoe::u32x4;

// Each lane keeps U 16-byte loads in flight per iteration; the loaded words
// are folded into one value so that no load is dead.
template <int U>
__global__ __launch_bounds__(256) void k_read(const uint4* __restrict__ p, size_t n16,
                                              uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const size_t bd = blockDim.x;
  const size_t stride = (size_t)gridDim.x * bd * U;
  for (size_t i = (size_t)blockIdx.x * bd * U + threadIdx.x; i + (U - 1) * bd < n16; i += stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) v[u] = p[i + u * bd];
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  if (acc == 0x9E3779B9u) sink[blockIdx.x] = acc;  // practically never
}

// Four independent accumulator chains of 32x32x16 bf16 ops per wave.
__global__ __launch_bounds__(256) void k_mfma(int iters, float* __restrict__ sink) {
  const uint32_t t = threadIdx.x;
  // small distinct bf16 operands (values near 2^-8) per chain
  const u32x4 a0 = {0x3B803B80u ^ (t & 7), 0x3B803B80u, 0x3B803B80u, 0x3B803B80u};
  const u32x4 a1 = {0x3B813B81u, 0x3B803B80u ^ (t & 3), 0x3B803B80u, 0x3B803B80u};
  const u32x4 a2 = {0x3B823B82u, 0x3B803B80u, 0x3B803B80u ^ (t & 5), 0x3B803B80u};
  const u32x4 a3 = {0x3B833B83u, 0x3B803B80u, 0x3B803B80u, 0x3B803B80u ^ (t & 6)};
  const u32x4 b = {0x3B803B80u, 0x3B803B80u, 0x3B803B80u, 0x3B803B80u ^ (t & 1)};
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = bqmoe::mfma32x32(a0, b, c0);
    c1 = bqmoe::mfma32x32(a1, b, c1);
    c2 = bqmoe::mfma32x32(a2, b, c2);
    c3 = bqmoe::mfma32x32(a3, b, c3);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  if (s == 12345.5f) sink[blockIdx.x] = s;  // practically never
}

}  // namespace bqceil

extern "C" {

int bqc_read_stream(const void* src, size_t bytes, int blocks, int unroll, uint32_t* sink,
                    void* stream) {
  if (!src || !sink || blocks <= 0 || (bytes & 15)) return 1;
  const size_t n16 = bytes / 16;
  hipStream_t s = (hipStream_t)stream;
  switch (unroll) {
    case 1: hipLaunchKernelGGL(bqceil::k_read<1>, dim3(blocks), dim3(256), 0, s, (const uint4*)src, n16, sink); break;
    case 2: hipLaunchKernelGGL(bqceil::k_read<2>, dim3(blocks), dim3(256), 0, s, (const uint4*)src, n16, sink); break;
    case 4: hipLaunchKernelGGL(bqceil::k_read<4>, dim3(blocks), dim3(256), 0, s, (const uint4*)src, n16, sink); break;
    default: return 1;
  }
  return (int)hipGetLastError();
}

int bqc_mfma_bf16(int blocks, int iters, float* sink, void* stream) {
  if (!sink || blocks <= 0 || iters <= 0) return 1;
  hipLaunchKernelGGL(bqceil::k_mfma, dim3(blocks), dim3(256), 0, (hipStream_t)stream, iters, sink);
  return (int)hipGetLastError();
}

double bqc_mfma_bf16_flops(int blocks, int iters) {
  return (double)blocks * 4 /* waves */ * iters * 4 /* ops */ * (32.0 * 32.0 * 16.0 * 2.0);
}

}  // extern "C"
