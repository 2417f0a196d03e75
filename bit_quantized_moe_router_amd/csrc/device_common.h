// Device helpers for the gfx950 kernels: number conversions, wavefront
// reductions, matrix-core wrappers and the packed-code unpackers.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bqmoe {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// round to nearest even; NaN stays NaN
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0x7FC0u;
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float f16_to_f32(uint32_t h16) {
  _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)h16);
  return (float)h;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// 16x16x32 bf16 matrix-core op (gfx950): lane l supplies A[l%16][8(l/16)..+7] and
// B[8(l/16)..+7][l%16]; it receives D[4(l/16)+i][l%16], i = 0..3.
__device__ __forceinline__ f32x4 mfma32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}
// Correction term of one 32-group as a 16x16x32 op (same shape as the main op,
// so the main op can take it as its C operand without a mixed-shape dependency):
// lanes 0..15 put the row's bf16 triple (-hi, -mid, -lo, 0) in k-slots 0..3 of A
// and (c, c, c, 0) in k-slots 0..3 of B; every other slot is zero.  Result:
// D[row][col] = -c * (hi + mid + lo)[row] for every column.
__device__ __forceinline__ f32x4 mfma_corr(u32x2 a, u32x2 b) {
  const u32x4 a4 = {a[0], a[1], 0u, 0u}, b4 = {b[0], b[1], 0u, 0u};
  return mfma32(a4, b4, f32x4{0.f, 0.f, 0.f, 0.f});
}

// ---------------------------------------------------------- code unpacking
// A lane's 32-bit plane-0 word holds two groups (parity 0 / 1) x 8 k-slots.
// k-slot s = 2v + h of group parity p sits at bit 16h + 2(4p + v).  The
// matrix-core operand wants slots (2v, 2v+1) in the low/high half of VGPR v,
// each as the bf16 value 128 + 16u: move the field to bits [5:4] of each half
// and or in 0x4300 (= 128.0).
template <int S>
__device__ __forceinline__ uint32_t shl_signed(uint32_t w) {
  if constexpr (S >= 0)
    return w << S;
  else
    return w >> (-S);
}

template <int F>
__device__ __forceinline__ uint32_t lo_field(uint32_t w0) {
  return shl_signed<4 - 2 * F>(w0) & 0x00300030u;
}
// bit 2 of a 3-bit level: plane-1 bit 16h + 4gb + v moved to bit 6 of each half
template <int HB>
__device__ __forceinline__ uint32_t hi_field(uint32_t w1) {
  return shl_signed<6 - HB>(w1) & 0x00400040u;
}

template <int P>
__device__ __forceinline__ u32x4 unpack2(uint32_t w) {
  u32x4 r;
  r[0] = lo_field<4 * P + 0>(w) | 0x43004300u;
  r[1] = lo_field<4 * P + 1>(w) | 0x43004300u;
  r[2] = lo_field<4 * P + 2>(w) | 0x43004300u;
  r[3] = lo_field<4 * P + 3>(w) | 0x43004300u;
  return r;
}

// 3-bit levels of group GB (0..3 inside the k-block): 128 + 16u, u <= 7.
template <int GB>
__device__ __forceinline__ u32x4 unpack3(uint32_t w0, uint32_t w1) {
  constexpr int P = GB & 1;
  u32x4 r;
  r[0] = lo_field<4 * P + 0>(w0) | hi_field<4 * GB + 0>(w1) | 0x43004300u;
  r[1] = lo_field<4 * P + 1>(w0) | hi_field<4 * GB + 1>(w1) | 0x43004300u;
  r[2] = lo_field<4 * P + 2>(w0) | hi_field<4 * GB + 2>(w1) | 0x43004300u;
  r[3] = lo_field<4 * P + 3>(w0) | hi_field<4 * GB + 3>(w1) | 0x43004300u;
  return r;
}

// exact level values (u - offset) as bf16, for the LDS-staged prefill operand
__device__ __forceinline__ uint32_t level_bf16(uint32_t u, float off) {
  return f32_to_bf16((float)u - off);
}

}  // namespace bqmoe
