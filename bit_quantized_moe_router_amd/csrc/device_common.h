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
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// round to nearest even (one v_cvt_pk_bf16_f32); NaN stays NaN
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
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
// 32x32x16 bf16 matrix-core op (gfx950): lane l supplies A[l%32][8(l/32)..+7]
// and B[8(l/32)..+7][l%32]; it receives D[8(i/4) + 4(l/32) + i%4][l%32],
// i = 0..15.  Measured on this chip at about 1.6 times the throughput of the
// 16x16x32 op.
typedef float f32x16 __attribute__((ext_vector_type(16)));
__device__ __forceinline__ f32x16 mfma32x32(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Correction term of one 32-group as a zero-padded 16x16x32 op (the same
// shape as the main op, which takes it as its C operand).  Lanes 0..15 hold
// their row's staged sums in k-slots 0..7 of A: (-W, -S) as two negated bf16
// triples and two zeros, where S = sum_k x_k and W = sum_k x_k * base_k / 16
// (see unpack2); lanes 0..15 hold the per-format constants in k-slots 0..7 of
// B, zeros elsewhere.  D[row][col] = -(b0 * W + b3 * S)[row] for every column.
__device__ __forceinline__ f32x4 mfma_corr(u32x4 a, u32x4 b) {
  return mfma32(a, b, f32x4{0.f, 0.f, 0.f, 0.f});
}

// bf16 bits of x split into hi + mid + lo (each an exact bf16; the sum is x to
// ~2^-24 relative), negated.
__device__ __forceinline__ void split3_neg(float s, uint32_t& a, uint32_t& b, uint32_t& c) {
  const uint32_t hi = f32_to_bf16(s);
  const float r1 = s - bf16_to_f32(hi);
  const uint32_t mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(mid);
  const uint32_t lo = f32_to_bf16(r2);
  a = hi ^ 0x8000u;
  b = mid ^ 0x8000u;
  c = lo ^ 0x8000u;
}

// Staged sums of one (row, 32-group): 8 bf16 = (-W, -S) triples + 2 zeros.
__device__ __forceinline__ uint4 stage_sums(float W, float S) {
  uint32_t w0, w1, w2, s0, s1, s2;
  split3_neg(W, w0, w1, w2);
  split3_neg(S, s0, s1, s2);
  uint4 v;
  v.x = (w0 & 0xFFFFu) | (w1 << 16);
  v.y = (w2 & 0xFFFFu) | (s0 << 16);
  v.z = (s1 & 0xFFFFu) | (s2 << 16);
  v.w = 0u;
  return v;
}

// The B operand of the correction op for a projection: every format (its
// levels sit on the same per-slot bases) subtracts W + offset * S.
__device__ __forceinline__ u32x4 corr_b_operand(bool lane_active, float off) {
  u32x4 b = {0u, 0u, 0u, 0u};
  if (lane_active) {
    const uint32_t one = 0x3F80u;
    const uint32_t c = f32_to_bf16(off);
    const uint32_t w = one;
    b[0] = w | (w << 16);
    b[1] = w | (c << 16);
    b[2] = c | (c << 16);
  }
  return b;
}

// Weight base_k / 16 of k-slot j (position inside its 32-group) in W.
__device__ __forceinline__ float slot_weight(int j) {
  const int v = (j & 7) >> 1;
  return v == 0 ? 128.0f : v == 1 ? 32.0f : 8.0f;
}

// ---------------------------------------------------------- code unpacking
// A lane's 32-bit plane-0 word holds two groups (parity 0 / 1) x 8 k-slots.
// k-slot s = 2v + h of group parity p sits at bit 16h + 2(4p + v).  The
// matrix-core operand wants slots (2v, 2v+1) in the low/high half of VGPR v.
// 2-bit levels become bf16 values base_v + 16u: the fields of v = 0, 1, 2 stay
// where they are (bits [1:0], [3:2], [5:4] of each half, after a shift by 8
// for parity 1) under the bases 2048 (0x4500), 512 (0x4400) and 128 (0x4300),
// whose unit in the last place is 16, 4 and 1; v = 3 is shifted down to bits
// [5:4] under base 128.  So one mask-and-or per pair of levels, plus two
// shifts per 8 levels.
template <int P>
__device__ __forceinline__ u32x4 unpack2(uint32_t w) {
  const uint32_t x = P ? (w >> 8) : w;
  u32x4 r;
  r[0] = (x & 0x00030003u) | 0x45004500u;
  r[1] = (x & 0x000C000Cu) | 0x44004400u;
  r[2] = (x & 0x00300030u) | 0x43004300u;
  r[3] = ((x >> 2) & 0x00300030u) | 0x43004300u;
  return r;
}

// exact level values (u - offset) as bf16, for the LDS-staged prefill operand
__device__ __forceinline__ uint32_t level_bf16(uint32_t u, float off) {
  return f32_to_bf16((float)u - off);
}

// Masks and bases of the 2-bit unpacking (see unpack2 in device_common.h),
// passed as kernel arguments.  The masks stay in scalar registers and the
// bases are copied once into vector registers (an identity lane move), so
// that each mask-and-or is one v_and_or_b32: with literal constants, or with
// both operands scalar, it would take two instructions (a VOP3 op here takes
// no literal and at most one scalar operand).
struct Unpack2K {
  uint32_t m0, m1, m2, b0, b1, b2;
};
static constexpr Unpack2K kUnpack2 = {0x00030003u, 0x000C000Cu, 0x00300030u,
                                  0x45004500u, 0x44004400u, 0x43004300u};

__device__ __forceinline__ uint32_t lane_copy(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xE4, 0xF, 0xF, true);  // quad_perm 0,1,2,3
}

struct Unpack2R {
  uint32_t m0, m1, m2, b0, b1, b2;  // b* in vector registers
};

template <int P>
__device__ __forceinline__ u32x4 unpack2_r(uint32_t w, const Unpack2R& c) {
  const uint32_t x = P ? (w >> 8) : w;
  u32x4 r;
  r[0] = (x & c.m0) | c.b0;
  r[1] = (x & c.m1) | c.b1;
  r[2] = (x & c.m2) | c.b2;
  r[3] = ((x >> 2) & c.m2) | c.b2;
  return r;
}

// 3-bit levels of group GB (0..3 inside the k-block) on the same bases as the
// 2-bit ones: the level's two low bits stay where unpack2_r leaves them and
// its bit 2 (from the plane-1 word w1) is inserted just above them, giving
// base_v + 16u with u <= 7 (bits [2v+2:2v] for v = 0, 1, 2; v = 3 is moved
// down to v = 2's place, as in unpack2_r).  Plane 1 holds the bit of pair v
// of group gb at 16h + 2v + 2 + (0, 1, 6, 7)[gb] for v <= 2 and at
// 16h + (0, 1, 14, 15)[gb] for v = 3, so one shift of w1 lines up pairs 0..2
// of a group and a second one pair 3: per 8 levels, four mask-and-ors, four
// bit-field inserts and up to four shifts.
__device__ __forceinline__ uint32_t bit_insert(uint32_t mask, uint32_t from, uint32_t into) {
  return (from & mask) | (into & ~mask);
}

template <int GB>
__device__ __forceinline__ u32x4 unpack3(uint32_t w0, uint32_t w1, const Unpack2R& c) {
  const uint32_t x = (GB & 1) ? (w0 >> 8) : w0;
  constexpr int SA = GB == 0 ? 0 : GB == 1 ? 1 : GB == 2 ? 6 : 7;
  const uint32_t ha = w1 >> SA;
  const uint32_t hb = GB == 0 ? (w1 << 6) : GB == 1 ? (w1 << 5) : GB == 2 ? (w1 >> 8) : (w1 >> 9);
  u32x4 r;
  r[0] = bit_insert(0x00040004u, ha, (x & c.m0) | c.b0);
  r[1] = bit_insert(0x00100010u, ha, (x & c.m1) | c.b1);
  r[2] = bit_insert(0x00400040u, ha, (x & c.m2) | c.b2);
  r[3] = bit_insert(0x00400040u, hb, ((x >> 2) & c.m2) | c.b2);
  return r;
}

}  // namespace bqmoe
