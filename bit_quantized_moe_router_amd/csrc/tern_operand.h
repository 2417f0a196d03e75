// The ternary fp16 operand shared by the prefill kernels on exact fp16 terms
// (the 4-wave ternary kernel and the 8-wave kernel's ternary variant).
#pragma once
#include "device_common.h"

namespace bqmoe {

// A lane's 32-bit code word holds two 32-groups' 8 levels each: group P
// (0 or 1) in bits 8P .. 8P+7 (levels k = 0, 2, 4, 6 of the lane's eight) and
// 16 + 8P .. (levels k = 1, 3, 5, 7), two bits per level, low bit first.
// fp16 pair D (levels 2D, 2D+1) of the operand is s * (u - 1) in both halves:
// a mask-and-or puts the level u into the mantissa of a power-of-two base
// where one step of the field is worth 1 (base 2^(10 - q) for a field at bit
// q), one packed add of -(base + 1) gives u - 1 exactly, and one packed
// multiply by the scale gives 0 or +-s, exact.  Group 1's fields sit at bits
// 8, 10, 12, 14: pair 0 stays in place under base 4, the others are shifted
// down by 8 onto group 0's positions.  The masks and offsets are kernel
// arguments (scalar registers); the bases are copied into vector registers
// once, so that each mask-and-or is one v_and_or_b32 (a VOP3 op takes one
// scalar operand and no literal).
struct TernK {
  uint32_t msk[4], base[4], off[4];  // per pair D at bit 2D: mask, base 2^(10-2D), -(base+1)
  uint32_t msk8, base8, off8;        // group 1's pair 0 at bit 8: mask, base 4, -5
};

template <int P>
__device__ __forceinline__ u32x4 build_tern(uint32_t word, uint32_t s2, const TernK& tk) {
  const uint32_t x = P ? (word >> 8) : word;
  u32x4 r;
#pragma unroll
  for (int D = 0; D < 4; ++D) {
    const bool in_place = P == 1 && D == 0;
    const uint32_t fv = in_place ? ((word & tk.msk8) | tk.base8) : ((x & tk.msk[D]) | tk.base[D]);
    const f16x2 c = __builtin_bit_cast(f16x2, fv) +
                    __builtin_bit_cast(f16x2, in_place ? tk.off8 : tk.off[D]);
    r[D] = __builtin_bit_cast(uint32_t, c * __builtin_bit_cast(f16x2, s2));
  }
  return r;
}

}  // namespace bqmoe
