// Top-k selection of one token's router logits by one wavefront, shared by
// the routing kernels and the single-token gate/up kernel (which selects its
// own experts), so that both make the same choice by construction.
#pragma once
#include <hip/hip_runtime.h>

#include <cstdint>

#include "device_common.h"

namespace bqmoe {

// Order-preserving integer key of a logit: a > b as floats iff key(a) >
// key(b), -0 and +0 share a key (they compare equal), and NaN gets the lowest
// key of all (1; key 0 marks "no entry"), so that ranking is a strict total
// order on (key, index) and every selected id is a valid, distinct expert
// whatever the inputs.
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 1u;  // NaN
  if ((u & 0x7FFFFFFFu) == 0u) u = 0u;              // -0 -> +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// One DPP lane move of a 32-bit value inside 16-lane rows.
// (bound_ctrl: a lane without a source would read 0, the identity of an
// unsigned maximum; these patterns have none, and the form lets the compiler
// fold the lane move into the max instruction.)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// Wave-wide maximum of a 32-bit value, left in every lane without scalar
// steps: the DPP steps leave each 16-lane row's maximum in all of its lanes,
// then the gfx950 lane swaps pair row 2m with row 2m+1 and the lower with the
// upper half.
__device__ __forceinline__ uint32_t wave_allmax_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));  // row_mirror
  const auto p = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = max((uint32_t)p[0], (uint32_t)p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return max((uint32_t)q[0], (uint32_t)q[1]);
}

// Sum over the 64 lanes by DPP lane moves and the gfx950 lane swaps (no LDS
// round trips): each step adds a lane's value to that of a partner lane in a
// disjoint pairing (xor 1, xor 2, the mirror within 8 lanes, within 16 lanes,
// then rows 2m/2m+1 and the two halves), so every lane ends with the same sum.
__device__ __forceinline__ float dpp_f32(float v, int which) {
  const int b = __float_as_int(v);
  switch (which) {
    case 0: return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, true));   // [1,0,3,2]
    case 1: return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, true));   // [2,3,0,1]
    case 2: return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x141, 0xF, 0xF, true));  // half mirror
    default: return __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x140, 0xF, 0xF, true)); // mirror
  }
}
__device__ __forceinline__ float wave_sum_lanes(float v) {
  v += dpp_f32(v, 0);
  v += dpp_f32(v, 1);
  v += dpp_f32(v, 2);
  v += dpp_f32(v, 3);
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
  const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// The logit back from its order key (key 1, NaN's, gives a NaN; -0 comes
// back as +0, which weighs the same).
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Top-k of one token's E logits by one wave (lane l holds experts l + 64i),
// larger logit first and the lower index first among equal ones.  Each lane
// first sorts its PER entries by (key descending, index ascending); then each
// of k rounds takes the largest head key of the wave, the lowest expert index
// among the heads holding it (a second maximum, of inverted indices) and pops
// that lane's head (one ballot instead of the second maximum when a single
// head holds the largest key).
// Lanes 0..k-1 return the ids in order and their softmax weights
// exp(l_j - l_0) / sum.  PER = entries per lane, a compile-time bound on E/64.
template <int PER>
__device__ void wave_topk(const float* __restrict__ L, int E, int k, int lane, int& my_id,
                          float& my_w) {
  const int per = (E + 63) / 64;
  uint32_t key[PER];
  int ix[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    const bool present = i < per && e < E;
    key[i] = present ? order_key(L[present ? e : 0]) : 0u;
    ix[i] = e;
  }
  // odd-even transposition sort of the lane's entries (indices ascend with i)
#pragma unroll
  for (int p = 0; p < PER; ++p) {
#pragma unroll
    for (int i = p & 1; i + 1 < PER; i += 2) {
      const bool sw = key[i + 1] > key[i] || (key[i + 1] == key[i] && ix[i + 1] < ix[i]);
      const uint32_t ka = key[i], kb = key[i + 1];
      const int ia = ix[i], ib = ix[i + 1];
      key[i] = sw ? kb : ka;
      key[i + 1] = sw ? ka : kb;
      ix[i] = sw ? ib : ia;
      ix[i + 1] = sw ? ia : ib;
    }
  }
  uint32_t top = 0u, my_key = 0u;
  my_id = -1;
  for (int j = 0; j < k; ++j) {
    const uint32_t kmax = wave_allmax_u32(key[0]);
    // The winner is the lowest expert index among the heads equal to kmax.
    // When one lane's head holds kmax (the usual case) that head is it: a
    // lane's entries are sorted, and every other head, hence every other
    // entry, is smaller.  Otherwise a second maximum, of inverted indices,
    // settles the tie (the branch is uniform over the wave).
    const uint64_t at_max = __ballot(key[0] == kmax);
    uint32_t win;
    if (__popcll(at_max) == 1)
      win = (uint32_t)__builtin_amdgcn_readlane(ix[0], (int)__ffsll((unsigned long long)at_max) - 1);
    else
      win = ~wave_allmax_u32(key[0] == kmax ? ~(uint32_t)ix[0] : 0u);
    const bool pop = (uint32_t)ix[0] == win;  // the winning lane pops its head
#pragma unroll
    for (int t = 0; t + 1 < PER; ++t) {
      key[t] = pop ? key[t + 1] : key[t];
      ix[t] = pop ? ix[t + 1] : ix[t];
    }
    key[PER - 1] = pop ? 0u : key[PER - 1];
    top = j == 0 ? kmax : top;
    my_key = lane == j ? kmax : my_key;
    my_id = lane == j ? (int)win : my_id;
  }
  const float ex = (lane < k) ? expf(key_value(my_key) - key_value(top)) : 0.f;
  const float den = wave_sum_lanes(ex);
  my_w = ex / den;
}

}  // namespace bqmoe
