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

// Wave-wide maximum of a 32-bit value (uniform result): DPP steps inside each
// 16-lane row, then the four row maxima read as scalars.
// (bound_ctrl: a lane without a source would read 0, the identity of an
// unsigned maximum; these patterns have none, and the form lets the compiler
// fold the lane move into the max instruction.)
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = max(v, dpp_u32<0xB1>(v));   // quad_perm [1,0,3,2]
  v = max(v, dpp_u32<0x4E>(v));   // quad_perm [2,3,0,1]
  v = max(v, dpp_u32<0x141>(v));  // row_half_mirror
  v = max(v, dpp_u32<0x140>(v));  // row_mirror
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return max(max(a, b), max(c, d));
}

// Top-k of one token's E logits by one wave (lane l holds experts l + 64i),
// larger logit first and the lower index first among equal ones.  Each lane
// first sorts its PER entries by (key descending, index ascending); then k
// rounds each take the largest head key of the wave (a wave maximum), the
// lowest expert index among the lanes whose head holds it (one ballot, and
// only on a tie across lanes one more per entry slot), and pop that lane's
// head.  Lanes 0..k-1 return the ids in order and their softmax weights
// exp(l_j - l_0) / sum.  PER = entries per lane, a compile-time bound on E/64.
template <int PER>
__device__ void wave_topk(const float* __restrict__ L, int E, int k, int lane, int& my_id,
                          float& my_w) {
  const int per = (E + 63) / 64;
  uint32_t key[PER];
  float v[PER];
  int ix[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int e = lane + 64 * i;
    const bool present = i < per && e < E;
    v[i] = present ? L[present ? e : 0] : 0.f;
    key[i] = present ? order_key(v[i]) : 0u;
    ix[i] = i;
  }
  // odd-even transposition sort of the lane's entries
#pragma unroll
  for (int p = 0; p < PER; ++p) {
#pragma unroll
    for (int i = p & 1; i + 1 < PER; i += 2) {
      const bool sw = key[i + 1] > key[i] || (key[i + 1] == key[i] && ix[i + 1] < ix[i]);
      const uint32_t ka = key[i], kb = key[i + 1];
      const float va = v[i], vb = v[i + 1];
      const int ia = ix[i], ib = ix[i + 1];
      key[i] = sw ? kb : ka;
      key[i + 1] = sw ? ka : kb;
      v[i] = sw ? vb : va;
      v[i + 1] = sw ? va : vb;
      ix[i] = sw ? ib : ia;
      ix[i + 1] = sw ? ia : ib;
    }
  }
  float top = 0.f, my_v = 0.f;
  my_id = -1;
  for (int j = 0; j < k; ++j) {
    const uint32_t kmax = wave_max_u32(key[0]);
    const uint64_t m = __ballot(key[0] == kmax);
    int sel_lane, sel_i;
    if (__popcll(m) == 1) {
      sel_lane = __ffsll((unsigned long long)m) - 1;
      sel_i = __builtin_amdgcn_readlane(ix[0], sel_lane);
    } else {  // equal keys in several lanes: lowest entry slot, then lowest lane
      sel_lane = 0;
      sel_i = 0;
#pragma unroll
      for (int i = 0; i < PER; ++i) {
        const uint64_t mi = __ballot(key[0] == kmax && ix[0] == i);
        if (mi) {
          sel_lane = __ffsll((unsigned long long)mi) - 1;
          sel_i = i;
          break;
        }
      }
    }
    const float val = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v[0]), sel_lane));
    if (lane == sel_lane) {  // pop the head
#pragma unroll
      for (int t = 0; t + 1 < PER; ++t) {
        key[t] = key[t + 1];
        v[t] = v[t + 1];
        ix[t] = ix[t + 1];
      }
      key[PER - 1] = 0u;
    }
    if (j == 0) top = val;
    if (lane == j) {
      my_id = sel_lane + 64 * sel_i;
      my_v = val;
    }
  }
  const float ex = (lane < k) ? expf(my_v - top) : 0.f;
  const float den = wave_sum(ex);
  my_w = ex / den;
}

}  // namespace bqmoe
