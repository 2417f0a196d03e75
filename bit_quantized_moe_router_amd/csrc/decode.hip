// Decode kernels (1..8 tokens): stream each selected expert's packed bytes
// once for all of the tokens routed to it (the pages' "Latest" section of the
// "Xolotl" README describes decoding an expert once for all its tokens; its
// "Fast mode" section notes that decode speed is set by the expert bytes read
// per token).
//
// Work unit: (slot, column group) where a slot is one active expert (or the
// shared expert) with its M <= 16 rows.  A block's waves split the reduction
// dimension into contiguous k-block ranges, issue every load of their range up
// front, then run the 16x16x32 bf16 matrix-core op with
//   A = activations / 16 of the slot's rows (rows beyond M are zero),
//   B = packed levels turned into the bf16 value 128 + 16u by one shift, one
//       mask and one or per pair of levels (see device_common.h),
//   C = -(8 + offset) * (sum of the group's activations), produced by a
//       second 16x16x32 op (zero-padded) from the activation sums staged in
//       three bf16 parts,
// so D is exactly sum_k x * (u - offset) for one 32-group; it is scaled by the
// group's fp16 scale and accumulated in fp32.  Partial sums of the waves meet
// in LDS in a fixed order (deterministic, no floating-point atomics).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "moe_internal.h"

namespace bqmoe {

__device__ __forceinline__ uint32_t bf16_pair(float lo, float hi) {
  return f32_to_bf16(lo) | (f32_to_bf16(hi) << 16);
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// One 32-group step for one n-tile: D = A*B + C, acc += scale * D.
template <bool Q3, int GB>
__device__ __forceinline__ void group_step(f32x4& acc, u32x4 a, u32x2 w0, uint32_t w1, u32x2 sc,
                                           f32x4 corr) {
  const uint32_t word = (GB < 2) ? w0[0] : w0[1];
  u32x4 b;
  if constexpr (Q3)
    b = unpack3<GB>(word, w1);
  else
    b = unpack2<GB & 1>(word);
  const f32x4 dd = mfma32(a, b, corr);
  const uint32_t sbits = ((GB < 2) ? sc[0] : sc[1]) >> (16 * (GB & 1));
  const float s = f16_to_f32(sbits & 0xFFFFu);
  acc[0] = fmaf(s, dd[0], acc[0]);
  acc[1] = fmaf(s, dd[1], acc[1]);
  acc[2] = fmaf(s, dd[2], acc[2]);
  acc[3] = fmaf(s, dd[3], acc[3]);
}

// Staged activation sums -> split sum in bf16 triple, (hi, mid, lo) negated.
__device__ __forceinline__ uint2 split3_neg(float s) {
  const uint32_t hi = f32_to_bf16(s);
  const float r1 = s - bf16_to_f32(hi);
  const uint32_t mid = f32_to_bf16(r1);
  const float r2 = r1 - bf16_to_f32(mid);
  const uint32_t lo = f32_to_bf16(r2);
  uint2 v;
  v.x = ((hi ^ 0x8000u) & 0xFFFFu) | (((mid ^ 0x8000u) & 0xFFFFu) << 16);
  v.y = (lo ^ 0x8000u) & 0xFFFFu;
  return v;
}

// ------------------------------------------------------------ gate / up
// Block = (slot, 32 intermediate columns = 2 n-tiles) for both gate and up.
template <bool QG3, bool QU3, int KSPLIT, int MAXKB>
__global__ __launch_bounds__(64 * KSPLIT) void k_dec_gateup(
    const uint8_t* __restrict__ experts, size_t stride, const uint8_t* __restrict__ shared,
    ProjDesc pg, ProjDesc pu, const int32_t* __restrict__ slots,
    const int32_t* __restrict__ perm_tok, const uint16_t* __restrict__ xs,
    const uint16_t* __restrict__ xsum, int d, int I, int Tk, float cg, float cu,
    uint16_t* __restrict__ hs, uint16_t* __restrict__ hsum) {
  __shared__ float red[KSPLIT][16][64];
  __shared__ float hval[16][32];
  const int groups = I / 32;
  const int slot = blockIdx.x / groups, grp = blockIdx.x % groups;
  if (slot >= slots[0]) return;
  const int e = slots[1 + 3 * slot], row0 = slots[2 + 3 * slot], M = slots[3 + 3 * slot];
  const uint8_t* blob = e >= 0 ? experts + (size_t)e * stride : shared;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, q = lane >> 4, r = lane & 15;
  const int KB = d / 128;
  const int per = (KB + KSPLIT - 1) / KSPLIT;
  const int kb0 = min(KB, wave * per), kb1 = min(KB, kb0 + per);
  const bool tok_ok = r < M;
  const int row = row0 + r;
  const int tok = tok_ok ? (row < Tk ? perm_tok[row] : row - Tk) : 0;
  const uint16_t* xrow = xs + (size_t)tok * d;
  const uint16_t* srow = xsum + (size_t)tok * (d / 32) * 4;

  u32x2 bcg = {0u, 0u}, bcu = {0u, 0u};
  if (q == 0) {
    bcg[0] = bf16_pair(cg, cg);
    bcg[1] = f32_to_bf16(cg);
    bcu[0] = bf16_pair(cu, cu);
    bcu[1] = f32_to_bf16(cu);
  }
  f32x4 ag[2], au[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) ag[j] = au[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nt0 = grp * 2;
  const uint8_t* g0 = blob + pg.off;
  const uint8_t* u0 = blob + pu.off;

  for (int kbase = kb0; kbase < kb1; kbase += MAXKB) {
    u32x2 wg[MAXKB][2], wu[MAXKB][2], sg[MAXKB][2], su[MAXKB][2];
    uint32_t hg[MAXKB][2], hu[MAXKB][2];
    u32x4 ax[MAXKB][4];
    u32x2 ac[MAXKB][4];
#pragma unroll
    for (int i = 0; i < MAXKB; ++i) {
      const int kb = kbase + i;
      if (kb < kb1) {
#pragma unroll
        for (int nt = 0; nt < 2; ++nt) {
          const size_t tile = (size_t)(nt0 + nt) * KB + kb;
          wg[i][nt] = *reinterpret_cast<const u32x2*>(g0 + tile * 512 + lane * 8);
          wu[i][nt] = *reinterpret_cast<const u32x2*>(u0 + tile * 512 + lane * 8);
          if constexpr (QG3) hg[i][nt] = *reinterpret_cast<const uint32_t*>(g0 + pg.plane1 + tile * 256 + lane * 4);
          else hg[i][nt] = 0;
          if constexpr (QU3) hu[i][nt] = *reinterpret_cast<const uint32_t*>(u0 + pu.plane1 + tile * 256 + lane * 4);
          else hu[i][nt] = 0;
          sg[i][nt] = *reinterpret_cast<const u32x2*>(g0 + pg.scales + tile * 128 + r * 8);
          su[i][nt] = *reinterpret_cast<const u32x2*>(u0 + pu.scales + tile * 128 + r * 8);
        }
#pragma unroll
        for (int gb = 0; gb < 4; ++gb) {
          if (tok_ok) {
            ax[i][gb] = *reinterpret_cast<const u32x4*>(xrow + kb * 128 + gb * 32 + q * 8);
            ac[i][gb] = (q == 0) ? *reinterpret_cast<const u32x2*>(srow + (kb * 4 + gb) * 4)
                                 : u32x2{0u, 0u};
          } else {
            ax[i][gb] = u32x4{0u, 0u, 0u, 0u};
            ac[i][gb] = u32x2{0u, 0u};
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MAXKB; ++i) {
      if (kbase + i < kb1) {
#define BQ_GU_STEP(GB)                                                                \
  {                                                                                   \
    const f32x4 cgc = mfma_corr(ac[i][GB], bcg);                                      \
    const f32x4 cuc = (QG3 == QU3 && cg == cu) ? cgc : mfma_corr(ac[i][GB], bcu);     \
    group_step<QG3, GB>(ag[0], ax[i][GB], wg[i][0], hg[i][0], sg[i][0], cgc);          \
    group_step<QG3, GB>(ag[1], ax[i][GB], wg[i][1], hg[i][1], sg[i][1], cgc);          \
    group_step<QU3, GB>(au[0], ax[i][GB], wu[i][0], hu[i][0], su[i][0], cuc);          \
    group_step<QU3, GB>(au[1], ax[i][GB], wu[i][1], hu[i][1], su[i][1], cuc);          \
  }
        BQ_GU_STEP(0)
        BQ_GU_STEP(1)
        BQ_GU_STEP(2)
        BQ_GU_STEP(3)
#undef BQ_GU_STEP
      }
    }
  }
  // cross-wave reduction in a fixed order
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    red[wave][0 + i][lane] = ag[0][i];
    red[wave][4 + i][lane] = ag[1][i];
    red[wave][8 + i][lane] = au[0][i];
    red[wave][12 + i][lane] = au[1][i];
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < 2 * 4 * 64; idx += 64 * KSPLIT) {
    const int nt = idx >> 8, i = (idx >> 6) & 3, ln = idx & 63;
    const int t = 4 * (ln >> 4) + i;
    const int nn = nt * 16 + (ln & 15);
    float g = 0.f, u = 0.f;
    for (int w = 0; w < KSPLIT; ++w) {
      g += red[w][nt * 4 + i][ln];
      u += red[w][8 + nt * 4 + i][ln];
    }
    if (t < M) {
      const uint32_t hb = f32_to_bf16(silu_f(g) * u);
      const float hf = bf16_to_f32(hb);
      hs[(size_t)(row0 + t) * I + grp * 32 + nn] = (uint16_t)f32_to_bf16(hf * 0.0625f);
      hval[t][nn] = hf;
    }
  }
  __syncthreads();
  // 32-group sums of h for the down projection's correction term
  if (threadIdx.x < 16 * 32) {
    const int t = threadIdx.x >> 5, j = threadIdx.x & 31;
    float s = (t < M) ? hval[t][j] : 0.f;
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) s += __shfl_xor(s, o, 32);
    if (t < M && j == 0)
      *reinterpret_cast<uint2*>(hsum + ((size_t)(row0 + t) * (I / 32) + grp) * 4) = split3_neg(s);
  }
}

// ------------------------------------------------------- down + combine
// Block = (slot, 64 output columns = 4 n-tiles).  y is rounded to bf16 and
// stored; the last block to finish a column range (arrival counter) adds the
// weighted expert outputs of every token for that range in a fixed order.
template <bool QD3, int KSPLIT, int MAXKB>
__global__ __launch_bounds__(64 * KSPLIT) void k_dec_down(
    const uint8_t* __restrict__ experts, size_t stride, const uint8_t* __restrict__ shared,
    ProjDesc pd, const int32_t* __restrict__ slots, const uint16_t* __restrict__ hs,
    const uint16_t* __restrict__ hsum, int d, int I, int T, int k, int n_shared, float cd,
    uint16_t* __restrict__ y, uint32_t* __restrict__ counters, const int32_t* __restrict__ inv_row,
    const float* __restrict__ topk_w, const uint16_t* __restrict__ x, int residual,
    uint16_t* __restrict__ out) {
  constexpr int NTW = 4;
  __shared__ float red[KSPLIT][NTW * 4][64];
  __shared__ int s_last;
  const int blocks_per_slot = d / (16 * NTW);
  const int slot = blockIdx.x / blocks_per_slot, cb = blockIdx.x % blocks_per_slot;
  const int n_slots = slots[0];
  if (slot >= n_slots) return;
  const int e = slots[1 + 3 * slot], row0 = slots[2 + 3 * slot], M = slots[3 + 3 * slot];
  const uint8_t* blob = (e >= 0 ? experts + (size_t)e * stride : shared) + pd.off;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, q = lane >> 4, r = lane & 15;
  const int KB = I / 128;
  const int per = (KB + KSPLIT - 1) / KSPLIT;
  const int kb0 = min(KB, wave * per), kb1 = min(KB, kb0 + per);
  const bool tok_ok = r < M;
  const uint16_t* hrow = hs + (size_t)(row0 + (tok_ok ? r : 0)) * I;
  const uint16_t* srow = hsum + (size_t)(row0 + (tok_ok ? r : 0)) * (I / 32) * 4;
  u32x2 bc = {0u, 0u};
  if (q == 0) {
    bc[0] = bf16_pair(cd, cd);
    bc[1] = f32_to_bf16(cd);
  }
  f32x4 acc[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int nt0 = cb * NTW;
  for (int kbase = kb0; kbase < kb1; kbase += MAXKB) {
    u32x2 wd[MAXKB][NTW], sd[MAXKB][NTW];
    uint32_t hd[MAXKB][NTW];
    u32x4 ax[MAXKB][4];
    u32x2 ac[MAXKB][4];
#pragma unroll
    for (int i = 0; i < MAXKB; ++i) {
      const int kb = kbase + i;
      if (kb < kb1) {
#pragma unroll
        for (int j = 0; j < NTW; ++j) {
          const size_t tile = (size_t)(nt0 + j) * KB + kb;
          wd[i][j] = *reinterpret_cast<const u32x2*>(blob + tile * 512 + lane * 8);
          if constexpr (QD3) hd[i][j] = *reinterpret_cast<const uint32_t*>(blob + pd.plane1 + tile * 256 + lane * 4);
          else hd[i][j] = 0;
          sd[i][j] = *reinterpret_cast<const u32x2*>(blob + pd.scales + tile * 128 + r * 8);
        }
#pragma unroll
        for (int gb = 0; gb < 4; ++gb) {
          if (tok_ok) {
            ax[i][gb] = *reinterpret_cast<const u32x4*>(hrow + kb * 128 + gb * 32 + q * 8);
            ac[i][gb] = (q == 0) ? *reinterpret_cast<const u32x2*>(srow + (kb * 4 + gb) * 4)
                                 : u32x2{0u, 0u};
          } else {
            ax[i][gb] = u32x4{0u, 0u, 0u, 0u};
            ac[i][gb] = u32x2{0u, 0u};
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < MAXKB; ++i) {
      if (kbase + i < kb1) {
#define BQ_DN_STEP(GB)                                                        \
  {                                                                           \
    const f32x4 cc = mfma_corr(ac[i][GB], bc);                                \
    _Pragma("unroll") for (int j = 0; j < NTW; ++j)                           \
        group_step<QD3, GB>(acc[j], ax[i][GB], wd[i][j], hd[i][j], sd[i][j], cc); \
  }
        BQ_DN_STEP(0)
        BQ_DN_STEP(1)
        BQ_DN_STEP(2)
        BQ_DN_STEP(3)
#undef BQ_DN_STEP
      }
    }
  }
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) red[wave][j * 4 + i][lane] = acc[j][i];
  __syncthreads();
  for (int idx = threadIdx.x; idx < NTW * 4 * 64; idx += 64 * KSPLIT) {
    const int j = idx >> 8, i = (idx >> 6) & 3, ln = idx & 63;
    const int t = 4 * (ln >> 4) + i;
    float s = 0.f;
    for (int w = 0; w < KSPLIT; ++w) s += red[w][j * 4 + i][ln];
    if (t < M) y[(size_t)(row0 + t) * d + (nt0 + j) * 16 + (ln & 15)] = (uint16_t)f32_to_bf16(s);
  }
  // arrival: the last block of this column range combines
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t old = atomicAdd(&counters[cb], 1u);
    s_last = (old == (uint32_t)(n_slots - 1));
  }
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  const int cols = 16 * NTW;
  for (int idx = threadIdx.x; idx < T * cols; idx += 64 * KSPLIT) {
    const int t = idx / cols, c = cb * cols + idx % cols;
    float a = residual ? bf16_to_f32(x[(size_t)t * d + c]) : 0.f;
    for (int j = 0; j < k; ++j) {
      const int rr = inv_row[(size_t)t * k + j];
      a = fmaf(topk_w[(size_t)t * k + j], bf16_to_f32(__builtin_nontemporal_load(y + (size_t)rr * d + c)), a);
    }
    if (n_shared) a += bf16_to_f32(__builtin_nontemporal_load(y + (size_t)(T * k + t) * d + c));
    out[(size_t)t * d + c] = (uint16_t)f32_to_bf16(a);
  }
  if (threadIdx.x == 0) counters[cb] = 0u;
}

int launch_decode_route(const moe_layer* L, const uint16_t* x, int T, uint32_t flags,
                        moe_routing* R, uint8_t* ws, const DecodeWs& W, void* stream);

static ProjDesc proj(const moe_layer* L, int m) {
  const int q = m == 0 ? L->q_gate : m == 1 ? L->q_up : L->q_down;
  const int K = m < 2 ? L->d : L->inter, N = m < 2 ? L->inter : L->d;
  ProjDesc p{};
  const PackedLayout lg = packed_layout(L->q_gate, L->d, L->inter);
  const PackedLayout lu = packed_layout(L->q_up, L->d, L->inter);
  const PackedLayout me = packed_layout(q, K, N);
  p.off = m == 0 ? 0 : m == 1 ? lg.total : lg.total + lu.total;
  p.plane1 = me.plane1;
  p.scales = me.scales;
  p.qtype = q;
  p.K = K;
  p.N = N;
  return p;
}

template <bool QG3, bool QU3>
static void launch_gateup(const moe_layer* L, dim3 grid, hipStream_t s, ProjDesc pg, ProjDesc pu,
                          const int32_t* slots, const int32_t* perm_tok, const uint16_t* xs,
                          const uint16_t* xsum, int Tk, uint16_t* hs, uint16_t* hsum) {
  hipLaunchKernelGGL((k_dec_gateup<QG3, QU3, 8, 4>), grid, dim3(512), 0, s,
                     (const uint8_t*)L->experts, L->expert_stride, (const uint8_t*)L->shared, pg,
                     pu, slots, perm_tok, xs, xsum, L->d, L->inter, Tk, corr_const(L->q_gate),
                     corr_const(L->q_up), hs, hsum);
}

int launch_decode(const moe_layer* L, const uint16_t* x, int T, uint32_t flags, moe_routing* R,
                  uint8_t* ws, const DecodeWs& W, uint16_t* out, void* stream) {
  int rc = launch_decode_route(L, x, T, flags, R, ws, W, stream);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  const int k = L->top_k, d = L->d, I = L->inter;
  const int Tk = T * k;
  const ProjDesc pg = proj(L, 0), pu = proj(L, 1), pdn = proj(L, 2);
  const int32_t* slots = (const int32_t*)(ws + W.slots);
  uint16_t* xs = (uint16_t*)(ws + W.xs);
  uint16_t* xsum = (uint16_t*)(ws + W.xsum);
  uint16_t* hs = (uint16_t*)(ws + W.hs);
  uint16_t* hsum = (uint16_t*)(ws + W.hsum);
  dim3 g1(W.max_slots * (I / 32));
  const bool g3 = L->q_gate == MOE_Q_INT3, u3 = L->q_up == MOE_Q_INT3;
  if (g3 && u3)
    launch_gateup<true, true>(L, g1, s, pg, pu, slots, R->perm_tok, xs, xsum, Tk, hs, hsum);
  else if (g3)
    launch_gateup<true, false>(L, g1, s, pg, pu, slots, R->perm_tok, xs, xsum, Tk, hs, hsum);
  else if (u3)
    launch_gateup<false, true>(L, g1, s, pg, pu, slots, R->perm_tok, xs, xsum, Tk, hs, hsum);
  else
    launch_gateup<false, false>(L, g1, s, pg, pu, slots, R->perm_tok, xs, xsum, Tk, hs, hsum);
  dim3 g2(W.max_slots * (d / 64));
  const int residual = (flags & MOE_ADD_RESIDUAL) ? 1 : 0;
  uint16_t* y = (uint16_t*)(ws + W.y);
  uint32_t* counters = (uint32_t*)(ws + W.counters);
  if (L->q_down == MOE_Q_INT3)
    hipLaunchKernelGGL((k_dec_down<true, 8, 2>), g2, dim3(512), 0, s, (const uint8_t*)L->experts,
                       L->expert_stride, (const uint8_t*)L->shared, pdn, slots, hs, hsum, d, I, T,
                       k, L->n_shared, corr_const(L->q_down), y, counters, R->inv_row, R->topk_w,
                       x, residual, out);
  else
    hipLaunchKernelGGL((k_dec_down<false, 8, 2>), g2, dim3(512), 0, s, (const uint8_t*)L->experts,
                       L->expert_stride, (const uint8_t*)L->shared, pdn, slots, hs, hsum, d, I, T,
                       k, L->n_shared, corr_const(L->q_down), y, counters, R->inv_row, R->topk_w,
                       x, residual, out);
  return (int)hipGetLastError();
}

}  // namespace bqmoe
