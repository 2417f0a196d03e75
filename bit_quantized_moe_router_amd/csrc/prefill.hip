// Prefill kernels: grouped GEMMs over the permuted rows on the gfx950 matrix
// cores.  At thousands of tokens every expert sees hundreds of rows, so each
// expert's packed weights are a dense contraction (the "Xolotl" README, "What
// one PC can do", measures prefill over 6K-17K-token prompts).
//
// A block takes one tile of <= 128 rows of one expert (the tile list comes from
// the routing kernels) and 4 waves, each wave owning 4 (projection, 16-column
// n-tile) pairs for all 8 row tiles of the block.  Per 128-wide k-block:
//   - the block stages the 128 rows of pre-scaled activations (x/16 or h/16)
//     and their 32-group sums in LDS (double-buffered through registers);
//   - each wave reads its packed tiles straight from global memory: a tile's
//     lane chunk is exactly the lane's B operand, so no LDS is needed for B;
//     levels become the bf16 value 128 + 16u with a shift, a mask and an or;
//   - per 32-group: C = -(8 + offset) * sum(x) by a zero-padded 16x16x32 op,
//     D = A*B + C by 16x16x32 ops, acc += scale * D in fp32.
// Epilogues: gate/up -> h = bf16(SiLU(g) * u), stored as h/16 with the 32-group
// sums of h for the down projection; down -> y = bf16(acc).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "moe_internal.h"

namespace bqmoe {

constexpr int kRows = kPrefillTileM;  // rows per tile = 16 * RT
constexpr int RT = kRows / 16;        // 16-row tiles per wave

__device__ __forceinline__ float silu_pf(float g) { return g / (1.0f + expf(-g)); }

// Activation staging for prefill: xs = x/16 and the 32-group sums (W, S).
__global__ __launch_bounds__(256) void k_stage(const uint16_t* __restrict__ x, int T, int d,
                                               uint16_t* __restrict__ xs,
                                               uint16_t* __restrict__ xsum) {
  const int G = d / 32;
  const long pairs = (long)T * G;
  const int half = threadIdx.x >> 5, j = threadIdx.x & 31;
  for (long p = (long)blockIdx.x * 8 + half; p < pairs; p += (long)gridDim.x * 8) {
    const long t = p / G;
    const int g = (int)(p % G);
    const float xf = bf16_to_f32(x[t * d + g * 32 + j]);
    xs[t * d + g * 32 + j] = (uint16_t)f32_to_bf16(xf * 0.0625f);
    float sw = xf * slot_weight(j), s = xf;
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) {
      sw += __shfl_xor(sw, o, 32);
      s += __shfl_xor(s, o, 32);
    }
    if (j == 0) *reinterpret_cast<uint4*>(xsum + (t * G + g) * 8) = stage_sums(sw, s);
  }
}

template <bool Q3, int GB>
__device__ __forceinline__ u32x4 unpack_b(u32x2 w0, uint32_t w1) {
  const uint32_t word = (GB < 2) ? w0[0] : w0[1];
  if constexpr (Q3)
    return unpack3<GB>(word, w1);
  else
    return unpack2<GB & 1>(word);
}

typedef __attribute__((address_space(3))) void lds_void;

// NMAT = 2: gate and up (NTPW n-tiles of each per wave); NMAT = 1: down (NTPW n-tiles).
//
// LDS per buffer: 16 chunk columns x kRows rows x 16 B of activations (chunk c
// of row R at c*kRows*16 + R*16: the 16 rows a matrix-core read touches are 256
// contiguous bytes, and every address is one base register plus an immediate),
// then the group sums in the same column form (group g of row R at
// g*kRows*16 + R*16).  Both are filled
// with direct global->LDS loads (64 lanes x 16 B = 64 rows of one chunk column
// per instruction), which need no registers.
constexpr int kColBytes = kRows * 16;
constexpr int kBufBytes = kRows * 256 + kRows * 64;
constexpr int kDmaA = 16 * kRows / 64;   // activation DMA instructions per k-block
constexpr int kDmaS = 4;                  // group-sum DMA instructions per k-block (one per group)
static_assert(kRows == 64 && kDmaA % 4 == 0, "one row per lane in the group-sum loads");

template <int NMAT, int NTPW, bool Q3A, bool Q3B, bool SAMEC>
__global__ __launch_bounds__(256, 2) void k_pf_gemm(
    const uint8_t* __restrict__ experts, size_t stride, const uint8_t* __restrict__ shared,
    ProjDesc pa, ProjDesc pb, const int32_t* __restrict__ tiles, const int32_t* __restrict__ ctrl,
    const int32_t* __restrict__ perm_tok, int Tk, int gather, const uint16_t* __restrict__ A,
    const uint16_t* __restrict__ Asum, int K, int N, float ca, float cb,
    uint16_t* __restrict__ out, uint16_t* __restrict__ out_sum, int ncol, Unpack2K uk) {
  static_assert(NMAT * NTPW == 4, "four (projection, n-tile) streams per wave");
  __shared__ __attribute__((aligned(16))) uint8_t sbuf[2 * kBufBytes];
  __shared__ int sTok[kRows];

  // Work item = (row tile, column group), tile-major.  Blocks go to the 8 XCDs
  // round-robin; each XCD takes one contiguous chunk of the items, so the
  // column groups of a row tile run together on one XCD and read the tile's
  // activations from that XCD's L2 instead of from HBM once per column group.
  const int n_items = ctrl[0] * ncol;
  const int chunk = (n_items + 7) / 8;
  const int local = blockIdx.x / 8;
  const int item = (blockIdx.x % 8) * chunk + local;
  if (local >= chunk || item >= n_items) return;
  const int tile = item / ncol, col = item % ncol;
  const int32_t* tl = tiles + 4 * tile;
  const int e = tl[0], row0 = tl[1], M = tl[2];
  const uint8_t* blob = e >= 0 ? experts + (size_t)e * stride : shared;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KB = K / 128, G = K / 32;

  // source row of each tile row; padding rows repeat the first row (never stored)
  if (tid < kRows) {
    const int row = row0 + (tid < M ? tid : 0);
    sTok[tid] = gather ? (row < Tk ? perm_tok[row] : row - Tk) : row;
  }
  __syncthreads();

  // per-lane source rows of the direct-to-LDS loads: rows 64*h + lane
  const uint16_t* arow[kRows / 64];
#pragma unroll
  for (int h = 0; h < kRows / 64; ++h) arow[h] = A + (size_t)sTok[64 * h + lane] * K;
  // group sums, stored group-major in LDS ([group][row][16 B]: the 16 rows a
  // matrix-core read touches are contiguous, free of bank conflicts); wave w
  // loads group w of the k-block, one row per lane
  const uint16_t* srow = Asum + ((size_t)sTok[lane] * G + (wave & 3)) * 8;

  // this wave's streams: stream j -> projection (j / NTPW), n-tile nt0 + j % NTPW
  const int nt0 = (col * 4 + wave) * NTPW;
  const uint8_t* const base0 = blob + pa.off;
  const uint8_t* const base1 = blob + pb.off;
  const size_t scl0 = pa.scales, scl1 = pb.scales, pl0 = pa.plane1, pl1 = pb.plane1;

  const Unpack2R ur = {uk.m0, uk.m1, uk.m2, lane_copy(uk.b0), lane_copy(uk.b1), lane_copy(uk.b2)};
  const u32x4 bc0 = corr_b_operand(q == 0, Q3A, ca);
  const u32x4 bc1 = corr_b_operand(q == 0, Q3B, cb);

  f32x4 acc[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[rt][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // packed tiles of the k-block being used (c*) and of the next one, in flight (n*)
  u32x2 cw[4], cs[4], nw[4], ns[4];
  uint32_t ch[4], nh[4];

#define BQ_ISSUE(KB_, BUF_)                                                                    \
  {                                                                                            \
    uint8_t* dst = sbuf + (BUF_) * kBufBytes;                                                  \
    _Pragma("unroll") for (int i = 0; i < kDmaA / 4; ++i) {                                    \
      const int ci = wave * (kDmaA / 4) + i; /* column ci / RH, rows 64 * (ci % RH) .. */      \
      constexpr int RH = kRows / 64;                                                           \
      const uint16_t* src = arow[ci % RH] + (KB_) * 128 + (ci / RH) * 8;                       \
      __builtin_amdgcn_global_load_lds((const void*)src,                                       \
                                       (lds_void*)(dst + (ci / RH) * kColBytes + (ci % RH) * 1024), \
                                       16, 0, 0);                                              \
    }                                                                                          \
    if (wave < kDmaS)                                                                          \
      __builtin_amdgcn_global_load_lds((const void*)(srow + (KB_) * 32),                       \
                                       (lds_void*)(dst + kRows * 256 + wave * 1024), 16, 0, 0); \
  }

#define BQ_LOADB(KB_, S_)                                                                      \
  {                                                                                            \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                            \
      const bool first = (j / NTPW == 0);                                                      \
      const uint8_t* bb = first ? base0 : base1;                                               \
      const size_t tile = (size_t)(nt0 + (j % NTPW)) * KB + (KB_);                             \
      S_##w[j] = *reinterpret_cast<const u32x2*>(bb + tile * 512 + lane * 8);                  \
      S_##s[j] = *reinterpret_cast<const u32x2*>(bb + (first ? scl0 : scl1) + tile * 128 +     \
                                                 r * 8);                                       \
      const bool q3 = first ? Q3A : Q3B;                                                       \
      S_##h[j] = q3 ? *reinterpret_cast<const uint32_t*>(bb + (first ? pl0 : pl1) +            \
                                                         tile * 256 + lane * 4)                \
                    : 0u;                                                                      \
    }                                                                                          \
  }

  // k-block kb: wait for its activations (LDS) and tiles (registers), then
  // issue k-block kb+1 into the other buffer and register set, then compute
  BQ_ISSUE(0, 0)
  BQ_LOADB(0, c)
  for (int kb = 0; kb < KB; ++kb) {
    const int buf = kb & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // k-block kb is in LDS for every wave; buffer buf^1 is free
    if (kb + 1 < KB) {
      BQ_ISSUE(kb + 1, buf ^ 1)
      BQ_LOADB(kb + 1, n)
    }
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* sA = sbuf + buf * kBufBytes;
    const uint8_t* sS = sA + kRows * 256;

#define BQ_PF_GROUP(GB)                                                                         \
  {                                                                                             \
    /* the group's LDS reads first (all row tiles), so that their latency runs */              \
    /* under the unpacking below rather than in front of each matrix-core op */                \
    u32x4 av[RT], aa[RT];                                                                       \
    _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) {                                         \
      /* lanes q != 0 meet zeros in the correction B operand: no select needed */              \
      av[rt] = *reinterpret_cast<const u32x4*>(sS + GB * kColBytes + (rt * 16 + r) * 16);       \
      aa[rt] = *reinterpret_cast<const u32x4*>(sA + (GB * 4 + q) * kColBytes + (rt * 16 + r) * 16); \
    }                                                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    u32x4 b[4];                                                                                 \
    float sc[4];                                                                                \
    _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                             \
      const bool q3 = (j / NTPW == 0) ? Q3A : Q3B;                                              \
      if (q3)                                                                                   \
        b[j] = unpack_b<true, GB>(cw[j], ch[j]);                                                \
      else                                                                                      \
        b[j] = unpack2_r<GB & 1>((GB < 2) ? cw[j][0] : cw[j][1], ur);                           \
      const uint32_t sbits = ((GB < 2) ? cs[j][0] : cs[j][1]) >> (16 * (GB & 1));               \
      sc[j] = f16_to_f32(sbits & 0xFFFFu);                                                      \
      /* an fp32 register: plain FMAs below rather than mixed-precision ones */                 \
      asm volatile("" : "+v"(sc[j]));                                                           \
    }                                                                                           \
    _Pragma("unroll") for (int rt = 0; rt < RT; ++rt) {                                         \
      const f32x4 corr0 = mfma_corr(av[rt], bc0);                                               \
      f32x4 corr1 = corr0;                                                                      \
      if constexpr (!SAMEC) corr1 = mfma_corr(av[rt], bc1);                                     \
      _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                           \
        const f32x4 dd = mfma32(aa[rt], b[j], (j / NTPW == 0) ? corr0 : corr1);                 \
        acc[rt][j][0] = fmaf(sc[j], dd[0], acc[rt][j][0]);                                      \
        acc[rt][j][1] = fmaf(sc[j], dd[1], acc[rt][j][1]);                                      \
        acc[rt][j][2] = fmaf(sc[j], dd[2], acc[rt][j][2]);                                      \
        acc[rt][j][3] = fmaf(sc[j], dd[3], acc[rt][j][3]);                                      \
      }                                                                                         \
    }                                                                                           \
  }
    BQ_PF_GROUP(0)
    __builtin_amdgcn_sched_barrier(0);
    BQ_PF_GROUP(1)
    __builtin_amdgcn_sched_barrier(0);
    BQ_PF_GROUP(2)
    __builtin_amdgcn_sched_barrier(0);
    BQ_PF_GROUP(3)
#undef BQ_PF_GROUP
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      cw[j] = nw[j];
      cs[j] = ns[j];
      ch[j] = nh[j];
    }
  }
#undef BQ_ISSUE
#undef BQ_LOADB

  // ------------------------------------------------------------ epilogues
  if constexpr (NMAT == 2) {
    // streams 0..NTPW-1 are gate n-tiles, NTPW..2*NTPW-1 the matching up n-tiles;
    // the wave's 2*16 = 32 columns form one 32-group of the down projection
    const int I = N;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = rt * 16 + 4 * q + i;
        float hs_part = 0.f, hw_part = 0.f;
        const float wgt = slot_weight(r);  // column nt*16 + r is k-slot (16 jn + r) of its group
#pragma unroll
        for (int jn = 0; jn < NTPW; ++jn) {
          const float g = acc[rt][jn][i], u = acc[rt][NTPW + jn][i];
          const uint32_t hb = f32_to_bf16(silu_pf(g) * u);
          const float hf = bf16_to_f32(hb);
          hs_part += hf;
          hw_part += hf * wgt;
          if (m < M)
            out[(size_t)(row0 + m) * I + (nt0 + jn) * 16 + r] = (uint16_t)f32_to_bf16(hf * 0.0625f);
        }
        // sum over the 16 lanes holding this row (r = 0..15)
#pragma unroll
        for (int o = 8; o > 0; o >>= 1) {
          hs_part += __shfl_xor(hs_part, o, 16);
          hw_part += __shfl_xor(hw_part, o, 16);
        }
        if (m < M && r == 0) {
          const int g32 = (nt0 * 16) / 32;
          *reinterpret_cast<uint4*>(out_sum + ((size_t)(row0 + m) * (I / 32) + g32) * 8) =
              stage_sums(hw_part, hs_part);
        }
      }
    }
  } else {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = rt * 16 + 4 * q + i;
        if (m < M) {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            out[(size_t)(row0 + m) * N + (nt0 + j) * 16 + r] = (uint16_t)f32_to_bf16(acc[rt][j][i]);
        }
      }
  }
}

// out[t] = bf16( [x[t]] + sum_j w[t][j] * y[inv_row[t][j]] + [y[Tk + t]] ), fixed order
__global__ __launch_bounds__(256) void k_pf_combine(const uint16_t* __restrict__ y, int T, int d,
                                                    int k, int n_shared,
                                                    const int32_t* __restrict__ inv_row,
                                                    const float* __restrict__ w,
                                                    const uint16_t* __restrict__ x, int residual,
                                                    uint16_t* __restrict__ out) {
  const int chunks = d / 8;
  const long idx = (long)blockIdx.x * 256 + threadIdx.x;
  if (idx >= (long)T * chunks) return;
  const int t = (int)(idx / chunks), c = (int)(idx % chunks) * 8;
  float a[8];
  if (residual) {
    const uint4 xv = *reinterpret_cast<const uint4*>(x + (size_t)t * d + c);
    const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[2 * i] = bf16_to_f32(xw[i] & 0xFFFFu);
      a[2 * i + 1] = bf16_to_f32(xw[i] >> 16);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) a[i] = 0.f;
  }
  // rows in batches of 8: all of a batch's loads are in flight together
  for (int j0 = 0; j0 < k; j0 += 8) {
    uint4 yv[8];
    float wt[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = min(j0 + jj, k - 1);
      const int rr = inv_row[(size_t)t * k + j];
      wt[jj] = j0 + jj < k ? w[(size_t)t * k + j] : 0.f;
      yv[jj] = *reinterpret_cast<const uint4*>(y + (size_t)rr * d + c);
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (j0 + jj < k) {
        const uint32_t yw[4] = {yv[jj].x, yv[jj].y, yv[jj].z, yv[jj].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          a[2 * i] = fmaf(wt[jj], bf16_to_f32(yw[i] & 0xFFFFu), a[2 * i]);
          a[2 * i + 1] = fmaf(wt[jj], bf16_to_f32(yw[i] >> 16), a[2 * i + 1]);
        }
      }
    }
  }
  if (n_shared) {
    const uint4 yv = *reinterpret_cast<const uint4*>(y + (size_t)(T * k + t) * d + c);
    const uint32_t yw[4] = {yv.x, yv.y, yv.z, yv.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[2 * i] += bf16_to_f32(yw[i] & 0xFFFFu);
      a[2 * i + 1] += bf16_to_f32(yw[i] >> 16);
    }
  }
  uint4 o;
  o.x = f32_to_bf16(a[0]) | (f32_to_bf16(a[1]) << 16);
  o.y = f32_to_bf16(a[2]) | (f32_to_bf16(a[3]) << 16);
  o.z = f32_to_bf16(a[4]) | (f32_to_bf16(a[5]) << 16);
  o.w = f32_to_bf16(a[6]) | (f32_to_bf16(a[7]) << 16);
  *reinterpret_cast<uint4*>(out + (size_t)t * d + c) = o;
}

static ProjDesc proj_pf(const moe_layer* L, int m) {
  const int q = m == 0 ? L->q_gate : m == 1 ? L->q_up : L->q_down;
  const int K = m < 2 ? L->d : L->inter, N = m < 2 ? L->inter : L->d;
  const PackedLayout lg = packed_layout(L->q_gate, L->d, L->inter);
  const PackedLayout lu = packed_layout(L->q_up, L->d, L->inter);
  const PackedLayout me = packed_layout(q, K, N);
  ProjDesc p{};
  p.off = m == 0 ? 0 : m == 1 ? lg.total : lg.total + lu.total;
  p.plane1 = me.plane1;
  p.scales = me.scales;
  p.qtype = q;
  p.K = K;
  p.N = N;
  return p;
}

template <bool A3, bool B3, bool SAMEC>
static void launch_gu(dim3 grid, hipStream_t s, const moe_layer* L, ProjDesc pg, ProjDesc pu,
                      const int32_t* tiles, const int32_t* ctrl, const int32_t* perm_tok, int Tk,
                      const uint16_t* xs, const uint16_t* xsum, uint16_t* hs, uint16_t* hsum) {
  hipLaunchKernelGGL((k_pf_gemm<2, 2, A3, B3, SAMEC>), grid, dim3(256), 0, s, (const uint8_t*)L->experts,
                     L->expert_stride, (const uint8_t*)L->shared, pg, pu, tiles, ctrl, perm_tok, Tk,
                     1, xs, xsum, L->d, L->inter, qtype_offset(L->q_gate), qtype_offset(L->q_up), hs,
                     hsum, L->inter / 128, kUnpack2);
}

int launch_prefill(const moe_layer* L, const uint16_t* x, int T, uint32_t flags, moe_routing* R,
                   uint8_t* ws, const PrefillWs& P, uint16_t* out, void* stream, uint32_t mask) {
  if (mask & MOE_PREFILL_STAGE_ROUTE) {
    const int rc = launch_route_generic(L, x, T, flags, R, ws, P, stream);
    if (rc) return rc;
  }
  hipStream_t s = (hipStream_t)stream;
  const int k = L->top_k, d = L->d, I = L->inter;
  const int Tk = T * k;
  uint16_t* xs = (uint16_t*)(ws + P.xs);
  uint16_t* xsum = (uint16_t*)(ws + P.xsum);
  uint16_t* hs = (uint16_t*)(ws + P.h);
  uint16_t* hsum = (uint16_t*)(ws + P.hsum);
  uint16_t* y = (uint16_t*)(ws + P.y);
  const int32_t* tiles = (const int32_t*)(ws + P.tiles);
  const int32_t* ctrl = (const int32_t*)(ws + P.ctrl);
  if (mask & MOE_PREFILL_STAGE_STAGE_X) {
    const long pairs = (long)T * (d / 32);
    const int blocks = (int)min(4096L, (pairs + 7) / 8);
    hipLaunchKernelGGL(k_stage, dim3(blocks), dim3(256), 0, s, x, T, d, xs, xsum);
  }
  const ProjDesc pg = proj_pf(L, 0), pu = proj_pf(L, 1), pdn = proj_pf(L, 2);
  // grids: every (row tile, column group) item of the largest possible tile list
  const dim3 g1((unsigned)(((long)P.max_tiles * (I / 128) + 7) / 8 * 8));
  if (mask & MOE_PREFILL_STAGE_GATEUP) {
  const bool g3 = L->q_gate == MOE_Q_INT3, u3 = L->q_up == MOE_Q_INT3;
  const bool same = L->q_gate == L->q_up;  // same correction operand
  if (g3 && u3)
    launch_gu<true, true, true>(g1, s, L, pg, pu, tiles, ctrl, R->perm_tok, Tk, xs, xsum, hs, hsum);
  else if (g3)
    launch_gu<true, false, false>(g1, s, L, pg, pu, tiles, ctrl, R->perm_tok, Tk, xs, xsum, hs, hsum);
  else if (u3)
    launch_gu<false, true, false>(g1, s, L, pg, pu, tiles, ctrl, R->perm_tok, Tk, xs, xsum, hs, hsum);
  else if (same)
    launch_gu<false, false, true>(g1, s, L, pg, pu, tiles, ctrl, R->perm_tok, Tk, xs, xsum, hs, hsum);
  else
    launch_gu<false, false, false>(g1, s, L, pg, pu, tiles, ctrl, R->perm_tok, Tk, xs, xsum, hs, hsum);
  }
  const dim3 g2((unsigned)(((long)P.max_tiles * (d / 256) + 7) / 8 * 8));
  if (!(mask & MOE_PREFILL_STAGE_DOWN)) {
  } else if (L->q_down == MOE_Q_INT3)
    hipLaunchKernelGGL((k_pf_gemm<1, 4, true, true, true>), g2, dim3(256), 0, s,
                       (const uint8_t*)L->experts, L->expert_stride, (const uint8_t*)L->shared, pdn,
                       pdn, tiles, ctrl, R->perm_tok, Tk, 0, hs, hsum, I, d, qtype_offset(L->q_down),
                       qtype_offset(L->q_down), y, (uint16_t*)nullptr, d / 256, kUnpack2);
  else
    hipLaunchKernelGGL((k_pf_gemm<1, 4, false, false, true>), g2, dim3(256), 0, s,
                       (const uint8_t*)L->experts, L->expert_stride, (const uint8_t*)L->shared, pdn,
                       pdn, tiles, ctrl, R->perm_tok, Tk, 0, hs, hsum, I, d, qtype_offset(L->q_down),
                       qtype_offset(L->q_down), y, (uint16_t*)nullptr, d / 256, kUnpack2);
  if (mask & MOE_PREFILL_STAGE_COMBINE) {
    const int rc = launch_combine(y, T, d, k, L->n_shared, R->inv_row, R->topk_w, x,
                                  (flags & MOE_ADD_RESIDUAL) ? 1 : 0, out, stream);
    if (rc) return rc;
  }
  return (int)hipGetLastError();
}

int launch_combine(const uint16_t* y, int T, int d, int k, int n_shared, const int32_t* inv_row,
                   const float* w, const uint16_t* x, int residual, uint16_t* out, void* stream) {
  const long n = (long)T * (d / 8);
  hipLaunchKernelGGL(k_pf_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, y, T, d, k, n_shared, inv_row, w, x, residual, out);
  return (int)hipGetLastError();
}

}  // namespace bqmoe
