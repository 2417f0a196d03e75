// Prefill kernels: grouped GEMMs over the permuted rows on the gfx950 matrix
// cores.  At thousands of tokens every expert sees hundreds of rows, so each
// expert's packed weights are a dense contraction (the "Xolotl" README, "What
// one PC can do", measures prefill over 6K-17K-token prompts).
//
// A block takes one tile of <= 64 rows of one expert (the tile list comes from
// the routing kernels) and one group of output columns, with 4 waves; each
// wave computes both 32-row halves of the tile against its own columns (gate
// and up: 32 columns of each; down: 64 columns) with 32x32x16 matrix-core ops.
// Per 128-wide k-block:
//   - the block stages the 64 rows of pre-scaled activations (x/16 or h/16)
//     and their 32-group sums in LDS with direct global->LDS loads
//     (double-buffered: k-block kb+1 lands while kb is used);
//   - each wave reads its packed tiles straight from global memory into
//     registers one k-block ahead: a lane's 8-byte code chunks are exactly its
//     B operand, so no LDS is needed for B; levels become bf16 values
//     base + 16u with one mask-and-or per pair;
//   - per 32-group: C = the correction term by a zero-padded op on the staged
//     sums, D = A*B + C by two 32x32x16 ops, acc += scale * D in fp32.
// Epilogues: gate/up -> h = bf16(SiLU(g) * u), stored as h/16 with the 32-group
// sums of h for the down projection; down -> y = bf16(acc).
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "moe_internal.h"

namespace bqmoe {

constexpr int kRows = kPrefillTileM;  // rows per tile (two 32-row matrix-core tiles)

// SiLU with the hardware exp2 and reciprocal (a few fp32 ulp; h is rounded
// to bf16 right after, whose unit is 2^16 times coarser)
__device__ __forceinline__ float silu_pf(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

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

// NMAT = 2: gate/up, wave w of column group c covers columns
//   [32 (4c + w), +32) of gate (column tile 0) and of up (column tile 1);
// NMAT = 1: down, wave w covers columns [64 (4c + w), +64) (two column tiles).
// Each wave computes both 32-row tiles of the block's 64 rows, so one 32x32
// output tile per (row tile, column tile): 4 accumulators of 16 values.
template <int NMAT, bool Q3A, bool Q3B, bool SAMEC>
__global__ __launch_bounds__(256, 2) void k_pf_gemm(
    const uint8_t* __restrict__ experts, size_t stride, const uint8_t* __restrict__ shared,
    ProjDesc pa, ProjDesc pb, const int32_t* __restrict__ tiles, const int32_t* __restrict__ ctrl,
    const int32_t* __restrict__ perm_tok, int Tk, int gather, const uint16_t* __restrict__ A,
    const uint16_t* __restrict__ Asum, int K, int N, float ca, float cb,
    uint16_t* __restrict__ out, uint16_t* __restrict__ out_sum, int ncol, Unpack2K uk) {
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
  const int tid = threadIdx.x, lane = tid & 63, l32 = lane & 31, hl = lane >> 5, r = lane & 15;
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
  // group sums, stored group-major in LDS ([group][row][16 B]: the rows a
  // matrix-core read touches are contiguous, free of bank conflicts); wave w
  // loads group w of the k-block, one row per lane
  const uint16_t* srow = Asum + ((size_t)sTok[lane] * G + (wave & 3)) * 8;

  // this wave's column tiles: projection and the n-tile holding this lane's column
  const int cw = col * 4 + wave;
  const uint8_t* const base0 = blob + pa.off;
  const uint8_t* const base1 = blob + pb.off;
  const size_t scl0 = pa.scales, scl1 = pb.scales, pl0 = pa.plane1, pl1 = pb.plane1;
  int ntl[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) ntl[ct] = (NMAT == 2 ? cw * 2 : cw * 4 + 2 * ct) + (l32 >> 4);

  const Unpack2R ur = {uk.m0, uk.m1, uk.m2, lane_copy(uk.b0), lane_copy(uk.b1), lane_copy(uk.b2)};
  // correction B operand: k-slots 0..7 (lanes 0..31) carry the constants
  const u32x4 bc0 = corr_b_operand(lane < 32, ca);
  const u32x4 bc1 = corr_b_operand(lane < 32, cb);

  f32x16 acc[2][2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rt][ct][i] = 0.f;

  // packed tiles of the k-block being used (c*) and of the next one (n*): per
  // column tile, the lane's two 8-B code chunks (k-slots 8(2h + lane/32) ..+7
  // of each group, h = 0, 1), its column's 4 group scales, and for 3-bit
  // levels the two level-bit-2 words
  u32x2 cw_[2][2], cs_[2], nw_[2][2], ns_[2];
  uint32_t ch_[2][2], nh_[2][2];

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

#define BQ_LOADB(KB_, W_, S_, H_)                                                              \
  {                                                                                            \
    _Pragma("unroll") for (int ct = 0; ct < 2; ++ct) {                                         \
      const bool sec = NMAT == 2 && ct == 1;                                                   \
      const uint8_t* bb = sec ? base1 : base0;                                                 \
      const size_t tile_ = (size_t)ntl[ct] * KB + (KB_);                                       \
      _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                          \
        const int chunk_ = 16 * (2 * h + hl) + r;                                              \
        W_[ct][h] = *reinterpret_cast<const u32x2*>(bb + tile_ * 512 + chunk_ * 8);            \
        H_[ct][h] = (sec ? Q3B : Q3A)                                                          \
                        ? *reinterpret_cast<const uint32_t*>(bb + (sec ? pl1 : pl0) +          \
                                                             tile_ * 256 + chunk_ * 4)         \
                        : 0u;                                                                  \
      }                                                                                        \
      S_[ct] = *reinterpret_cast<const u32x2*>(bb + (sec ? scl1 : scl0) + tile_ * 128 + r * 8); \
    }                                                                                          \
  }

  // k-block kb: wait for its activations (LDS) and tiles (registers), then
  // issue k-block kb+1 into the other buffer and register set, then compute
  BQ_ISSUE(0, 0)
  BQ_LOADB(0, cw_, cs_, ch_)
  for (int kb = 0; kb < KB; ++kb) {
    const int buf = kb & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // k-block kb is in LDS for every wave; buffer buf^1 is free
    if (kb + 1 < KB) {
      BQ_ISSUE(kb + 1, buf ^ 1)
      BQ_LOADB(kb + 1, nw_, ns_, nh_)
    }
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* sA = sbuf + buf * kBufBytes;
    const uint8_t* sS = sA + kRows * 256;

#define BQ_PF_GROUP(GB)                                                                         \
  {                                                                                             \
    /* the group's LDS reads first, so that their latency runs under the unpacking */          \
    u32x4 aa[2][2], av[2];                                                                      \
    _Pragma("unroll") for (int rt = 0; rt < 2; ++rt) {                                          \
      _Pragma("unroll") for (int h = 0; h < 2; ++h) aa[rt][h] =                                 \
          *reinterpret_cast<const u32x4*>(sA + (GB * 4 + 2 * h + hl) * kColBytes +             \
                                          (rt * 32 + l32) * 16);                                \
      /* lanes 32..63 meet zeros in the correction B operand: any value is fine */             \
      av[rt] = *reinterpret_cast<const u32x4*>(sS + GB * kColBytes + (rt * 32 + l32) * 16);    \
    }                                                                                           \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    u32x4 b[2][2];                                                                              \
    float sc[2];                                                                                \
    _Pragma("unroll") for (int ct = 0; ct < 2; ++ct) {                                          \
      const bool q3 = (NMAT == 2 && ct == 1) ? Q3B : Q3A;                                       \
      _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                           \
        const uint32_t word = (GB < 2) ? cw_[ct][h][0] : cw_[ct][h][1];                        \
        if (q3)                                                                                 \
          b[ct][h] = unpack3<GB>(word, ch_[ct][h], ur);                                         \
        else                                                                                    \
          b[ct][h] = unpack2_r<GB & 1>(word, ur);                                               \
      }                                                                                         \
      const uint32_t sbits = ((GB < 2) ? cs_[ct][0] : cs_[ct][1]) >> (16 * (GB & 1));           \
      sc[ct] = f16_to_f32(sbits & 0xFFFFu);                                                     \
      /* an fp32 register: plain FMAs below rather than mixed-precision ones */                 \
      asm volatile("" : "+v"(sc[ct]));                                                          \
    }                                                                                           \
    _Pragma("unroll") for (int rt = 0; rt < 2; ++rt) {                                          \
      const f32x16 zero = {};                                                                   \
      const f32x16 corr0 = mfma32x32(av[rt], bc0, zero);                                        \
      f32x16 corr1 = corr0;                                                                     \
      if constexpr (!SAMEC) corr1 = mfma32x32(av[rt], bc1, zero);                               \
      _Pragma("unroll") for (int ct = 0; ct < 2; ++ct) {                                        \
        f32x16 d = mfma32x32(aa[rt][0], b[ct][0], (NMAT == 2 && ct == 1) ? corr1 : corr0);      \
        d = mfma32x32(aa[rt][1], b[ct][1], d);                                                  \
        _Pragma("unroll") for (int i = 0; i < 16; ++i)                                          \
            acc[rt][ct][i] = fmaf(sc[ct], d[i], acc[rt][ct][i]);                                \
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
    for (int ct = 0; ct < 2; ++ct) {
      cs_[ct] = ns_[ct];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        cw_[ct][h] = nw_[ct][h];
        ch_[ct][h] = nh_[ct][h];
      }
    }
  }
#undef BQ_ISSUE
#undef BQ_LOADB

  // ------------------------------------------------------------ epilogues
  // acc[rt][ct][i] is row rt*32 + 8(i/4) + 4(lane/32) + i%4, column l32 of
  // column tile ct
  if constexpr (NMAT == 2) {
    // gate (tile 0) and up (tile 1) of the same 32 columns of I: one 32-group
    // of the down projection
    const int I = N;
    const float wgt = slot_weight(l32);
    // the (W, S) sums of row slot c = 16 rt + i end up in lane c of each
    // half, which stages them: one stage_sums per lane instead of per row
    float my_w = 0.f, my_s = 0.f;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = rt * 32 + 8 * (i >> 2) + 4 * hl + (i & 3);
        const float g = acc[rt][0][i], u = acc[rt][1][i];
        const float hf = bf16_to_f32(f32_to_bf16(silu_pf(g) * u));
        if (m < M) out[(size_t)(row0 + m) * I + cw * 32 + l32] = (uint16_t)f32_to_bf16(hf * 0.0625f);
        float hs_part = hf, hw_part = hf * wgt;
        // sum over the 32 lanes holding this row (columns 0..31)
#pragma unroll
        for (int o = 16; o > 0; o >>= 1) {
          hs_part += __shfl_xor(hs_part, o, 32);
          hw_part += __shfl_xor(hw_part, o, 32);
        }
        my_w = l32 == rt * 16 + i ? hw_part : my_w;
        my_s = l32 == rt * 16 + i ? hs_part : my_s;
      }
    }
    const int mrow = (l32 >> 4) * 32 + 8 * ((l32 & 15) >> 2) + 4 * hl + (l32 & 3);
    if (mrow < M)
      *reinterpret_cast<uint4*>(out_sum + ((size_t)(row0 + mrow) * (I / 32) + cw) * 8) =
          stage_sums(my_w, my_s);
  } else {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int m = rt * 32 + 8 * (i >> 2) + 4 * hl + (i & 3);
        if (m < M) {
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
            out[(size_t)(row0 + m) * N + cw * 64 + ct * 32 + l32] =
                (uint16_t)f32_to_bf16(acc[rt][ct][i]);
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

// The same combine for a few tokens (decode): block = (256 columns, token), 4
// columns per lane, so that T = 8 still spreads over 128 blocks; the token's
// row indices and weights are uniform over the block (scalar loads).  Same
// order of operations as k_pf_combine, so the same bits.
__global__ __launch_bounds__(64) void k_combine_few(const uint16_t* __restrict__ y, int T, int d,
                                                    int k, int n_shared,
                                                    const int32_t* __restrict__ inv_row,
                                                    const float* __restrict__ w,
                                                    const uint16_t* __restrict__ x, int residual,
                                                    uint16_t* __restrict__ out) {
  const int t = blockIdx.y, c = blockIdx.x * 256 + threadIdx.x * 4;
  if (c >= d) return;  // d % 128 == 0: a lane's 4 columns are all in or all out
  // the residual's load is issued first and converted last (x may be null
  // without the residual: then row t of y stands in for it, unused)
  const uint2 xv =
      *reinterpret_cast<const uint2*>((residual ? x : y) + (size_t)t * d + c);
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  bool first = true;
  // rows in batches of 8: the batch's indices first, then all of its loads
  for (int j0 = 0; j0 < k; j0 += 8) {
    int rr[8];
    float wt[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      const int j = min(j0 + jj, k - 1);
      rr[jj] = inv_row[(size_t)t * k + j];
      wt[jj] = w[(size_t)t * k + j];
    }
    // the weights' loads stay here, beside the indices' (the compiler would
    // otherwise sink each into the branch below, one wait apiece)
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) asm volatile("" : "+s"(wt[jj]));
    uint2 yv[8];
#pragma unroll
    for (int jj = 0; jj < 8; ++jj)
      yv[jj] = *reinterpret_cast<const uint2*>(y + (size_t)rr[jj] * d + c);
    if (first) {
      // a = x (or 0), then a = fma(w_j, y_j, a) for j = 0, 1, ...: the order of
      // k_pf_combine
      if (residual) {
        acc[0] = bf16_to_f32(xv.x & 0xFFFFu);
        acc[1] = bf16_to_f32(xv.x >> 16);
        acc[2] = bf16_to_f32(xv.y & 0xFFFFu);
        acc[3] = bf16_to_f32(xv.y >> 16);
      }
      first = false;
    }
#pragma unroll
    for (int jj = 0; jj < 8; ++jj) {
      if (j0 + jj < k) {
        acc[0] = fmaf(wt[jj], bf16_to_f32(yv[jj].x & 0xFFFFu), acc[0]);
        acc[1] = fmaf(wt[jj], bf16_to_f32(yv[jj].x >> 16), acc[1]);
        acc[2] = fmaf(wt[jj], bf16_to_f32(yv[jj].y & 0xFFFFu), acc[2]);
        acc[3] = fmaf(wt[jj], bf16_to_f32(yv[jj].y >> 16), acc[3]);
      }
    }
  }
  if (n_shared) {
    const uint2 yv = *reinterpret_cast<const uint2*>(y + (size_t)(T * k + t) * d + c);
    acc[0] += bf16_to_f32(yv.x & 0xFFFFu);
    acc[1] += bf16_to_f32(yv.x >> 16);
    acc[2] += bf16_to_f32(yv.y & 0xFFFFu);
    acc[3] += bf16_to_f32(yv.y >> 16);
  }
  uint2 o;
  o.x = f32_to_bf16(acc[0]) | (f32_to_bf16(acc[1]) << 16);
  o.y = f32_to_bf16(acc[2]) | (f32_to_bf16(acc[3]) << 16);
  *reinterpret_cast<uint2*>(out + (size_t)t * d + c) = o;
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
  hipLaunchKernelGGL((k_pf_gemm<2, A3, B3, SAMEC>), grid, dim3(256), 0, s, (const uint8_t*)L->experts,
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
  if (prefill_exact16(L) || prefill_x2(L)) {
    int rc = prefill_exact16(L) ? launch_prefill16(L, x, T, R, ws, P, stream, mask)
                                : launch_prefill_x2(L, x, T, R, ws, P, stream, mask);
    if (!rc && (mask & MOE_PREFILL_STAGE_COMBINE))
      rc = launch_combine((const uint16_t*)(ws + P.y), T, L->d, L->top_k, L->n_shared, R->inv_row,
                          R->topk_w, x, (flags & MOE_ADD_RESIDUAL) ? 1 : 0, out, stream);
    return rc;
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
    hipLaunchKernelGGL((k_pf_gemm<1, true, true, true>), g2, dim3(256), 0, s,
                       (const uint8_t*)L->experts, L->expert_stride, (const uint8_t*)L->shared, pdn,
                       pdn, tiles, ctrl, R->perm_tok, Tk, 0, hs, hsum, I, d, qtype_offset(L->q_down),
                       qtype_offset(L->q_down), y, (uint16_t*)nullptr, d / 256, kUnpack2);
  else
    hipLaunchKernelGGL((k_pf_gemm<1, false, false, true>), g2, dim3(256), 0, s,
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
  if (T <= 64) {
    hipLaunchKernelGGL(k_combine_few, dim3((unsigned)((d + 255) / 256), (unsigned)T), dim3(64), 0,
                       (hipStream_t)stream, y, T, d, k, n_shared, inv_row, w, x, residual, out);
    return (int)hipGetLastError();
  }
  const long n = (long)T * (d / 8);
  hipLaunchKernelGGL(k_pf_combine, dim3((unsigned)((n + 255) / 256)), dim3(256), 0,
                     (hipStream_t)stream, y, T, d, k, n_shared, inv_row, w, x, residual, out);
  return (int)hipGetLastError();
}

}  // namespace bqmoe
