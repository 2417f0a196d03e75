// Prefill on exact fp16 terms, for layers whose three projections hold
// ternary codes (the code families of the "Xolotl" README's "Quick start";
// the value of a code is scale * (u - offset), see include/moe.h).
//
// The group scale goes into the matrix-core operand instead of a per-group
// fp32 multiply of the partial sums: a ternary weight s * (u - 1) is 0 or
// +-s, exact in fp16.  The activations are fp16 copies of the bf16 rows
// scaled by a power of two per row (exact in fp16's range; the epilogue
// undoes the scale).  Each product is then exact and the matrix core
// accumulates the whole of K in fp32: no correction term and no per-group
// FMA, so the vector ALU only builds the operands.  A wave covers 128 rows
// (four 32-row tiles) of its columns, so one operand build feeds four
// matrix-core ops.  (2-bit codes split the same way into two exact terms,
// +-s and +-s/2, which doubles the matrix-core work; measured slower than
// the bf16-operand kernel, so they stay there.)
//
// A block takes one 128-row tile of one expert (tiles of this height come
// from the routing's tile list for such layers) and one group of output
// columns, with 4 waves:
//   gate/up: wave w covers columns [32 (4c + w), +32) of gate and of up;
//   down:    wave w covers columns [64 (4c + w), +64) (two column tiles).
// Two blocks share a CU.  Per 128-wide k-block the block stages the 128
// rows' fp16 activations in LDS with direct-to-LDS buffer loads
// (double-buffered), and each wave reads its packed tiles straight into
// registers one k-block ahead.
//
// Layers whose inter is a multiple of 256 and d of 512 run their GEMMs on
// the 8-wave kernel of the 2-bit path instead (k_pfx<NMAT, true> in
// prefill2x.hip: one block per CU, 512 output columns per staged tile, a
// three-stage ring whose waits leave the next step's loads in flight), with
// the same operand build; this kernel serves the other shapes.  (An 8-wave
// version of this kernel's own double-buffered loop was 11 % slower than two
// 4-wave blocks: there the blocks' barriers, not the activation traffic, set
// the time.)
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "tern_operand.h"
#include "moe_internal.h"

namespace bqmoe {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRows16 = 128;                  // rows per tile
constexpr int kBuf16 = kRows16 * 256;         // one k-block of activations
constexpr int kDma16 = 16 * kRows16 / 64;     // direct loads per k-block (64 lanes x 16 B each)
constexpr int kW16 = 4;                       // waves per block

__device__ __forceinline__ f32x16 mfma_f16(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// SiLU with the hardware exp2 and reciprocal (h is rounded to bf16 right after)
__device__ __forceinline__ float silu16(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

// ------------------------------------------------------------------ staging
// One wave per row of bf16 values: e = (exponent of max|v|) - 14, kept in
// [-100, 114] so that 2^e and 2^-e are normal floats; every |v| * 2^-e is then
// below 2^15 and, unless the row's maximum is below 2^-86, its maximum is at
// least 2^14.  dst = fp16(v * 2^-e) (exact for the row's values down to 2^-17
// of its maximum, rounded to nearest below), scale = 2^e.  src and dst may be
// the same rows (each lane rewrites what it read).
__global__ __launch_bounds__(256) void k_stage16(const uint16_t* src, int rows, int K,
                                                 uint16_t* dst, float* __restrict__ scale) {
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (row >= rows) return;
  const uint16_t* s = src + (size_t)row * K;
  uint16_t* d = dst + (size_t)row * K;
  uint32_t m = 0;
  for (int i = lane * 8; i < K; i += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(s + i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) m = max(m, max(w[j] & 0x7FFFu, (w[j] >> 16) & 0x7FFFu));
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) m = max(m, (uint32_t)__shfl_xor((int)m, o));
  const int e = min(114, max(-100, (int)(m >> 7) - 127 - 14));
  const float f = __uint_as_float((uint32_t)(127 - e) << 23);  // 2^-e
  for (int i = lane * 8; i < K; i += 512) {
    const uint4 v = *reinterpret_cast<const uint4*>(s + i);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const _Float16 lo = (_Float16)(bf16_to_f32(w[j] & 0xFFFFu) * f);
      const _Float16 hi = (_Float16)(bf16_to_f32(w[j] >> 16) * f);
      o[j] = (uint32_t)__builtin_bit_cast(uint16_t, lo) |
             ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
    }
    *reinterpret_cast<uint4*>(d + i) = make_uint4(o[0], o[1], o[2], o[3]);
  }
  if (lane == 0) scale[row] = __uint_as_float((uint32_t)(127 + e) << 23);
}

// ------------------------------------------------------------- grouped GEMM
// NMAT = 2: gate (column tile 0) and up (column tile 1); NMAT = 1: down (two
// column tiles).  A: fp16 rows (gather: tile row -> token through perm_tok),
// rscale: 2^e of each source row.
template <int NMAT>
__global__ __launch_bounds__(64 * kW16, 2) void k_pf16(
    const uint8_t* __restrict__ experts, size_t stride, const uint8_t* __restrict__ shared,
    ProjDesc pa, ProjDesc pb, const int32_t* __restrict__ tiles, const int32_t* __restrict__ ctrl,
    const int32_t* __restrict__ perm_tok, int Tk, int gather, const uint16_t* __restrict__ A,
    const float* __restrict__ rscale, int K, int N, uint16_t* __restrict__ out, int ncol,
    TernK tk) {
  __shared__ __attribute__((aligned(16))) uint8_t sbuf[2 * kBuf16];
  __shared__ int sTok[kRows16];
  __shared__ float sScale[kRows16];

  // work item = (row tile, column group), tile-major; each XCD takes one
  // contiguous chunk of the items (blocks go to the 8 XCDs round-robin), so
  // the column groups of a row tile share its activations in one L2
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
  const int KB = K / 128;

  // source row of each tile row; padding rows repeat the first row (never stored)
  if (tid < kRows16) {
    const int row = row0 + (tid < M ? tid : 0);
    const int src = gather ? (row < Tk ? perm_tok[row] : row - Tk) : row;
    sTok[tid] = src;
    sScale[tid] = rscale[src];
  }
  __syncthreads();
  // LDS, per buffer: row R at R * 256, its 16-byte chunk c (8 k) in slot
  // c ^ (R % 16).  A direct-to-LDS load writes 16 bytes per lane at
  // consecutive slots, so 16 lanes fill one row's 256 bytes from 2 cache
  // lines (with one row per lane, a load would touch 64 lines); the swizzle
  // keeps the matrix-core reads (16 rows, one chunk) free of bank conflicts.
  // Wave w loads rows 32w .. 32w + 31, four per load, with byte offsets into
  // A from the buffer resource rA (the host bounds A below 4 GiB).
  static_assert(kDma16 == 8 * kW16, "eight loads of 4 rows per wave");
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)A, 0, -1, 0x00020000);
  uint32_t aoffs[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int R = 32 * wave + 4 * i + (lane >> 4);
    aoffs[i] = (uint32_t)sTok[R] * (uint32_t)(2 * K) + (((lane & 15) ^ (R & 15)) << 4);
  }
  // matrix-core reads: chunk c = 4 GB + 2h + hl of row rt * 32 + l32 at
  // l32 * 256 + (((4 GB + 2h) ^ ya) << 4) + rt * 8192; the lane's part la16
  // (the XOR term occupies bits 4..7, which no other term touches, so a
  // k-block's base takes it once and each read XORs in its chunk)
  const uint32_t la16 = (uint32_t)(l32 * 256) | ((uint32_t)(hl ^ (l32 & 15)) << 4);

  TernK tv = tk;
#pragma unroll
  for (int D = 0; D < 4; ++D) tv.base[D] = lane_copy(tk.base[D]);
  tv.base8 = lane_copy(tk.base8);

  // packed tiles, one buffer over the expert: the lane's two code chunks of
  // column tile ct and k-half h at wu[ct] + 256 h + wl, its column's four
  // scales at su[ct] + sl, plus 512 (resp. 128) per k-block; wu, su are the
  // same for the whole wave (scalar offsets), wl, sl the lane's
  const int cw = col * kW16 + wave;
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc((void*)blob, 0, -1, 0x00020000);
  const uint32_t wl = (uint32_t)((l32 >> 4) * KB * 512 + (16 * hl + r) * 8);
  const uint32_t sl = (uint32_t)((l32 >> 4) * KB * 128 + r * 8);
  uint32_t wu[2], su[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const bool sec = NMAT == 2 && ct == 1;
    const uint32_t ntl = (uint32_t)(NMAT == 2 ? cw * 2 : cw * 4 + 2 * ct);
    wu[ct] = (uint32_t)(sec ? pb.off : pa.off) + ntl * KB * 512;
    su[ct] = (uint32_t)(sec ? pb.off + pb.scales : pa.off + pa.scales) + ntl * KB * 128;
  }

  f32x16 acc[4][2];
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rt][ct][i] = 0.f;

  // packed tiles of the k-block in use (c*) and of the next one (n*): per
  // column tile the lane's two 8-B code chunks and its column's 4 scales
  u32x2 cw_[2][2], cs_[2], nw_[2][2], ns_[2];

#define BQ16_ISSUE(KB_, BUF_)                                                                  \
  {                                                                                            \
    _Pragma("unroll") for (int i = 0; i < 8; ++i)                                              \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                \
          rA, (lds_void*)(sbuf + (BUF_) * kBuf16 + (8 * wave + i) * 1024), 16, aoffs[i],       \
          (KB_) * 256, 0, 0);                                                                  \
  }
#define BQ16_LOADB(KB_, W_, S_)                                                                \
  {                                                                                            \
    _Pragma("unroll") for (int ct = 0; ct < 2; ++ct) {                                         \
      _Pragma("unroll") for (int h = 0; h < 2; ++h) W_[ct][h] =                                \
          __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(                      \
                                        rB, (int)wl, (int)(wu[ct] + 256 * h + (KB_) * 512), 0)); \
      S_[ct] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(                \
                                              rB, (int)sl, (int)(su[ct] + (KB_) * 128), 0));   \
    }                                                                                          \
  }

  BQ16_ISSUE(0, 0)
  BQ16_LOADB(0, cw_, cs_)
  for (int kb = 0; kb < KB; ++kb) {
    const int buf = kb & 1;
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();  // k-block kb is in LDS for every wave; buffer buf^1 is free
    if (kb + 1 < KB) {
      BQ16_ISSUE(kb + 1, buf ^ 1)
      BQ16_LOADB(kb + 1, nw_, ns_)
    }
    __builtin_amdgcn_sched_barrier(0);
    const uint32_t aS = la16 + (uint32_t)(buf * kBuf16);

    // A fragments of group GB (8 reads of 16 B per lane)
#define BQ16_READA(DST, GB)                                                                     \
  _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                               \
    const uint8_t* pa_ = sbuf + (aS ^ ((4u * (GB) + 2u * h) << 4));                              \
    _Pragma("unroll") for (int rt = 0; rt < 4; ++rt) DST[rt][h] =                               \
        *reinterpret_cast<const u32x4*>(pa_ + rt * 8192);                                       \
  }
    // group GB on the fragments in aa; the next group's are read first, so
    // that their LDS latency runs under this group's matrix-core ops
#define BQ16_GROUP(GB)                                                                          \
  {                                                                                             \
    if constexpr ((GB) < 3) { BQ16_READA(an, (GB) + 1) }                                        \
    __builtin_amdgcn_sched_barrier(0);                                                          \
    uint32_t s2[2];                                                                             \
    _Pragma("unroll") for (int ct = 0; ct < 2; ++ct) {                                          \
      /* fp16 scale of (column l32, group GB), in both halves */                                \
      const uint32_t sh = ((((GB) < 2) ? cs_[ct][0] : cs_[ct][1]) >> (16 * ((GB) & 1))) & 0xFFFFu; \
      s2[ct] = sh | (sh << 16);                                                                 \
    }                                                                                           \
    /* per k-half: both column tiles' operands, then 8 independent ops */                       \
    _Pragma("unroll") for (int h = 0; h < 2; ++h) {                                             \
      u32x4 t[2];                                                                               \
      _Pragma("unroll") for (int ct = 0; ct < 2; ++ct)                                          \
          t[ct] = build_tern<(GB) & 1>(((GB) < 2) ? cw_[ct][h][0] : cw_[ct][h][1], s2[ct], tv); \
      _Pragma("unroll") for (int rt = 0; rt < 4; ++rt)                                          \
          _Pragma("unroll") for (int ct = 0; ct < 2; ++ct)                                      \
              acc[rt][ct] = mfma_f16(aa[rt][h], t[ct], acc[rt][ct]);                            \
    }                                                                                           \
    if constexpr ((GB) < 3) {                                                                   \
      _Pragma("unroll") for (int rt = 0; rt < 4; ++rt)                                          \
          _Pragma("unroll") for (int h = 0; h < 2; ++h) aa[rt][h] = an[rt][h];                  \
    }                                                                                           \
  }
    u32x4 aa[4][2], an[4][2];
    BQ16_READA(aa, 0)
    BQ16_GROUP(0)
    BQ16_GROUP(1)
    BQ16_GROUP(2)
    BQ16_GROUP(3)
#undef BQ16_GROUP
#undef BQ16_READA
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      cs_[ct] = ns_[ct];
#pragma unroll
      for (int h = 0; h < 2; ++h) cw_[ct][h] = nw_[ct][h];
    }
  }
#undef BQ16_ISSUE
#undef BQ16_LOADB

  // acc[rt][ct][i] is row rt*32 + 8(i/4) + 4(lane/32) + i%4, column l32 of
  // column tile ct; the row's 2^e undoes the activation scale
#pragma unroll
  for (int rt = 0; rt < 4; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = rt * 32 + 8 * (i >> 2) + 4 * hl + (i & 3);
      if (m < M) {
        const float sc = sScale[m];
        if constexpr (NMAT == 2) {
          // gate and up of the same column of I: h = bf16(SiLU(g) * u)
          const float g = acc[rt][0][i] * sc, u = acc[rt][1][i] * sc;
          out[(size_t)(row0 + m) * N + cw * 32 + l32] = (uint16_t)f32_to_bf16(silu16(g) * u);
        } else {
#pragma unroll
          for (int ct = 0; ct < 2; ++ct)
            out[(size_t)(row0 + m) * N + cw * 64 + ct * 32 + l32] =
                (uint16_t)f32_to_bf16(acc[rt][ct][i] * sc);
        }
      }
    }
}

// --------------------------------------------------------------- launchers
bool prefill_exact16(const moe_layer* L) {
  return L->q_gate == MOE_Q_TERNARY && L->q_up == MOE_Q_TERNARY && L->q_down == MOE_Q_TERNARY &&
         L->inter % (32 * kW16) == 0 && L->d % (64 * kW16) == 0;
}

int prefill_tile_rows(const moe_layer* L) {
  if (prefill_x2(L)) return prefill_x2_tile_rows();
  return prefill_exact16(L) ? kRows16 : kPrefillTileM;
}

static ProjDesc proj16(const moe_layer* L, int m) {
  const int K = m < 2 ? L->d : L->inter, N = m < 2 ? L->inter : L->d;
  const PackedLayout lt = packed_layout(MOE_Q_TERNARY, L->d, L->inter);
  const PackedLayout me = packed_layout(MOE_Q_TERNARY, K, N);
  ProjDesc p{};
  p.off = (size_t)m * lt.total;
  p.plane1 = me.plane1;
  p.scales = me.scales;
  p.qtype = MOE_Q_TERNARY;
  p.K = K;
  p.N = N;
  return p;
}

TernK tern_constants() {
  // per pair D (field at bit q = 2D): the field's mask, the fp16 base
  // 2^(10 - q) and -(base + 1), in both halves: 1024, 256, 64, 16 and -1025,
  // -257, -65, -17; group 1's pair 0 at bit 8: base 4, -5
  TernK k{};
  const uint32_t m[4] = {0x00030003u, 0x000C000Cu, 0x00300030u, 0x00C000C0u};
  const uint32_t b[4] = {0x64006400u, 0x5C005C00u, 0x54005400u, 0x4C004C00u};
  const uint32_t o[4] = {0xE401E401u, 0xDC04DC04u, 0xD410D410u, 0xCC40CC40u};
  for (int D = 0; D < 4; ++D) {
    k.msk[D] = m[D];
    k.base[D] = b[D];
    k.off[D] = o[D];
  }
  k.msk8 = 0x03000300u;
  k.base8 = 0x44004400u;
  k.off8 = 0xC500C500u;
  return k;
}

// The workspace areas of the bf16-operand path hold, here: xs the fp16 rows
// of x, xsum their scales; h the bf16 h and then (by the end of the gate/up
// stage) its fp16 rows, hsum their scales.
int launch_prefill16(const moe_layer* L, const uint16_t* x, int T, moe_routing* R, uint8_t* ws,
                     const PrefillWs& P, void* stream, uint32_t mask) {
  hipStream_t s = (hipStream_t)stream;
  const int k = L->top_k, d = L->d, I = L->inter;
  const int Tk = T * k;
  const int rows = Tk + (L->n_shared ? T : 0);
  uint16_t* xs = (uint16_t*)(ws + P.xs);
  float* xscale = (float*)(ws + P.xsum);
  uint16_t* hs = (uint16_t*)(ws + P.h);
  float* hscale = (float*)(ws + P.hsum);
  uint16_t* y = (uint16_t*)(ws + P.y);
  const int32_t* tiles = (const int32_t*)(ws + P.tiles);
  const int32_t* ctrl = (const int32_t*)(ws + P.ctrl);
  const uint8_t* experts = (const uint8_t*)L->experts;
  const uint8_t* shared = (const uint8_t*)L->shared;
  if (mask & MOE_PREFILL_STAGE_STAGE_X)
    hipLaunchKernelGGL(k_stage16, dim3((T + 3) / 4), dim3(256), 0, s, x, T, d, xs, xscale);
  // grids: every (row tile, column group) item of the largest possible tile list
  // shapes that fit the 8-wave kernel (512 output columns per staged tile)
  // run there, the rest on the 4-wave one
  const bool wide = prefill_x2_shape(L);
  if ((mask & MOE_PREFILL_STAGE_GATEUP) && wide) {
    const int rc = launch_pfx_tern(L, T, R, ws, P, stream, true);
    if (rc) return rc;
    hipLaunchKernelGGL(k_stage16, dim3((rows + 3) / 4), dim3(256), 0, s, hs, rows, I, hs, hscale);
  } else if (mask & MOE_PREFILL_STAGE_GATEUP) {
    const int ncol = I / (32 * kW16);
    const dim3 g1((unsigned)(((long)P.max_tiles * ncol + 7) / 8 * 8));
    hipLaunchKernelGGL(k_pf16<2>, g1, dim3(64 * kW16), 0, s, experts, L->expert_stride, shared,
                       proj16(L, 0), proj16(L, 1), tiles, ctrl, R->perm_tok, Tk, 1, xs, xscale, d,
                       I, hs, ncol, tern_constants());
    // h to scaled fp16 rows in place, within this stage, so that every stage can be re-run
    hipLaunchKernelGGL(k_stage16, dim3((rows + 3) / 4), dim3(256), 0, s, hs, rows, I, hs, hscale);
  }
  if ((mask & MOE_PREFILL_STAGE_DOWN) && wide) {
    const int rc = launch_pfx_tern(L, T, R, ws, P, stream, false);
    if (rc) return rc;
  } else if (mask & MOE_PREFILL_STAGE_DOWN) {
    const int ncol = d / (64 * kW16);
    const dim3 g2((unsigned)(((long)P.max_tiles * ncol + 7) / 8 * 8));
    const ProjDesc pdn = proj16(L, 2);
    hipLaunchKernelGGL(k_pf16<1>, g2, dim3(64 * kW16), 0, s, experts, L->expert_stride, shared, pdn,
                       pdn, tiles, ctrl, R->perm_tok, Tk, 0, hs, hscale, I, d, y, ncol,
                       tern_constants());
  }
  return (int)hipGetLastError();
}

}  // namespace bqmoe
