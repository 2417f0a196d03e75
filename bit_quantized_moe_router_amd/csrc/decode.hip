// Decode kernels (1..8 tokens): stream each selected expert's packed bytes
// once for all of the tokens routed to it (the "Xolotl" README's "Latest"
// section describes decoding an expert once for all its tokens; its "Fast
// mode" section notes that decode speed is set by the expert bytes read per
// token).
//
// One kernel template serves both projections.  A block is (slot, column
// group): a slot is one active expert (or the shared expert) with its M <= 8
// rows; the column group is one 16-column n-tile of gate and of up (2
// streams), or 4 n-tiles (64 output columns) of down (4 streams).  The
// block's waves split the reduction dimension into contiguous k-block ranges,
// each wave owning up to 16 (stream, k-block) tiles (32 in single-token gate/up
// launches, whose waves are fewer and longer-lived).  A wave works through its
// k-blocks with the loads of the next one in flight:
//   1. it fetches the k-block's M activation rows (pre-scaled by 1/16) and
//      their 32-group sums into registers, with the k-block's packed tiles;
//   2. it writes the rows and sums to its own small LDS buffer when the
//      k-block's turn comes, and reads them back in matrix-operand order;
//   3. per 32-group:
//        A = the rows (lanes of rows >= M read row 0; those outputs are
//            discarded),
//        B = packed levels turned into bf16 values base + 16u by one
//            mask-and-or per pair of levels (see device_common.h),
//        C = the group's correction term (see mfma_corr in device_common.h),
//      so D = sum_k x * (u - offset) exactly for the group; D is scaled by the
//      group's fp16 scale (2 bytes per lane, broadcast with a lane shuffle)
//      and accumulated in fp32, only in the accumulator rows that hold real
//      rows.
// Every wait is placed by the compiler (no direct-to-LDS loads), and there
// are no branches around the work on a k-block: a load whose only use sits in
// a branch may be moved into it, which would undo the prefetch.
// Partial sums of the waves meet in LDS in a fixed order: no floating-point
// atomics, no cross-block synchronisation.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "moe_internal.h"
#include "topk_common.h"

namespace bqmoe {

typedef __attribute__((address_space(3))) void lds_void;

constexpr int kDecMaxRows = 8;  // rows of one slot (<= T <= 8)

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// ---------------------------------------------------------------- wave steps
// Row c of a slot is source row `base + c`, or with `gather` token
// (tok3 >> 3c) & 7 (decode tokens are < 8; no indexed array, which the
// compiler would place in scratch memory).
__device__ __forceinline__ int dec_src_row(int c, bool gather, int base, uint32_t tok3) {
  return gather ? (int)((tok3 >> (3 * c)) & 7u) : base + c;
}

// 1. A k-block of a slot's rows passes through a small per-wave LDS buffer:
//    rows [RC][256 B + 16 B pad] (the pad spreads the rows over the LDS
//    banks), then their staged sums [RC][64 B]; RC is the row cap (1 for a
//    single-token launch, else 8).  Rows >= M fetch row 0 (never read).  For
//    the down projection the fetched (W, S) half sums are turned into staged
//    sums on the way.
__host__ __device__ constexpr int ring_row_stride() { return 256 + 16; }
// staged sums of a row: 64 B, at a stride of 80 B (8 rows' 16-B reads then hit
// disjoint LDS banks; at 64 B rows r and r + 4 would share them)
__host__ __device__ constexpr int ring_sum_stride() { return 64 + 16; }
__host__ __device__ constexpr int ring_bytes(int rc) {
  return rc * (ring_row_stride() + ring_sum_stride());
}
// LDS of one wave: the buffer rounded to 256 B, then 256 B of zeros (the A
// operand of band rows that hold no row; see the band pipeline) placed 208 B
// further, in banks that no real-row read of the same instruction uses
// (row caps 1, 2 and 4).  Its offset in the buffer:
__host__ __device__ constexpr int ring_zero_offset(int rc) {
  return ((ring_bytes(rc) + 255) & ~255) + 208;
}
__host__ __device__ constexpr int ring_wave_bytes(int rc) { return ring_zero_offset(rc) + 256; }

template <int RC>
struct KbRegs {
  u32x4 a[(RC * 16 + 63) / 64];  // 16-byte pieces of the rows, one per lane
  u32x4 s;                       // one 32-group of one row (lanes < 4 RC)
};

template <int RC, bool CLAMP>
__device__ __forceinline__ void dec_kb_fetch(KbRegs<RC>& v, int lane, int M, bool gather,
                                             int base, uint32_t tok3,
                                             const uint16_t* __restrict__ A,
                                             const uint8_t* __restrict__ Asum, int K, int kb) {
  const int G = K / 32;
#pragma unroll
  for (int p = 0; p < (RC * 16 + 63) / 64; ++p) {
    const int piece = (p * 64 + lane) & (RC * 16 - 1);
    int c = piece >> 4;
    c = c < M ? c : 0;
    const int src = dec_src_row(c, gather, base, tok3);
    v.a[p] = *reinterpret_cast<const u32x4*>(reinterpret_cast<const uint8_t*>(A + (size_t)src * K) +
                                             kb * 256 + (piece & 15) * 16);
  }
  int c = (lane >> 2) & (RC - 1);
  c = c < M ? c : 0;
  const int src = dec_src_row(c, gather, base, tok3);
  v.s = *reinterpret_cast<const u32x4*>(Asum + (size_t)src * G * 16 + (kb * 4 + (lane & 3)) * 16);
}

// Every lane stores (lanes past the pieces repeat a piece with the same
// data): a store under a lane test would let the compiler move the fetch
// into that branch, next to its only use.
template <int RC, bool HALF_SUMS>
__device__ __forceinline__ void dec_kb_store(uint8_t* buf, const KbRegs<RC>& v, int lane) {
#pragma unroll
  for (int p = 0; p < (RC * 16 + 63) / 64; ++p) {
    const int piece = (p * 64 + lane) & (RC * 16 - 1);
    *reinterpret_cast<u32x4*>(buf + (piece >> 4) * ring_row_stride() + (piece & 15) * 16) =
        v.a[p];
  }
  u32x4 sv = v.s;
  if constexpr (HALF_SUMS) {
    // (Wa, Sa, Wb, Sb): fp32 sums of h over the group's two 16-column halves
    const uint4 st = stage_sums(__uint_as_float(sv[0]) + __uint_as_float(sv[2]),
                                __uint_as_float(sv[1]) + __uint_as_float(sv[3]));
    sv = u32x4{st.x, st.y, st.z, st.w};
  }
  const int slot = lane & (RC * 4 - 1);  // row slot / 4, group slot % 4
  *reinterpret_cast<u32x4*>(buf + RC * ring_row_stride() + (slot >> 2) * ring_sum_stride() +
                            (slot & 3) * 16) = sv;
}

// 2. Packed tiles of one of a wave's k-blocks (kb0 + i) for NS streams: codes
//    (8 B / lane), level bit 2 (4 B / lane, 3-bit only), and the 4 group
//    scales of the lane's column r (8 B / lane; the 4 lanes of a column read
//    the same bytes).  Stream j reads n-tile nt[j] of projection second(j) =
//    (GATEUP && j == 1).  The loads are unconditional; with CLAMP a wave past
//    the last k-block re-reads the last tile, without it (a wave that owns
//    all KBW k-blocks) the addresses of successive k-blocks differ by
//    constants.
template <int NS, bool GATEUP, bool QA3, bool QB3>
__host__ __device__ constexpr int dec_kb_loads() {
  return (2 + (QA3 ? 1 : 0)) + (NS - 1) * (2 + ((GATEUP ? QB3 : QA3) ? 1 : 0));
}

//    With WS = uint32_t (single-row k-blocks, below) a lane loads just the
//    scale of group lane / 16 of its column (2 B).
template <int NS, bool GATEUP, bool QA3, bool QB3, int KBW, bool CLAMP, typename WS>
__device__ __forceinline__ void dec_load_kb(int i, u32x2 (&wc)[KBW][NS], uint32_t (&wh)[KBW][NS],
                                            WS (&ws)[KBW][NS],
                                            const uint8_t* const (&code_base)[2],
                                            const size_t (&plane1)[2],
                                            const size_t (&scale_off)[2], const int (&nt)[NS],
                                            int KB, int kb0, int lane) {
  const int r = lane & 15;
  const int kbc = CLAMP ? min(kb0 + i, KB - 1) : kb0 + i;
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    const int second = GATEUP && j == 1;
    const bool q3 = second ? QB3 : QA3;
    const uint8_t* base = code_base[second];
    const size_t tile = (size_t)nt[j] * KB + kbc;
    wc[i][j] = *reinterpret_cast<const u32x2*>(base + tile * 512 + lane * 8);
    wh[i][j] =
        q3 ? *reinterpret_cast<const uint32_t*>(base + plane1[second] + tile * 256 + lane * 4)
           : 0u;
    if constexpr (std::is_same_v<WS, uint32_t>)
      ws[i][j] = *reinterpret_cast<const uint16_t*>(base + scale_off[second] + tile * 128 + r * 8 +
                                                    (lane >> 4) * 2);
    else
      ws[i][j] = *reinterpret_cast<const u32x2*>(base + scale_off[second] + tile * 128 + r * 8);
  }
}

// 3. Matrix-core work on one k-block; per 32-group one correction op (two if
//    the projections differ) and one op per stream; the group's scale
//    multiplies MR accumulator rows (rows 4*(lane/16) + i carry real rows for
//    i < M; MR = M for M <= 2, else 4).  A and the sums come from the
//    k-block's LDS buffer.  GUARD: a k-block past the wave's range (live
//    false) adds zero, through a zero scale.
template <int NS, bool GATEUP, bool QA3, bool QB3, bool SAMEC, int KBW, int MR, bool GUARD>
__device__ __forceinline__ void dec_mfma_kb(int i, f32x4 (&acc)[NS], const u32x2 (&wc)[KBW][NS],
                                            const uint32_t (&wh)[KBW][NS],
                                            const u32x2 (&ws)[KBW][NS], const uint8_t* aptr,
                                            const uint8_t* sptr, u32x4 bca, u32x4 bcb,
                                            const Unpack2R& ur, bool live = true) {
#pragma unroll
  for (int GB = 0; GB < 4; ++GB) {
    const u32x4 a = *reinterpret_cast<const u32x4*>(aptr + GB * 64);
    const u32x4 sv = *reinterpret_cast<const u32x4*>(sptr + GB * 16);
    const f32x4 corr_a = mfma_corr(sv, bca);
    f32x4 corr_b = corr_a;
    if constexpr (!SAMEC) corr_b = mfma_corr(sv, bcb);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const bool second = GATEUP && j == 1;
      const bool q3 = second ? QB3 : QA3;
      const uint32_t word = (GB < 2) ? wc[i][j][0] : wc[i][j][1];
      u32x4 b;
      if (q3) {
        if (GB == 0) b = unpack3<0>(word, wh[i][j], ur);
        if (GB == 1) b = unpack3<1>(word, wh[i][j], ur);
        if (GB == 2) b = unpack3<2>(word, wh[i][j], ur);
        if (GB == 3) b = unpack3<3>(word, wh[i][j], ur);
      } else {
        b = (GB & 1) ? unpack2_r<1>(word, ur) : unpack2_r<0>(word, ur);
      }
      const f32x4 dd = mfma32(a, b, second ? corr_b : corr_a);
      // fp16 scale of (column r, group GB): half GB & 1 of word GB >> 1
      const uint32_t sw = ws[i][j][GB >> 1];
      float s = f16_to_f32((GB & 1) ? (sw >> 16) : sw);
      if constexpr (GUARD) s = live ? s : 0.f;
#pragma unroll
      for (int m = 0; m < MR; ++m) acc[j][m] = fmaf(s, dd[m], acc[j][m]);
    }
  }
}

// 4. A wave's k-blocks: k-block i's rows, sums and tiles are fetched PRE
//    k-blocks ahead of its matrix-core work, in the wave's own instruction
//    stream (when the memory system pushes back on issue, the wave keeps
//    computing on what it has); its rows and sums are written to the wave's
//    LDS buffer just before its turn (LDS operations of a wave run in order,
//    so the writes wait for the previous k-block's reads).  With FULL the
//    wave owns KBW k-blocks, otherwise those past nkb add zero.
template <int NS, bool GATEUP, bool QA3, bool QB3, bool SAMEC, int KBW, int PRE, int MR, int RC,
          bool FULL>
__device__ __forceinline__ void dec_pipeline(
    f32x4 (&acc)[NS], u32x2 (&wc)[KBW][NS], uint32_t (&wh)[KBW][NS], u32x2 (&ws)[KBW][NS],
    const uint8_t* const (&code_base)[2], const size_t (&plane1)[2], const size_t (&scale_off)[2],
    const int (&nt)[NS], int KB, int kb0, int nkb, int lane, uint8_t* buf, int M, bool gather,
    int row0, uint32_t tok3, const uint16_t* __restrict__ A, const uint8_t* __restrict__ Asum,
    int K, u32x4 bca, u32x4 bcb, const Unpack2R& ur) {
  const int q = lane >> 4, r = lane & 15;
  const int arow = r < M ? r : 0;
  KbRegs<RC> v[KBW];
#pragma unroll
  for (int i = 0; i < PRE; ++i) {
    dec_kb_fetch<RC, !FULL>(v[i], lane, M, gather, row0, tok3, A, Asum, K,
                            FULL ? kb0 + i : min(kb0 + i, KB - 1));
    dec_load_kb<NS, GATEUP, QA3, QB3, KBW, !FULL>(i, wc, wh, ws, code_base, plane1, scale_off, nt, KB,
                                           kb0, lane);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < KBW; ++i) {
    if (i + PRE < KBW) {
      dec_kb_fetch<RC, !FULL>(v[i + PRE], lane, M, gather, row0, tok3, A, Asum, K,
                              FULL ? kb0 + i + PRE : min(kb0 + i + PRE, KB - 1));
      dec_load_kb<NS, GATEUP, QA3, QB3, KBW, !FULL>(i + PRE, wc, wh, ws, code_base, plane1, scale_off,
                                             nt, KB, kb0, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    dec_kb_store<RC, !GATEUP>(buf, v[i], lane);
    dec_mfma_kb<NS, GATEUP, QA3, QB3, SAMEC, KBW, MR, !FULL>(
        i, acc, wc, wh, ws, buf + arow * ring_row_stride() + q * 16,
        buf + RC * ring_row_stride() + arow * ring_sum_stride(), bca, bcb, ur, i < nkb);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// 3'. Matrix-core work on a k-block of at most 4 rows (MR).  The k-block's
//     four 32-groups go to accumulator row bands 4g .. 4g + MR - 1: for group
//     g the A operand is the rows' group g in band g and zeros elsewhere
//     (lanes of the other rows read a zeroed LDS area), so the four ops of a
//     stream add to disjoint rows of one accumulator.  One correction op, its
//     A operand the four groups' staged sums in the same rows, starts that
//     accumulator.  Lane l then holds group l / 16 of column l % 16 for rows
//     0 .. MR-1 in elements 0 .. MR-1 and applies that group's scale with MR
//     FMAs (one 2-byte scale load per lane).  The four lane quarters are
//     added at the end of the wave's range.
template <int NS, bool GATEUP, bool QA3, bool QB3, bool SAMEC, int KBW, int MR, int ASTRIDE,
          int SSTRIDE, bool GUARD>
__device__ __forceinline__ void dec_mfma_kb_band(int i, f32x4 (&acc)[NS],
                                                 const u32x2 (&wc)[KBW][NS],
                                                 const uint32_t (&wh)[KBW][NS],
                                                 const uint32_t (&ws)[KBW][NS],
                                                 const uint8_t* a0, const uint8_t* a1,
                                                 const uint8_t* a2, const uint8_t* a3,
                                                 const uint8_t* sp, u32x4 bca, u32x4 bcb,
                                                 const Unpack2R& ur, bool live) {
  const u32x4 sv = *reinterpret_cast<const u32x4*>(sp + i * SSTRIDE);
  const f32x4 corr_a = mfma_corr(sv, bca);
  f32x4 corr_b = corr_a;
  if constexpr (!SAMEC) corr_b = mfma_corr(sv, bcb);
  f32x4 d[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) d[j] = (GATEUP && j == 1) ? corr_b : corr_a;
#pragma unroll
  for (int GB = 0; GB < 4; ++GB) {
    const uint8_t* ap = GB == 0 ? a0 : GB == 1 ? a1 : GB == 2 ? a2 : a3;
    const u32x4 a = *reinterpret_cast<const u32x4*>(ap + i * ASTRIDE);
#pragma unroll
    for (int j = 0; j < NS; ++j) {
      const bool second = GATEUP && j == 1;
      const bool q3 = second ? QB3 : QA3;
      const uint32_t word = (GB < 2) ? wc[i][j][0] : wc[i][j][1];
      u32x4 b;
      if (q3) {
        if (GB == 0) b = unpack3<0>(word, wh[i][j], ur);
        if (GB == 1) b = unpack3<1>(word, wh[i][j], ur);
        if (GB == 2) b = unpack3<2>(word, wh[i][j], ur);
        if (GB == 3) b = unpack3<3>(word, wh[i][j], ur);
      } else {
        b = (GB & 1) ? unpack2_r<1>(word, ur) : unpack2_r<0>(word, ur);
      }
      d[j] = mfma32(a, b, d[j]);
    }
  }
#pragma unroll
  for (int j = 0; j < NS; ++j) {
    float s = f16_to_f32(ws[i][j]);
    if constexpr (GUARD) s = live ? s : 0.f;
#pragma unroll
    for (int m = 0; m < MR; ++m) acc[j][m] = fmaf(s, d[j][m], acc[j][m]);
  }
}

// Sum over a 16-lane row, left in all of its lanes: each step adds the value
// of a partner lane in a disjoint pairing (xor 1, xor 2, the mirror within 8
// lanes, the mirror within 16 lanes).
__device__ __forceinline__ float row16_sum(float v) {
  int b = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_mov_dpp(b, 0xB1, 0xF, 0xF, true));  // [1,0,3,2]
  b = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x4E, 0xF, 0xF, true));  // [2,3,0,1]
  b = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x141, 0xF, 0xF, true));  // half mirror
  b = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_mov_dpp(b, 0x140, 0xF, 0xF, true));  // mirror
  return v;
}

// The four lane quarters (groups) of a column added: lanes 0..15 then hold
// rows 0..MR-1 in elements 0..MR-1, the matrix-core layout of rows 0..3.
template <int NS, int MR>
__device__ __forceinline__ void dec_band_fold(f32x4 (&acc)[NS]) {
#pragma unroll
  for (int j = 0; j < NS; ++j)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float v = m < MR ? acc[j][m] : 0.f;
      if (m < MR) {
        // partner lanes l ^ 16, then l ^ 32, by the gfx950 lane swaps (each
        // lane adds the same two values in the same order)
        const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v),
                                                        false, false);
        v = __uint_as_float(p[0]) + __uint_as_float(p[1]);
        const auto q = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v),
                                                        false, false);
        v = __uint_as_float(q[0]) + __uint_as_float(q[1]);
      }
      acc[j][m] = v;
    }
}

// 4b. dec_pipeline for slots of at most 4 rows (MR: 1, 2 or 4; RC >= M) in
//     the banded form of step 3': the rows' groups go to row bands of the
//     accumulator, so a k-block takes one correction op and MR FMAs per
//     stream.  The wave's LDS buffer is the same as dec_pipeline's, its zeroed
//     256 B at the end.  On return rows 0..M-1 sit in lanes 0..15, elements
//     0..M-1.
template <int NS, bool GATEUP, bool QA3, bool QB3, bool SAMEC, int KBW, int PRE, int MR, int RC,
          bool FULL>
__device__ __forceinline__ void dec_pipeline_bandr(
    f32x4 (&acc)[NS], u32x2 (&wc)[KBW][NS], uint32_t (&wh)[KBW][NS], uint32_t (&ws)[KBW][NS],
    const uint8_t* const (&code_base)[2], const size_t (&plane1)[2], const size_t (&scale_off)[2],
    const int (&nt)[NS], int KB, int kb0, int nkb, int lane, uint8_t* buf, int M, bool gather,
    int row0, uint32_t tok3, const uint16_t* __restrict__ A, const uint8_t* __restrict__ Asum,
    int K, u32x4 bca, u32x4 bcb, const Unpack2R& ur) {
  static_assert(MR <= 4 && RC >= MR, "band rows");
  uint8_t* zbuf = buf + ring_zero_offset(RC);
  *reinterpret_cast<u32x4*>(zbuf + (lane & 15) * 16) = u32x4{0u, 0u, 0u, 0u};
  // per-lane operand addresses: lane l reads row c = l % 4 of group g = (l % 16) / 4
  const int q = lane >> 4, c = lane & 3, g = (lane >> 2) & 3;
  const bool real = c < M;
  const uint8_t* a0 = (real && g == 0 ? buf + c * ring_row_stride() : zbuf) + q * 16;
  const uint8_t* a1 = (real && g == 1 ? buf + c * ring_row_stride() + 64 : zbuf + 64) + q * 16;
  const uint8_t* a2 = (real && g == 2 ? buf + c * ring_row_stride() + 128 : zbuf + 128) + q * 16;
  const uint8_t* a3 = (real && g == 3 ? buf + c * ring_row_stride() + 192 : zbuf + 192) + q * 16;
  const uint8_t* sp = (lane < 16 && real) ? buf + RC * ring_row_stride() + c * ring_sum_stride() +
                                                g * 16
                                          : zbuf;
  KbRegs<RC> v[KBW];
#pragma unroll
  for (int i = 0; i < PRE; ++i) {
    dec_kb_fetch<RC, !FULL>(v[i], lane, M, gather, row0, tok3, A, Asum, K,
                            FULL ? kb0 + i : min(kb0 + i, KB - 1));
    dec_load_kb<NS, GATEUP, QA3, QB3, KBW, !FULL>(i, wc, wh, ws, code_base, plane1, scale_off, nt,
                                                  KB, kb0, lane);
  }
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int i = 0; i < KBW; ++i) {
    if (i + PRE < KBW) {
      dec_kb_fetch<RC, !FULL>(v[i + PRE], lane, M, gather, row0, tok3, A, Asum, K,
                              FULL ? kb0 + i + PRE : min(kb0 + i + PRE, KB - 1));
      dec_load_kb<NS, GATEUP, QA3, QB3, KBW, !FULL>(i + PRE, wc, wh, ws, code_base, plane1,
                                                    scale_off, nt, KB, kb0, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    dec_kb_store<RC, !GATEUP>(buf, v[i], lane);
    dec_mfma_kb_band<NS, GATEUP, QA3, QB3, SAMEC, KBW, MR, 0, 0, !FULL>(
        i, acc, wc, wh, ws, a0, a1, a2, a3, sp, bca, bcb, ur, i < nkb);
    __builtin_amdgcn_sched_barrier(0);
  }
  dec_band_fold<NS, MR>(acc);
}

// 4'. The pipeline of a single-token launch: the wave's whole slice of the
//     row (KBW k-blocks, [KBW][256 B], then the sums [KBW][64 B]) is fetched
//     into registers ahead of the first tiles and written to LDS once, next
//     to a zeroed area of [KBW][256 B] (64 B further, so that the real and
//     the zero lanes of one read use different banks); a k-block's work then
//     only reads LDS.
//     On return acc[j][0] of lanes 0..15 holds the wave's sum for column
//     lane (the other elements are zero).
__host__ __device__ constexpr int one_wave_bytes(int kbw) { return kbw * (256 + 64 + 256) + 64; }

template <int NS, bool GATEUP, bool QA3, bool QB3, bool SAMEC, int KBW, int PRE, bool FULL>
__device__ __forceinline__ void dec_pipeline_band(
    f32x4 (&acc)[NS], u32x2 (&wc)[KBW][NS], uint32_t (&wh)[KBW][NS], uint32_t (&ws)[KBW][NS],
    const uint8_t* const (&code_base)[2], const size_t (&plane1)[2], const size_t (&scale_off)[2],
    const int (&nt)[NS], int KB, int kb0, int nkb, int lane, uint8_t* buf, bool gather, int row0,
    uint32_t tok3, const uint16_t* __restrict__ A, const uint8_t* __restrict__ Asum, int K,
    u32x4 bca, u32x4 bcb, const Unpack2R& ur) {
  constexpr int NPA = (KBW * 16 + 63) / 64;  // 16-byte pieces of the slice per lane
  const int G = K / 32;
  const int src = dec_src_row(0, gather, row0, tok3);
  const uint8_t* arow = reinterpret_cast<const uint8_t*>(A + (size_t)src * K);
  u32x4 va[NPA];
#pragma unroll
  for (int p = 0; p < NPA; ++p) {
    const int piece = (p * 64 + lane) & (KBW * 16 - 1);
    const int kb = FULL ? kb0 + (piece >> 4) : min(kb0 + (piece >> 4), KB - 1);
    va[p] = *reinterpret_cast<const u32x4*>(arow + kb * 256 + (piece & 15) * 16);
  }
  const int spiece = lane & (KBW * 4 - 1);
  u32x4 vs = *reinterpret_cast<const u32x4*>(
      Asum + (size_t)src * G * 16 +
      ((FULL ? kb0 + (spiece >> 2) : min(kb0 + (spiece >> 2), KB - 1)) * 4 + (spiece & 3)) * 16);
#pragma unroll
  for (int i = 0; i < PRE; ++i)
    dec_load_kb<NS, GATEUP, QA3, QB3, KBW, !FULL>(i, wc, wh, ws, code_base, plane1, scale_off, nt,
                                                  KB, kb0, lane);
  __builtin_amdgcn_sched_barrier(0);
  uint8_t* zbuf = buf + KBW * (256 + 64) + 64;
#pragma unroll
  for (int p = 0; p < NPA; ++p) {
    const int piece = (p * 64 + lane) & (KBW * 16 - 1);
    *reinterpret_cast<u32x4*>(zbuf + piece * 16) = u32x4{0u, 0u, 0u, 0u};
    *reinterpret_cast<u32x4*>(buf + piece * 16) = va[p];
  }
  if constexpr (!GATEUP) {
    // (Wa, Sa, Wb, Sb): fp32 sums of h over the group's two 16-column halves
    const uint4 st = stage_sums(__uint_as_float(vs[0]) + __uint_as_float(vs[2]),
                                __uint_as_float(vs[1]) + __uint_as_float(vs[3]));
    vs = u32x4{st.x, st.y, st.z, st.w};
  }
  *reinterpret_cast<u32x4*>(buf + KBW * 256 + spiece * 16) = vs;
  // per-lane operand addresses: group g of a k-block from the slice in the
  // lanes of row 4g, from the zeroed area in the others
  const int q = lane >> 4, r16 = lane & 15;
  const uint8_t* a0 = (r16 == 0 ? buf : zbuf) + q * 16;
  const uint8_t* a1 = (r16 == 4 ? buf : zbuf) + 64 + q * 16;
  const uint8_t* a2 = (r16 == 8 ? buf : zbuf) + 128 + q * 16;
  const uint8_t* a3 = (r16 == 12 ? buf : zbuf) + 192 + q * 16;
  const uint8_t* sp = (lane < 16 && (lane & 3) == 0) ? buf + KBW * 256 + (lane >> 2) * 16 : zbuf;
#pragma unroll
  for (int i = 0; i < KBW; ++i) {
    if (i + PRE < KBW) {
      dec_load_kb<NS, GATEUP, QA3, QB3, KBW, !FULL>(i + PRE, wc, wh, ws, code_base, plane1,
                                                    scale_off, nt, KB, kb0, lane);
      __builtin_amdgcn_sched_barrier(0);
    }
    dec_mfma_kb_band<NS, GATEUP, QA3, QB3, SAMEC, KBW, 1, 256, 64, !FULL>(
        i, acc, wc, wh, ws, a0, a1, a2, a3, sp, bca, bcb, ur, i < nkb);
    __builtin_amdgcn_sched_barrier(0);
  }
  dec_band_fold<NS, 1>(acc);
}

// k-blocks whose tile loads run ahead of the matrix-core work.  Shallow on
// purpose: every wave of the launch streams at once, the memory pipeline is
// saturated throughout, and deeper per-wave prefetch only lets the oldest waves
// hold the issue queue longer (measured: 1 ahead is best for 8 k-blocks per
// wave, 2 for 16).
__host__ __device__ constexpr int dec_pre(int kbw) { return kbw >= 16 ? 2 : 1; }



// ---------------------------------------- expert selection for one token
// Outputs of the selection, written by block 0 of a ROUTE launch.
struct DecRoute {
  const float* logits;
  int E, k, n_shared, max_slots;
  int32_t* ids;
  float* wts;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm_tok;
  int32_t* inv_row;
  int32_t* slots;
};

// Wave 0: top-k of token 0 (wave_topk, E <= 256), the rank of each selected
// id among them, and this block's slot: (expert, first permuted row, row
// count), handed to the block's other waves through LDS.  Block 0 also stores
// the routing outputs, as the select kernel does for T = 1: row j of the
// token goes to permuted position rank_j.  (The selection repeated by every
// wave of the launch cost several microseconds of issue.)
__device__ __forceinline__ void dec_select_one_token(const DecRoute& ro, int slot, int& e,
                                                     int& row0, int& M) {
  __shared__ int s_ids[64];
  __shared__ int s_slot[3];
  const int tid = threadIdx.x, lane = tid & 63;
  const int k = ro.k;
  if (tid < 64) {
    // the block's work waits on this chain; other blocks' waves on the SIMD
    // are already streaming, so it takes the issue slots first
    __builtin_amdgcn_s_setprio(3);
    int id;
    float w;
    wave_topk<4>(ro.logits, ro.E, k, lane, id, w);
    int rank = 0;  // selected ids below this lane's (lanes < k)
    for (int j = 0; j < k; ++j) rank += __builtin_amdgcn_readlane(id, j) < id ? 1 : 0;
    if (lane < k) s_ids[lane] = id;
    const uint64_t m = __ballot(lane < k && rank == slot);  // whole wave
    const int e_slot = m ? __builtin_amdgcn_readlane(id, __ffsll((unsigned long long)m) - 1) : -1;
    if (lane == 0) {
      if (slot < k) {
        s_slot[0] = e_slot;
        s_slot[1] = slot;
        s_slot[2] = 1;
      } else {
        s_slot[0] = -1;
        s_slot[1] = k;
        s_slot[2] = slot == k && ro.n_shared ? 1 : 0;
      }
    }
    if (blockIdx.x == 0) {
      if (lane < k) {
        ro.ids[lane] = id;
        ro.wts[lane] = w;
        ro.inv_row[lane] = rank;
        ro.perm_tok[lane] = 0;
        int32_t* rec = ro.slots + kSlotRec * (1 + rank);
        rec[0] = id;
        rec[1] = rank;
        rec[2] = 1;
        rec[3] = 0;
        rec[kSlotTok] = 0;
      }
      if (lane == 0) {
        if (ro.n_shared) {
          int32_t* rec = ro.slots + kSlotRec * (1 + k);
          rec[0] = -1;
          rec[1] = k;
          rec[2] = 1;
          rec[3] = 0;
          rec[kSlotTok] = 0;
        }
        ro.slots[0] = k + (ro.n_shared ? 1 : 0);
        ro.offsets[ro.E] = k;
      }
    }
    __builtin_amdgcn_s_setprio(0);
  }
  __syncthreads();
  e = __builtin_amdgcn_readfirstlane(s_slot[0]);
  row0 = __builtin_amdgcn_readfirstlane(s_slot[1]);
  M = __builtin_amdgcn_readfirstlane(s_slot[2]);
  if (blockIdx.x != 0) return;
  for (int x = tid; x < ro.E; x += blockDim.x) {
    int cnt = 0, off = 0;
    for (int j = 0; j < k; ++j) {
      const int o = s_ids[j];
      cnt += o == x ? 1 : 0;
      off += o < x ? 1 : 0;
    }
    ro.counts[x] = cnt;
    ro.offsets[x] = off;
  }
  // records past the last slot: no rows
  for (int sidx = k + (ro.n_shared ? 1 : 0) + tid; sidx < ro.max_slots; sidx += blockDim.x) {
    int32_t* rec = ro.slots + kSlotRec * (1 + sidx);
    rec[0] = 0;
    rec[1] = 0;
    rec[2] = 0;
    rec[3] = 0;
  }
}

// ------------------------------------------------------- projection kernel
// GATEUP = true: streams 0 (gate) and 1 (up) of n-tile blockIdx % groups;
//   epilogue h = bf16(SiLU(g) * u), stored as h/16, plus fp32 (W, S) sums of
//   h over the tile's 16 columns (half of a 32-group of the down projection).
// GATEUP = false (down): streams 0..3 = n-tiles 4g .. 4g+3; the 32-group sums
//   of h are the two half sums added; epilogue y = bf16(acc).
// ONE_ROW: launched for a single token, so every slot has M == 1 (the wave's
// whole slice of the row is staged at once).
// want_alt >= 0: only the slots whose record says they read the second
// expert copy (1) or the first (0); the caller passes that copy's blobs.
// ROUTE (single-token gate/up, E <= 256): the kernel makes the expert
// selection itself instead of reading the slot list: wave 0 takes the token's
// top-k from the logits (the routing kernels' own wave_topk), and the k
// selected experts in ascending id are slots 0..k-1, then the shared expert
// (for one token, slot s is also permuted row s).  Block 0 writes every
// routing output the select kernel would have written (ids, weights, counts,
// offsets, permutation, slot list), for the down projection and the caller.
template <bool GATEUP, bool QA3, bool QB3, bool SAMEC, int KSPLIT, int KBW, bool ONE_ROW,
          bool ROUTE = false>
__device__ __forceinline__ void dec_proj_body(
    const uint8_t* __restrict__ experts, size_t stride, const uint8_t* __restrict__ shared,
    ProjDesc pa, ProjDesc pb, const int32_t* __restrict__ slots, const uint16_t* __restrict__ A,
    const uint8_t* __restrict__ Asum, int K, int N, int Mmax, float ca, float cb,
    uint16_t* __restrict__ out, float* __restrict__ out_psum, Unpack2K uk, DecRoute ro,
    int want_alt) {
  constexpr int NS = GATEUP ? 2 : 4;
  static_assert(!ROUTE || (GATEUP && ONE_ROW), "selection inside single-token gate/up only");
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int groups = N / (16 * (GATEUP ? 1 : 4));
  const int slot = blockIdx.x / groups, grp = blockIdx.x % groups;
  int e, row0, M;
  uint32_t tok3 = 0;  // tokens of the slot's rows, 3 bits each
  if constexpr (ROUTE) {
    if (slot == ro.k && ro.n_shared) {
      // the shared expert's blocks need no selection (slot k, permuted row k):
      // they stream at once, under the routed blocks' top-k
      e = -1;
      row0 = ro.k;
      M = 1;
    } else {
      dec_select_one_token(ro, slot, e, row0, M);
    }
  } else {
    // the slot record is uniform: scalar loads, which do not wait behind the
    // packed-tile loads below; records past the last slot have M == 0
    const int32_t* rec = slots + kSlotRec * (1 + slot);
    e = rec[0];
    row0 = rec[1];
    M = rec[2];
    // with a second expert copy, the launch for one copy skips the other's slots
    if (want_alt >= 0 && rec[3] != want_alt) M = 0;
    if (GATEUP) {
#pragma unroll
      for (int c = 0; c < kDecMaxRows; ++c)
        tok3 |= c < M ? (uint32_t)rec[kSlotTok + c] << (3 * c) : 0u;
    }
  }
  if (M == 0) return;
  const uint8_t* blob = e >= 0 ? experts + (size_t)e * stride : shared;
  // projection offsets in registers before any LDS write (which the compiler
  // cannot tell apart from the argument memory)
  const uint8_t* const code_base[2] = {blob + pa.off, blob + pb.off};
  const size_t plane1[2] = {pa.plane1, pb.plane1};
  const size_t scale_off[2] = {pa.scales, pb.scales};
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int KB = K / 128;
  const int per = (KB + KSPLIT - 1) / KSPLIT;
  const int kb0 = min(KB, wave * per);
  const int nkb = min(KB, kb0 + per) - kb0;  // 0 .. KBW
  int nt[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) nt[j] = GATEUP ? grp : grp * 4 + j;
  constexpr int PRE = dec_pre(KBW);
  const u32x4 bca = corr_b_operand(q == 0, ca);
  const u32x4 bcb = corr_b_operand(q == 0, cb);
  const Unpack2R ur = {uk.m0, uk.m1, uk.m2, lane_copy(uk.b0), lane_copy(uk.b1), lane_copy(uk.b2)};
  f32x4 acc[NS];
#pragma unroll
  for (int j = 0; j < NS; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  u32x2 wc[KBW][NS];
  uint32_t wh[KBW][NS];
  if constexpr (ONE_ROW) {
    uint32_t ws[KBW][NS];
    uint8_t* buf = lds + wave * one_wave_bytes(KBW);
    if (nkb < KBW)
      dec_pipeline_band<NS, GATEUP, QA3, QB3, SAMEC, KBW, PRE, false>(
          acc, wc, wh, ws, code_base, plane1, scale_off, nt, KB, kb0, nkb, lane, buf, GATEUP,
          row0, tok3, A, Asum, K, bca, bcb, ur);
    else
      dec_pipeline_band<NS, GATEUP, QA3, QB3, SAMEC, KBW, PRE, true>(
          acc, wc, wh, ws, code_base, plane1, scale_off, nt, KB, kb0, nkb, lane, buf, GATEUP,
          row0, tok3, A, Asum, K, bca, bcb, ur);
  } else {
    u32x2 ws[KBW][NS];
    uint32_t wsb[KBW][NS];
    uint8_t* buf = lds + wave * ring_wave_bytes(kDecMaxRows);
    if (nkb < KBW)
      dec_pipeline<NS, GATEUP, QA3, QB3, SAMEC, KBW, PRE, 4, kDecMaxRows, false>(
          acc, wc, wh, ws, code_base, plane1, scale_off, nt, KB, kb0, nkb, lane, buf, M, GATEUP,
          row0, tok3, A, Asum, K, bca, bcb, ur);
    else if (M == 1)
      dec_pipeline_bandr<NS, GATEUP, QA3, QB3, SAMEC, KBW, PRE, 1, 1, true>(
          acc, wc, wh, wsb, code_base, plane1, scale_off, nt, KB, kb0, nkb, lane, buf, M, GATEUP,
          row0, tok3, A, Asum, K, bca, bcb, ur);
    else if (M == 2)
      dec_pipeline_bandr<NS, GATEUP, QA3, QB3, SAMEC, KBW, PRE, 2, 2, true>(
          acc, wc, wh, wsb, code_base, plane1, scale_off, nt, KB, kb0, nkb, lane, buf, M, GATEUP,
          row0, tok3, A, Asum, K, bca, bcb, ur);
    else if (M <= 4)
      dec_pipeline_bandr<NS, GATEUP, QA3, QB3, SAMEC, KBW, PRE, 4, 4, true>(
          acc, wc, wh, wsb, code_base, plane1, scale_off, nt, KB, kb0, nkb, lane, buf, M, GATEUP,
          row0, tok3, A, Asum, K, bca, bcb, ur);
    else
      dec_pipeline<NS, GATEUP, QA3, QB3, SAMEC, KBW, PRE, 4, kDecMaxRows, true>(
          acc, wc, wh, ws, code_base, plane1, scale_off, nt, KB, kb0, nkb, lane, buf, M, GATEUP,
          row0, tok3, A, Asum, K, bca, bcb, ur);
  }

  // 5. cross-wave reduction in a fixed order (every wave is done with LDS)
  __syncthreads();
  float* red = reinterpret_cast<float*>(lds);  // [KSPLIT][NS][4][32 lanes]
  if (lane < 32) {
#pragma unroll
    for (int j = 0; j < NS; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) red[((wave * NS + j) * 4 + i) * 32 + lane] = acc[j][i];
  }
  __syncthreads();
  if constexpr (GATEUP) {
    // 16 threads per row (whole 16-lane segments of waves 0 and 1)
    if (tid < kDecMaxRows * 16) {
      const int row = tid >> 4, col = tid & 15;
      const int ln = 16 * (row >> 2) + col, i = row & 3;
      float hf = 0.f;
      if (row < M) {
        float g = 0.f, u = 0.f;
        for (int w = 0; w < KSPLIT; ++w) {
          g += red[((w * 2 + 0) * 4 + i) * 32 + ln];
          u += red[((w * 2 + 1) * 4 + i) * 32 + ln];
        }
        hf = bf16_to_f32(f32_to_bf16(silu_f(g) * u));
        out[(size_t)(row0 + row) * N + grp * 16 + col] = (uint16_t)f32_to_bf16(hf * 0.0625f);
      }
      // (W, S) of h over this tile's 16 columns: k-slots 16*(grp%2) + col of
      // the down projection's 32-group grp/2
      // (sums over the 16 lanes of the row by DPP moves: xor 1, xor 2, then
      // the mirrors within 8 and 16 lanes)
      float sw = hf * slot_weight(16 * (grp & 1) + col), s = hf;
      sw = row16_sum(sw);
      s = row16_sum(s);
      if (row < M && col == 0)
        *reinterpret_cast<float2*>(out_psum + ((size_t)(row0 + row) * (N / 16) + grp) * 2) =
            make_float2(sw, s);
    }
  } else {
    for (int t = tid; t < M * 64; t += 64 * KSPLIT) {
      const int row = t >> 6, j = (t >> 4) & 3, col = t & 15;
      const int ln = 16 * (row >> 2) + col, i = row & 3;
      float s = 0.f;
      for (int w = 0; w < KSPLIT; ++w) s += red[((w * 4 + j) * 4 + i) * 32 + ln];
      out[(size_t)(row0 + row) * N + (nt[0] + j) * 16 + col] = (uint16_t)f32_to_bf16(s);
    }
  }
}

template <bool GATEUP, bool QA3, bool QB3, bool SAMEC, int KSPLIT, int KBW, bool ONE_ROW,
          bool ROUTE = false>
__global__ __launch_bounds__(64 * KSPLIT) void k_dec_proj(
    const uint8_t* __restrict__ experts, size_t stride, const uint8_t* __restrict__ shared,
    ProjDesc pa, ProjDesc pb, const int32_t* __restrict__ slots, const uint16_t* __restrict__ A,
    const uint8_t* __restrict__ Asum, int K, int N, int Mmax, float ca, float cb,
    uint16_t* __restrict__ out, float* __restrict__ out_psum, Unpack2K uk, DecRoute ro,
    int want_alt) {
  dec_proj_body<GATEUP, QA3, QB3, SAMEC, KSPLIT, KBW, ONE_ROW, ROUTE>(
      experts, stride, shared, pa, pb, slots, A, Asum, K, N, Mmax, ca, cb, out, out_psum, uk, ro,
      want_alt);
}

// Both expert copies in one launch: each block reads its slot's copy flag
// (uniform over the block) and runs the projection on that copy's blobs,
// code families (QA3.. for the first copy, XA3.. for the second) and offsets.
template <bool GATEUP, bool QA3, bool QB3, bool SAMEC, bool XA3, bool XB3, bool XSAMEC,
          int KSPLIT, int KBW, bool ONE_ROW>
__global__ __launch_bounds__(64 * KSPLIT) void k_dec_proj_mixed(
    const uint8_t* __restrict__ experts, size_t stride, const uint8_t* __restrict__ shared,
    ProjDesc pa, ProjDesc pb, const uint8_t* __restrict__ alt_experts, size_t alt_stride,
    ProjDesc xpa, ProjDesc xpb, const int32_t* __restrict__ slots, const uint16_t* __restrict__ A,
    const uint8_t* __restrict__ Asum, int K, int N, int Mmax, float ca, float cb, float xca,
    float xcb, uint16_t* __restrict__ out, float* __restrict__ out_psum, Unpack2K uk) {
  const int groups = N / (16 * (GATEUP ? 1 : 4));
  const int slot = blockIdx.x / groups;
  if (slots[kSlotRec * (1 + slot) + 3] != 0)
    dec_proj_body<GATEUP, XA3, XB3, XSAMEC, KSPLIT, KBW, ONE_ROW>(
        alt_experts, alt_stride, shared, xpa, xpb, slots, A, Asum, K, N, Mmax, xca, xcb, out,
        out_psum, uk, DecRoute{}, 1);
  else
    dec_proj_body<GATEUP, QA3, QB3, SAMEC, KSPLIT, KBW, ONE_ROW>(
        experts, stride, shared, pa, pb, slots, A, Asum, K, N, Mmax, ca, cb, out, out_psum, uk,
        DecRoute{}, 0);
}

// ------------------------------------------------- down projection + combine
// For few slots (<= 16) and a short reduction (I <= 2048): block = one
// 16-column n-tile of the output, wave s = slot s over the whole of I (no
// cross-wave reduction).  Each wave leaves y = bf16(h . Wd) of its rows for
// the tile in LDS; the block then forms
//   out[t] = bf16( [x[t]] + sum_j w[t][j] * y[inv_row[t][j]] + [y[T*k + t]] )
// for its 16 columns in the same order as the separate combine kernel.
template <bool Q3, int KBW, bool ONE_ROW>
__global__ __launch_bounds__(1024) void k_dec_down_combine(
    const uint8_t* __restrict__ experts, size_t stride, const uint8_t* __restrict__ shared,
    ProjDesc pd, const int32_t* __restrict__ slots, int max_slots,
    const uint16_t* __restrict__ hs, const uint8_t* __restrict__ hsum, int K, int N, int Mmax,
    float cd, Unpack2K uk, int T, int k, int n_shared, const int32_t* __restrict__ inv_row,
    const float* __restrict__ topk_w, const uint16_t* __restrict__ x, int residual,
    uint16_t* __restrict__ out, const uint8_t* __restrict__ alt_experts, size_t alt_stride,
    ProjDesc pda) {
  extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
  const int nwaves = blockDim.x >> 6;
  const int tid = threadIdx.x, lane = tid & 63, q = lane >> 4, r = lane & 15;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nt = blockIdx.x;
  const int rows_total = T * k + T * n_shared;
  constexpr int WB = ONE_ROW ? one_wave_bytes(KBW) : ring_wave_bytes(kDecMaxRows);
  float* ylds = reinterpret_cast<float*>(lds + nwaves * WB);  // [rows][16]
  int* s_inv = reinterpret_cast<int*>(ylds + rows_total * 16);
  float* s_w = reinterpret_cast<float*>(s_inv + kDecodeMaxRoutedRows);
  // the combine's inputs, loaded first (they are long complete when used)
  int my_inv = 0;
  float my_w = 0.f, my_x = 0.f;
  if (tid < T * k) {
    my_inv = inv_row[tid];
    my_w = topk_w[tid];
  }
  if (tid < T * 16 && residual) my_x = bf16_to_f32(x[(size_t)(tid >> 4) * N + nt * 16 + (tid & 15)]);
  const int32_t* rec = slots + kSlotRec * (1 + (wave < max_slots ? wave : 0));
  const int e = rec[0], row0 = rec[1], M = wave < max_slots ? rec[2] : 0;
  if (M > 0) {
    // a slot whose record says so reads the second expert copy (same down family)
    const bool alt = rec[3] != 0;
    if (alt) pd = pda;
    const uint8_t* blob = e < 0 ? shared
                          : alt ? alt_experts + (size_t)e * alt_stride
                                : experts + (size_t)e * stride;
    const uint8_t* const code_base[2] = {blob + pd.off, blob + pd.off};
    const size_t plane1[2] = {pd.plane1, pd.plane1};
    const size_t scale_off[2] = {pd.scales, pd.scales};
    const int KB = K / 128;
    uint8_t* buf = lds + wave * WB;
    const int ntl[1] = {nt};
    constexpr int PRE = dec_pre(KBW);
    u32x2 wc[KBW][1];
    uint32_t wh[KBW][1];
    u32x2 ws[KBW][1];
    uint32_t wsb[KBW][1];
    const u32x4 bc = corr_b_operand(q == 0, cd);
    const Unpack2R ur = {uk.m0, uk.m1, uk.m2, lane_copy(uk.b0), lane_copy(uk.b1),
                         lane_copy(uk.b2)};
    f32x4 acc[1] = {f32x4{0.f, 0.f, 0.f, 0.f}};
    if constexpr (ONE_ROW) {
      if (KB < KBW)
        dec_pipeline_band<1, false, Q3, Q3, true, KBW, PRE, false>(
            acc, wc, wh, wsb, code_base, plane1, scale_off, ntl, KB, 0, KB, lane, buf, false, row0,
            0u, hs, hsum, K, bc, bc, ur);
      else
        dec_pipeline_band<1, false, Q3, Q3, true, KBW, PRE, true>(
            acc, wc, wh, wsb, code_base, plane1, scale_off, ntl, KB, 0, KB, lane, buf, false, row0,
            0u, hs, hsum, K, bc, bc, ur);
    } else {
      if (KB < KBW)
        dec_pipeline<1, false, Q3, Q3, true, KBW, PRE, 4, kDecMaxRows, false>(
            acc, wc, wh, ws, code_base, plane1, scale_off, ntl, KB, 0, KB, lane, buf, M, false,
            row0, 0u, hs, hsum, K, bc, bc, ur);
      else if (M == 1)
        dec_pipeline_bandr<1, false, Q3, Q3, true, KBW, PRE, 1, 1, true>(
            acc, wc, wh, wsb, code_base, plane1, scale_off, ntl, KB, 0, KB, lane, buf, M, false,
            row0, 0u, hs, hsum, K, bc, bc, ur);
      else if (M == 2)
        dec_pipeline_bandr<1, false, Q3, Q3, true, KBW, PRE, 2, 2, true>(
            acc, wc, wh, wsb, code_base, plane1, scale_off, ntl, KB, 0, KB, lane, buf, M, false,
            row0, 0u, hs, hsum, K, bc, bc, ur);
      else if (M <= 4)
        dec_pipeline_bandr<1, false, Q3, Q3, true, KBW, PRE, 4, 4, true>(
            acc, wc, wh, wsb, code_base, plane1, scale_off, ntl, KB, 0, KB, lane, buf, M, false,
            row0, 0u, hs, hsum, K, bc, bc, ur);
      else
        dec_pipeline<1, false, Q3, Q3, true, KBW, PRE, 4, kDecMaxRows, true>(
            acc, wc, wh, ws, code_base, plane1, scale_off, ntl, KB, 0, KB, lane, buf, M, false,
            row0, 0u, hs, hsum, K, bc, bc, ur);
    }
    // rows 4*(lane/16) + i, column lane % 16 -> y of permuted row row0 + row
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * (lane >> 4) + i;
      if (lane < 32 && row < M) ylds[(row0 + row) * 16 + r] = bf16_to_f32(f32_to_bf16(acc[0][i]));
    }
  }
  if (tid < T * k) {
    s_inv[tid] = my_inv;
    s_w[tid] = my_w;
  }
  __syncthreads();
  // weighted combine of this tile's 16 columns, one thread per (token, column)
  if (tid < T * 16) {
    const int t = tid >> 4, col = tid & 15;
    float a = my_x;
    for (int j = 0; j < k; ++j) a = fmaf(s_w[t * k + j], ylds[s_inv[t * k + j] * 16 + col], a);
    if (n_shared) a += ylds[(T * k + t) * 16 + col];
    out[(size_t)t * N + nt * 16 + col] = (uint16_t)f32_to_bf16(a);
  }
}

int launch_decode_route(const moe_layer* L, const uint16_t* x, int T, uint32_t flags,
                        moe_routing* R, uint8_t* ws, const DecodeWs& W, void* stream,
                        uint32_t mask);

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

// Launch shape of one projection: waves per block (split of the reduction
// dimension) and k-blocks per wave, each wave owning at most 16
// (stream, k-block) tiles, or 32 for single-token gate/up.
struct DecShape {
  int ksplit, kbw;
};

// Down launches for a single token split K over up to 16 waves of at most 4
// k-blocks; for several rows at most 8 waves of up to 8 k-blocks (a 16-wave
// block leaves 128 registers per lane, too few for 8 rows of 4 streams).
static DecShape dec_shape(bool gateup, int K, int Mmax) {
  const int KB = K / 128;
  // single-token gate/up over 17..32 k-blocks: two waves of up to 16 (fewer,
  // longer-lived waves; measured at d = 4096 against four waves of eight:
  // 15.1 against 15.7 us)
  if (gateup && Mmax == 1 && KB > 16 && KB <= 32) return {2, 16};
  const int cap = gateup || Mmax > 1 ? 8 : 4, kmax = gateup || Mmax > 1 ? 8 : 16;
  int ks = 4;
  while (ks < kmax && (KB + ks - 1) / ks > cap) ks *= 2;
  const int per = (KB + ks - 1) / ks;
  if (per > cap) return {0, 0};
  int kbw = 2;
  while (kbw < per) kbw *= 2;
  return {ks, kbw};
}

static size_t dec_lds_bytes(bool gateup, DecShape sh, int Mmax) {
  const size_t rows =
      (size_t)sh.ksplit * (Mmax == 1 ? one_wave_bytes(sh.kbw) : ring_wave_bytes(kDecMaxRows));
  const size_t red = (size_t)sh.ksplit * (gateup ? 2 : 4) * 4 * 32 * 4;
  return rows > red ? rows : red;
}

constexpr size_t kLdsLimit = 160 * 1024;

bool decode_shape_ok(const moe_layer* L, int T) {
  const int Mmax = T < kDecMaxRows ? T : kDecMaxRows;
  const DecShape gu = dec_shape(true, L->d, Mmax), dn = dec_shape(false, L->inter, Mmax);
  return gu.ksplit && dn.ksplit && dec_lds_bytes(true, gu, Mmax) <= kLdsLimit &&
         dec_lds_bytes(false, dn, Mmax) <= kLdsLimit;
}

// Fused down projection + combine: at most 16 slots (one wave each) and
// I <= 2048 (16 k-blocks per wave).
static int dc_waves(int T, int max_slots) {
  const int need = (T * 16 + 63) / 64;  // the combine's (token, column) threads
  return max_slots > need ? max_slots : need;
}

static int dc_kbw(int I) {
  const int KB = I / 128;
  int kbw = 2;
  while (kbw < KB) kbw *= 2;
  return kbw;
}

static size_t dc_lds_bytes(const moe_layer* L, int T, int max_slots, int Mmax) {
  const int waves = dc_waves(T, max_slots);
  const int rows = T * L->top_k + T * L->n_shared;
  const int kbw = dc_kbw(L->inter);
  return (size_t)waves * (Mmax == 1 ? one_wave_bytes(kbw) : ring_wave_bytes(kDecMaxRows)) +
         (size_t)rows * 16 * 4 +
         (size_t)kDecodeMaxRoutedRows * 8;
}

static bool dc_ok(const moe_layer* L, int T, int max_slots, int Mmax) {
  return max_slots <= 16 && L->inter <= 2048 && dc_lds_bytes(L, T, max_slots, Mmax) <= kLdsLimit;
}

template <bool GATEUP, bool QA3, bool QB3, bool SAMEC>
static int launch_proj(DecShape sh, int n_blocks, int Mmax, hipStream_t s, const moe_layer* L,
                       ProjDesc pa, ProjDesc pb, const int32_t* slots, const uint16_t* A,
                       const uint8_t* Asum, int K, int N, float ca, float cb, uint16_t* out,
                       float* psum, const DecRoute* route, int want_alt) {
  const size_t lds = dec_lds_bytes(GATEUP, sh, Mmax);
  const DecRoute ro = route ? *route : DecRoute{};
#define BQ_L(KS, KBW)                                                                         \
  do {                                                                                        \
    if (Mmax == 1 && route) {                                                                 \
      if constexpr (GATEUP)                                                                   \
        hipLaunchKernelGGL((k_dec_proj<GATEUP, QA3, QB3, SAMEC, KS, KBW, true, true>),        \
                           dim3(n_blocks), dim3(64 * KS), lds, s, (const uint8_t*)L->experts, \
                           L->expert_stride, (const uint8_t*)L->shared, pa, pb, slots, A,     \
                           Asum, K, N, Mmax, ca, cb, out, psum, kUnpack2, ro, want_alt);      \
    } else if (Mmax == 1)                                                                     \
      hipLaunchKernelGGL((k_dec_proj<GATEUP, QA3, QB3, SAMEC, KS, KBW, true>), dim3(n_blocks), \
                         dim3(64 * KS), lds, s, (const uint8_t*)L->experts, L->expert_stride, \
                         (const uint8_t*)L->shared, pa, pb, slots, A, Asum, K, N, Mmax, ca,   \
                         cb, out, psum, kUnpack2, ro, want_alt);                              \
    else if constexpr (KS >= 4 && KS < 16)                                                               \
      hipLaunchKernelGGL((k_dec_proj<GATEUP, QA3, QB3, SAMEC, KS, KBW, false>),               \
                         dim3(n_blocks), dim3(64 * KS), lds, s, (const uint8_t*)L->experts,   \
                         L->expert_stride, (const uint8_t*)L->shared, pa, pb, slots, A, Asum, \
                         K, N, Mmax, ca, cb, out, psum, kUnpack2, ro, want_alt);              \
    else                                                                                      \
      return -1;                                                                              \
  } while (0)
  if (sh.ksplit == 4 && sh.kbw == 2)
    BQ_L(4, 2);
  else if (sh.ksplit == 4 && sh.kbw == 4)
    BQ_L(4, 4);
  else if constexpr (GATEUP) {
    if (sh.ksplit == 4 && sh.kbw == 8)
      BQ_L(4, 8);
    else if (sh.ksplit == 8 && sh.kbw == 8)
      BQ_L(8, 8);
    else if (sh.ksplit == 2 && sh.kbw == 16)
      BQ_L(2, 16);
    else
      return -1;
  } else {
    if (sh.ksplit == 8 && sh.kbw == 4)
      BQ_L(8, 4);
    else if (sh.ksplit == 4 && sh.kbw == 8)
      BQ_L(4, 8);
    else if (sh.ksplit == 16 && sh.kbw == 4)
      BQ_L(16, 4);
    else if (sh.ksplit == 8 && sh.kbw == 8)
      BQ_L(8, 8);
    else
      return -1;
  }
#undef BQ_L
  return 0;
}

// Both copies in one launch (k_dec_proj_mixed); same launch shapes as launch_proj.
template <bool GATEUP, bool QA3, bool QB3, bool SAMEC, bool XA3, bool XB3, bool XSAMEC>
static int launch_proj_mixed(DecShape sh, int n_blocks, int Mmax, hipStream_t s,
                             const moe_layer* L, ProjDesc pa, ProjDesc pb, ProjDesc xpa,
                             ProjDesc xpb, const int32_t* slots, const uint16_t* A,
                             const uint8_t* Asum, int K, int N, float ca, float cb, float xca,
                             float xcb, uint16_t* out, float* psum) {
  const size_t lds = dec_lds_bytes(GATEUP, sh, Mmax);
  const uint8_t* ex = (const uint8_t*)L->experts;
  const uint8_t* ax = (const uint8_t*)L->alt_experts;
  const uint8_t* shb = (const uint8_t*)L->shared;
#define BQ_M(KS, KBW)                                                                          \
  do {                                                                                         \
    if (Mmax == 1)                                                                             \
      hipLaunchKernelGGL(                                                                      \
          (k_dec_proj_mixed<GATEUP, QA3, QB3, SAMEC, XA3, XB3, XSAMEC, KS, KBW, true>),        \
          dim3(n_blocks), dim3(64 * KS), lds, s, ex, L->expert_stride, shb, pa, pb, ax,        \
          L->alt_stride, xpa, xpb, slots, A, Asum, K, N, Mmax, ca, cb, xca, xcb, out, psum,    \
          kUnpack2);                                                                           \
    else if constexpr (KS >= 4 && KS < 16)                                                                \
      hipLaunchKernelGGL(                                                                      \
          (k_dec_proj_mixed<GATEUP, QA3, QB3, SAMEC, XA3, XB3, XSAMEC, KS, KBW, false>),       \
          dim3(n_blocks), dim3(64 * KS), lds, s, ex, L->expert_stride, shb, pa, pb, ax,        \
          L->alt_stride, xpa, xpb, slots, A, Asum, K, N, Mmax, ca, cb, xca, xcb, out, psum,    \
          kUnpack2);                                                                           \
    else                                                                                       \
      return -1;                                                                               \
  } while (0)
  if (sh.ksplit == 4 && sh.kbw == 2)
    BQ_M(4, 2);
  else if (sh.ksplit == 4 && sh.kbw == 4)
    BQ_M(4, 4);
  else if constexpr (GATEUP) {
    if (sh.ksplit == 4 && sh.kbw == 8)
      BQ_M(4, 8);
    else if (sh.ksplit == 8 && sh.kbw == 8)
      BQ_M(8, 8);
    else if (sh.ksplit == 2 && sh.kbw == 16)
      BQ_M(2, 16);
    else
      return -1;
  } else {
    if (sh.ksplit == 8 && sh.kbw == 4)
      BQ_M(8, 4);
    else if (sh.ksplit == 4 && sh.kbw == 8)
      BQ_M(4, 8);
    else if (sh.ksplit == 16 && sh.kbw == 4)
      BQ_M(16, 4);
    else if (sh.ksplit == 8 && sh.kbw == 8)
      BQ_M(8, 8);
    else
      return -1;
  }
#undef BQ_M
  return 0;
}

// Single-token gate/up makes the expert selection itself (see
// dec_select_one_token) for up to 256 experts; a call that runs the gate/up
// stage then skips the select kernel.
static bool select_in_gateup(const moe_layer* L, int T) {
  return T == 1 && L->n_experts <= 256 && L->top_k <= 64;
}

// The second expert copy of L as a layer of its own (its blobs and code
// families; the rest of L unchanged).
static moe_layer alt_view(const moe_layer* L) {
  moe_layer A = *L;
  A.experts = L->alt_experts;
  A.expert_stride = L->alt_stride;
  A.q_gate = L->q_alt_gate;
  A.q_up = L->q_alt_up;
  A.q_down = L->q_alt_down;
  return A;
}

// Gate/up of the slots of one expert copy (want_alt as in k_dec_proj).
static int launch_gateup(const moe_layer* L, DecShape sh, int nb, int Mmax, hipStream_t s,
                         const int32_t* slots, const uint16_t* xs, const uint8_t* xsum,
                         uint16_t* hs, float* hsum, const DecRoute* rp, int want_alt) {
  const int d = L->d, I = L->inter;
  const ProjDesc pg = proj(L, 0), pu = proj(L, 1);
  const float cg = qtype_offset(L->q_gate), cu = qtype_offset(L->q_up);
  const bool g3 = L->q_gate == MOE_Q_INT3, u3 = L->q_up == MOE_Q_INT3;
  const bool same = L->q_gate == L->q_up;
#define BQ_GU(A3, B3, SC)                                                                       \
  return launch_proj<true, A3, B3, SC>(sh, nb, Mmax, s, L, pg, pu, slots, xs, xsum, d, I, cg, \
                                       cu, hs, hsum, rp, want_alt)
  if (g3 && u3) BQ_GU(true, true, true);
  if (g3) BQ_GU(true, false, false);
  if (u3) BQ_GU(false, true, false);
  if (same) BQ_GU(false, false, true);
  BQ_GU(false, false, false);
#undef BQ_GU
}

int launch_decode(const moe_layer* L, const uint16_t* x, int T, uint32_t flags, moe_routing* R,
                  uint8_t* ws, const DecodeWs& W, uint16_t* out, void* stream, uint32_t mask) {
  // with a second expert copy the selection stays in the select kernel, whose
  // slot records say which copy each slot reads
  const bool has_alt = L->alt_experts != nullptr;
  const bool fused_select = select_in_gateup(L, T) && (mask & MOE_DECODE_STAGE_GATEUP) && !has_alt;
  int rc = launch_decode_route(L, x, T, flags, R, ws, W, stream,
                               fused_select ? mask & ~(uint32_t)MOE_DECODE_STAGE_SELECT : mask);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)stream;
  const int k = L->top_k, d = L->d, I = L->inter;
  const int Mmax = T < kDecMaxRows ? T : kDecMaxRows;
  const int32_t* slots = (const int32_t*)(ws + W.slots);
  const uint16_t* xs = (const uint16_t*)(ws + W.xs);
  const uint8_t* xsum = ws + W.xsum;
  uint16_t* hs = (uint16_t*)(ws + W.hs);
  float* hsum = (float*)(ws + W.hsum);
  uint16_t* y = (uint16_t*)(ws + W.y);
  const moe_layer La = has_alt ? alt_view(L) : *L;
  if (mask & MOE_DECODE_STAGE_GATEUP) {
    const DecShape sh = dec_shape(true, d, Mmax);
    const int nb = W.max_slots * (I / 16);
    const DecRoute route = {R->logits,   L->n_experts, k,         L->n_shared, W.max_slots,
                            R->topk_ids, R->topk_w,    R->counts, R->offsets,  R->perm_tok,
                            R->inv_row,  (int32_t*)(ws + W.slots)};
    const DecRoute* rp = fused_select ? &route : nullptr;
    if (has_alt && L->q_gate == L->q_up && La.q_gate == La.q_up) {
      // both copies in one launch (gate and up share a family within each copy)
      const bool m3 = L->q_gate == MOE_Q_INT3, a3 = La.q_gate == MOE_Q_INT3;
      const ProjDesc pg = proj(L, 0), pu = proj(L, 1), xg = proj(&La, 0), xu = proj(&La, 1);
      const float cm = qtype_offset(L->q_gate), ca = qtype_offset(La.q_gate);
#define BQ_GM(M3, A3)                                                                          \
  rc = launch_proj_mixed<true, M3, M3, true, A3, A3, true>(sh, nb, Mmax, s, L, pg, pu, xg, xu, \
                                                           slots, xs, xsum, d, I, cm, cm, ca,  \
                                                           ca, hs, hsum)
      if (m3 && a3)
        BQ_GM(true, true);
      else if (m3)
        BQ_GM(true, false);
      else if (a3)
        BQ_GM(false, true);
      else
        BQ_GM(false, false);
#undef BQ_GM
      if (rc) return rc;
    } else {
      rc = launch_gateup(L, sh, nb, Mmax, s, slots, xs, xsum, hs, hsum, rp, has_alt ? 0 : -1);
      if (rc) return rc;
      if (has_alt) {
        rc = launch_gateup(&La, sh, nb, Mmax, s, slots, xs, xsum, hs, hsum, nullptr, 1);
        if (rc) return rc;
      }
    }
  }
  // the fused down + combine takes both copies when their down families agree
  const bool fused_down = dc_ok(L, T, W.max_slots, Mmax) && (!has_alt || La.q_down == L->q_down);
  if ((mask & MOE_DECODE_STAGE_DOWN) && fused_down) {
    const ProjDesc pd = proj(L, 2), pda = proj(&La, 2);
    const int waves = dc_waves(T, W.max_slots), kbw = dc_kbw(I);
    const size_t lds = dc_lds_bytes(L, T, W.max_slots, Mmax);
    const float cd = qtype_offset(L->q_down);
    const uint8_t* hsb = (const uint8_t*)hsum;
    const int res = (flags & MOE_ADD_RESIDUAL) ? 1 : 0;
    const uint8_t* alt_ex = (const uint8_t*)L->alt_experts;
#define BQ_DC(Q3, KBW)                                                                         \
  do {                                                                                         \
    if (Mmax == 1)                                                                             \
      hipLaunchKernelGGL((k_dec_down_combine<Q3, KBW, true>), dim3(d / 16), dim3(64 * waves),  \
                         lds, s, (const uint8_t*)L->experts, L->expert_stride,                 \
                         (const uint8_t*)L->shared, pd, slots, W.max_slots, hs, hsb, I, d,     \
                         Mmax, cd, kUnpack2, T, k, L->n_shared, R->inv_row, R->topk_w, x, res, \
                         out, alt_ex, L->alt_stride, pda);                                     \
    else                                                                                       \
      hipLaunchKernelGGL((k_dec_down_combine<Q3, KBW, false>), dim3(d / 16), dim3(64 * waves), \
                         lds, s, (const uint8_t*)L->experts, L->expert_stride,                 \
                         (const uint8_t*)L->shared, pd, slots, W.max_slots, hs, hsb, I, d,     \
                         Mmax, cd, kUnpack2, T, k, L->n_shared, R->inv_row, R->topk_w, x, res, \
                         out, alt_ex, L->alt_stride, pda);                                     \
  } while (0)
#define BQ_DCQ(Q3)        \
  do {                    \
    if (kbw == 2)         \
      BQ_DC(Q3, 2);       \
    else if (kbw == 4)    \
      BQ_DC(Q3, 4);       \
    else if (kbw == 8)    \
      BQ_DC(Q3, 8);       \
    else                  \
      BQ_DC(Q3, 16);      \
  } while (0)
    if (L->q_down == MOE_Q_INT3)
      BQ_DCQ(true);
    else
      BQ_DCQ(false);
#undef BQ_DCQ
#undef BQ_DC
  } else if (mask & MOE_DECODE_STAGE_DOWN) {
    const DecShape sh = dec_shape(false, I, Mmax);
    const int nb = W.max_slots * (d / 64);
    const uint8_t* hsb = (const uint8_t*)hsum;
    if (has_alt) {
      // both copies in one launch
      const bool m3 = L->q_down == MOE_Q_INT3, a3 = La.q_down == MOE_Q_INT3;
      const ProjDesc pd = proj(L, 2), xpd = proj(&La, 2);
      const float cd = qtype_offset(L->q_down), xcd = qtype_offset(La.q_down);
#define BQ_DM(M3, A3)                                                                          \
  rc = launch_proj_mixed<false, M3, M3, true, A3, A3, true>(sh, nb, Mmax, s, L, pd, pd, xpd,   \
                                                            xpd, slots, hs, hsb, I, d, cd, cd, \
                                                            xcd, xcd, y, nullptr)
      if (m3 && a3)
        BQ_DM(true, true);
      else if (m3)
        BQ_DM(true, false);
      else if (a3)
        BQ_DM(false, true);
      else
        BQ_DM(false, false);
#undef BQ_DM
      if (rc) return rc;
    } else {
      const ProjDesc pd = proj(L, 2);
      const float cd = qtype_offset(L->q_down);
      if (L->q_down == MOE_Q_INT3)
        rc = launch_proj<false, true, true, true>(sh, nb, Mmax, s, L, pd, pd, slots, hs, hsb, I,
                                                  d, cd, cd, y, nullptr, nullptr, -1);
      else
        rc = launch_proj<false, false, false, true>(sh, nb, Mmax, s, L, pd, pd, slots, hs, hsb,
                                                    I, d, cd, cd, y, nullptr, nullptr, -1);
      if (rc) return rc;
    }
    rc = launch_combine(y, T, d, k, L->n_shared, R->inv_row, R->topk_w, x,
                        (flags & MOE_ADD_RESIDUAL) ? 1 : 0, out, stream);
    if (rc) return rc;
  }
  return (int)hipGetLastError();
}

}  // namespace bqmoe
