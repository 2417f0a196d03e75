// Prefill for layers whose three projections hold 2-bit codes, on fp16
// matrix-core terms with a small correction on the scaled fp6 x fp4 ops of
// gfx950.  (Code families: the "Xolotl" README's "Quick start"; the value of
// a code is scale * (u - 1.5), see include/moe.h.)
//
// The bf16-operand kernel keeps the weights exact by multiplying every
// 32-group's partial sums by the group's fp16 scale in fp32: one vector FMA
// per output element per group, as much vector work as the matrix core's.
// Here the scale goes into the operand instead.  A weight is s * c with
// c = u - 1.5 in {+-0.5, +-1.5}; the operand is the fp16 value
//   v(u) = fp16(s * c / 2)  (round to nearest even; halved so that no finite
//                            fp16 scale overflows),
// exact for c = +-0.5 (unless |s| < 2^-12, where s/4 itself is rounded), and
// for c = +-1.5 off by r = 0.75 s - fp16(0.75 s), which is 0 or a signed power
// of two (0.75 s has at most 13 significant bits, fp16 keeps 11).  So
//   x . W[:, n] = 2 * ( sum_k x_k v(u_k)  +  sum_g r_g * sum_{k in g} x_k tau_k )
// with tau = +1 for u = 3, -1 for u = 0 and 0 otherwise.  The first sum is an
// fp16 matrix-core product accumulated over the whole of K (activations as
// fp16 rows scaled by a power of two per row, as for ternary layers).  The
// second, 2^-11 of the first at most, runs on the scaled 32x32x64 op with
// fp6 (e2m3) activations and one power-of-two scale per (row, 32-group), and
// fp4 (e2m1) tau/2 with the scale 2 |r_g| per (column, 32-group): both scales
// are exactly what that op applies per 32-element block.  fp6 activations
// carry a relative error of 2^-4, on a term 2^-11 of the sum: relL1 of an
// expert's output about 1.4e-4 against the exact layer (a per-group fp32 scale
// multiply gives about 1e-5; plain fp16 weights without the correction,
// 1e-3).
//
// Block: one 128-row tile of one expert and 8 waves (gate/up: wave w covers
// 32 columns of gate and the same of up; down: 64 columns), so a tile's
// activations are staged once per 256 (gate/up) or 512 (down) output
// columns.  Per 128-wide k-step the block loads the fp16 rows (32 KB) and
// their fp6 records (16 KB) into a ring of three LDS stages with
// direct-to-LDS buffer loads two steps ahead, and each wave its packed words
// and scales into registers one step ahead; each wave builds both weight
// operands in registers.  All-ternary layers of the same shapes run on the
// same kernel (TERN): exact operands s * (u - 1), no records, no correction.
#include <hip/hip_runtime.h>

#include <type_traits>

#include "device_common.h"
#include "tern_operand.h"
#include "moe_internal.h"

namespace bqmoe {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x6 __attribute__((ext_vector_type(6)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kRowsX = 128;                // rows per tile
constexpr int kRtX = kRowsX / 32;          // 32-row sub-tiles per tile
constexpr int kKbX = 128;                  // k per step (one packed tile along K)
constexpr int kA16X = kRowsX * kKbX * 2;   // fp16 rows of one k-step
constexpr int kA6X = kRowsX * 4 * 32;      // fp6 records of one k-step
constexpr int kWavesX = 8;
constexpr int kRowsPerWaveX = kRowsX / kWavesX;  // rows each wave loads
constexpr int kStagesX = 3;                // LDS ring depth (k-steps in flight: 2)
constexpr int kLdsX = kStagesX * (kA16X + kA6X);
constexpr int kDmaA16X = kA16X / 1024 / kWavesX;  // direct loads of fp16 rows per wave and k-step
constexpr int kDmaA6X = kA6X / 1024 / kWavesX;    // of records
constexpr int kDmaX = kDmaA16X + kDmaA6X;         // of activations
constexpr int kRecX = 32;                  // bytes per (row, 32-group) record
constexpr int kRsrcX = 0x00020000;         // buffer resource word 3: raw 32-bit dwords

// s_waitcnt immediate: vector-memory count vm (0..63), LDS/scalar count lgkm
// (0..15, 15 = no wait), export count not waited for
constexpr int waitcnt_vm_lgkm(int vm, int lgkm) {
  return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | ((vm >> 4) << 14);
}

// ------------------------------------------------------- activation records
// A (row, 32-group) record: 32 fp6 e2m3 codes (6 bits each, code j at bits
// 6j..6j+5 of bytes 0..23, little-endian), then the group's E8M0 scale byte
// (the codes' values times 2^(byte - 127) give the fp16 row's values), then
// 7 zero bytes.  Code j holds k-slot kslot(j) of the group: the order in
// which a lane of the scaled op holds its 32 fp4 weights (see tau_operand).
__host__ __device__ constexpr int x_kslot(int j) {
  return (j >> 3 == 0 ? 0 : j >> 3 == 1 ? 16 : j >> 3 == 2 ? 8 : 24) +
         ((j & 7) >> 1) + 4 * (j & 1);
}

// e2m3 code of |t| < 4, rounded to nearest even: the codes are monotone
// (0..7 = 0..7/8, then 8 + m = (1 + m/8) * 2^(E-1) per binade), so a carry
// out of a binade's mantissa lands on the next binade's first code.
__device__ __forceinline__ uint32_t e2m3_code(float t) {
  const float a = fabsf(t);
  uint32_t c;
  if (a < 1.f)
    c = (uint32_t)__builtin_rintf(a * 8.f);
  else if (a < 2.f)
    c = 8u + (uint32_t)__builtin_rintf((a - 1.f) * 8.f);
  else
    c = 16u + (uint32_t)__builtin_rintf((a - 2.f) * 4.f);
  return c | (t < 0.f ? 0x20u : 0u);
}

// One wave per row of bf16 values: e = (exponent of max|v|) - 14, in
// [-100, 114]; dst = fp16(v * 2^-e) (exact for the row's values down to 2^-31
// of its maximum), scale = 2^e, and per 32-group the record above, of the
// values w = v * 2^-e with the group's scale 2^(floor(log2 max|w|) - 1)
// (codes below 4).  src and dst may be the same rows: every element is read
// and rewritten by the same lane.  K is a multiple of 256.
//
// The second pass takes 8 consecutive values per lane (one 16-byte load and
// store), so a 32-group spans 4 lanes: its maximum by two lane exchanges.  A
// lane's 8 codes are record positions 8 jb .. 8 jb + 7, jb = (0, 2, 1, 3)[c]
// for its chunk c of the group, in the order of k-slots (0, 4, 1, 5, 2, 6,
// 3, 7) of the chunk (x_kslot); the group's chunk-0 lane gathers the four
// 48-bit pieces and stores the record with two 16-byte stores.
__global__ __launch_bounds__(256) void k_stage_x2(const uint16_t* src, int rows, int K,
                                                  uint16_t* dst, float* __restrict__ scale,
                                                  uint8_t* __restrict__ rec) {
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
  if (lane == 0) scale[row] = __uint_as_float((uint32_t)(127 + e) << 23);
  uint8_t* rrow = rec + (size_t)row * (K / 32) * kRecX;
  const int c = lane & 3;  // chunk of the lane's group
  for (int i = lane * 8; i < K; i += 512) {  // the lanes of a group take the same trips
    const uint4 v = *reinterpret_cast<const uint4*>(s + i);
    const uint32_t vw[4] = {v.x, v.y, v.z, v.w};
    float w[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      w[2 * j] = bf16_to_f32(vw[j] & 0xFFFFu) * f;
      w[2 * j + 1] = bf16_to_f32(vw[j] >> 16) * f;
    }
    uint4 o16;
    uint32_t* o16w = reinterpret_cast<uint32_t*>(&o16);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      o16w[j] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)w[2 * j]) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)w[2 * j + 1]) << 16);
    *reinterpret_cast<uint4*>(d + i) = o16;
    float gm = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) gm = fmaxf(gm, fabsf(w[j]));
    gm = fmaxf(gm, __shfl_xor(gm, 1, 4));
    gm = fmaxf(gm, __shfl_xor(gm, 2, 4));
    // group scale 2^ea with max|w| / 2^ea in [2, 4); a zero group gets 2^-126
    int ea = (int)((__float_as_uint(gm) >> 23) & 0xFF) - 127 - 1;
    ea = max(-126, min(126, ea));
    const float inv = __uint_as_float((uint32_t)(127 - ea) << 23);
    // the 8 codes in record order: k-slots 0, 4, 1, 5, 2, 6, 3, 7 of the chunk
    uint64_t piece = 0;
#pragma unroll
    for (int t = 0; t < 8; ++t)
      piece |= (uint64_t)e2m3_code(w[(t >> 1) + 4 * (t & 1)] * inv) << (6 * t);
    // record bytes 0..23 hold the pieces of chunks 0, 2, 1, 3 (jb = 0..3)
    const int base = lane & ~3;
    uint64_t pc[4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
      const int from = base + (jb == 1 ? 2 : jb == 2 ? 1 : jb);
      const uint32_t lo = (uint32_t)__shfl((int)(uint32_t)piece, from);
      const uint32_t hi = (uint32_t)__shfl((int)(uint32_t)(piece >> 32), from);
      pc[jb] = (uint64_t)lo | ((uint64_t)hi << 32);
    }
    if (c == 0) {
      uint4 r0, r1;
      r0.x = (uint32_t)pc[0];
      r0.y = (uint32_t)(pc[0] >> 32) | ((uint32_t)pc[1] << 16);
      r0.z = (uint32_t)(pc[1] >> 16);
      r0.w = (uint32_t)pc[2];
      r1.x = (uint32_t)(pc[2] >> 32) | ((uint32_t)pc[3] << 16);
      r1.y = (uint32_t)(pc[3] >> 16);
      r1.z = (uint32_t)(ea + 127);
      r1.w = 0u;
      uint8_t* rg = rrow + (size_t)(i / 32) * kRecX;
      *reinterpret_cast<uint4*>(rg) = r0;
      *reinterpret_cast<uint4*>(rg + 16) = r1;
    }
  }
}

// ------------------------------------------------------------ operand build
// fp16 pair v of the main operand of one (group parity P, k-half) of a lane:
// the levels of k-slots (2v, 2v+1) sit at bits (p, 16 + p) of the word,
// p = 8P + 2v.  After a shift by 8P they sit at 2v; a mask-and-or puts each
// into the fp16 value base + u, where base = 2^(10 - q) makes bit q of the
// field worth 1 (pair 0 is moved up to q = 2 first: at q = 0 the base would
// be 1024, and 1024 + 1.5 is not an fp16 value); one packed FMA gives
// (u - 1.5) / 2 exactly, one packed multiply by the scale rounds
// s * (u - 1.5) / 2 to nearest even.  The constants are kernel arguments; the
// bases are copied into vector registers once (see Unpack2R), so that each
// mask-and-or is a single v_and_or_b32 (a VOP3 op takes one scalar operand).
// Parity 1's pair 0 sits at bit 8, inside the fp16 mantissa as it is: under
// the base 2.0 the field is worth 1/2 per step, and one packed add of -2.75
// gives (u - 1.5) / 2, without the shift.  (Pairs 0 and 1 share a base.)
struct MainK {
  uint32_t msk[4], base[4], off[4];  // per pair: field mask, base bits, -(base/2 + 0.75)
  uint32_t msk8, base8, off8;        // parity 1's pair 0 in place: mask, base 2.0, -2.75
};

template <int P>
__device__ __forceinline__ u32x4 main_operand(uint32_t word, uint32_t s2, const MainK& mk) {
  const uint32_t x1 = P ? (word >> 8) : word;  // fields of pairs 0..3 at bits 0, 2, 4, 6
  u32x4 r;
#pragma unroll
  for (int v = 0; v < 4; ++v) {
    f16x2 c;
    if (P == 1 && v == 0) {
      const uint32_t fv = (word & mk.msk8) | mk.base8;
      c = __builtin_bit_cast(f16x2, fv) + __builtin_bit_cast(f16x2, mk.off8);
    } else {
      // pair 0 of parity 0 moves up to bit 2 (at bit 0 the offset would not
      // be an fp16 value)
      const uint32_t fv = ((v == 0 ? word << 2 : x1) & mk.msk[v]) | mk.base[v == 0 ? 1 : v];
      c = __builtin_bit_cast(f16x2, fv) * __builtin_bit_cast(f16x2, 0x38003800u) +
          __builtin_bit_cast(f16x2, mk.off[v]);
    }
    r[v] = __builtin_bit_cast(uint32_t, c * __builtin_bit_cast(f16x2, s2));
  }
  return r;
}

// The fp4 operand tau/2 (u = 3: +0.5, code 1; u = 0: -0.5, code 9; else 0)
// of a lane's two words of one group pair (k-halves h = 0, 1), for the scaled
// 32x32x64 op covering both groups: lanes 0..31 end up with all 32 k-slots of
// the pair's first group (parity 0), lanes 32..63 with those of the second,
// in the order x_kslot (8 k-slots per register: the lane's own chunk of h = 0
// and h = 1, then its partner's, lanes l and l ^ 32 exchanging halves).
__device__ __forceinline__ uint32_t tau_fields(uint32_t w) {
  // per 2-bit field: bit 0 = (b0 == b1), bit 1 = (u == 0)
  const uint32_t a = w >> 1;
  const uint32_t eq = ((w ^ a) ^ 0x55555555u) & 0x55555555u;
  const uint32_t z = eq & (a ^ 0x55555555u);
  return eq | (z << 1);
}

__device__ __forceinline__ void tau_split(uint32_t w, uint32_t& g0, uint32_t& g1) {
  const uint32_t f = tau_fields(w);
  // fields 2m -> nibble m of ne, fields 2m+1 -> nibble m of no; code = eq | z << 3
  const uint32_t ne = (f & 0x11111111u) | ((f & 0x22222222u) << 2);
  const uint32_t no = ((f >> 2) & 0x11111111u) | (f & 0x88888888u);
  // parity-0 fields are nibbles 0, 1, 4, 5 of both; parity 1 nibbles 2, 3, 6, 7
  g0 = __builtin_amdgcn_perm(no, ne, 0x06040200u);
  g1 = __builtin_amdgcn_perm(no, ne, 0x07050301u);
}

// (from the two words' splits a0, b0 and a1, b1)
__device__ __forceinline__ i32x8 tau_operand(uint32_t a0, uint32_t b0, uint32_t a1, uint32_t b1,
                                             uint32_t sgn, uint32_t keep) {
  const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
  const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
  i32x8 r;
  r[0] = (int)((s0[0] ^ sgn) & keep);
  r[1] = (int)((s1[0] ^ sgn) & keep);
  r[2] = (int)((s0[1] ^ sgn) & keep);
  r[3] = (int)((s1[1] ^ sgn) & keep);
  r[4] = r[5] = r[6] = r[7] = 0;
  return r;
}

// The correction of one (column, 32-group) in the halved units of the main
// product (operand fp16(s c / 2)): r = 0.75 s - fp16(0.75 s), 0 or +-2^j, times
// tau.  The fp4 operand holds tau / 2, so the op's column scale is 2|r|:
// returns its E8M0 byte, the mask that flips the operand's sign bits when
// r < 0, and the mask that clears the operand when r == 0 (E8M0 has no zero).
__device__ __forceinline__ void corr_scale(uint32_t s16, uint32_t& e8, uint32_t& sgn,
                                           uint32_t& keep) {
  const float t = f16_to_f32(s16) * 0.75f;
  const float r = t - (float)(_Float16)t;
  const uint32_t b = __float_as_uint(r);
  e8 = ((b >> 23) & 0xFFu) + 1u;  // 2|r|: the operand holds tau / 2
  sgn = (b >> 31) ? 0x88888888u : 0u;
  keep = r != 0.f ? 0xFFFFFFFFu : 0u;
  // the mask as a register (an empty statement), so that each operand
  // register takes one three-input bit op instead of a bit op and a select
  __asm__("" : "+v"(keep));
}

__device__ __forceinline__ f32x16 mfma_f16x(u32x4 a, u32x4 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a),
                                                __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
}

// SiLU with the hardware exp2 and reciprocal (h is rounded to bf16 right after)
__device__ __forceinline__ float silu_x(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(-1.4426950408889634f * g));
}

// ------------------------------------------------------------- grouped GEMM
// NMAT = 2: gate (column tile 0) and up (column tile 1) of 32 columns per
// wave; NMAT = 1: down (two column tiles of 32).  A16: fp16 rows (gather: tile
// row -> token through perm_tok), rscale: 2^e of each row, A6: their records.
//
// Two waves per SIMD: each wave holds the 4 x 2 accumulator tiles of the
// tile's 128 rows and its 64 columns (128 registers), so that a weight operand
// built in registers feeds 4 matrix-core ops, and a block covers 512 columns:
// the activations staged once serve 128 x 512 outputs.  The tile shape is set
// by the L2 -> CU traffic per flop (about 4 bytes per thousand flops here,
// and a vector-memory instruction per 7 matrix-core ops): with 256-row tiles
// of 256 columns the traffic is half as large again and the L2, which the
// activations are read from once per column group, becomes the bound.
//
// TERN: the same GEMM on an all-ternary layer, whose operands s * (u - 1)
// are exact in fp16 (build_tern): no records, no correction ops, and the
// product is the weight itself (no factor 2 in the epilogue).
template <int NMAT, bool TERN = false>
__global__ __launch_bounds__(64 * kWavesX, 1) void k_pfx(
    const uint8_t* __restrict__ experts, size_t stride, const uint8_t* __restrict__ shared,
    ProjDesc pa, ProjDesc pb, const int32_t* __restrict__ tiles, const int32_t* __restrict__ ctrl,
    const int32_t* __restrict__ perm_tok, int Tk, int gather, const uint16_t* __restrict__ A16,
    const float* __restrict__ rscale, const uint8_t* __restrict__ A6, int K, int N,
    uint16_t* __restrict__ out, int ncol, MainK mk, TernK tk) {
  extern __shared__ __attribute__((aligned(16))) uint8_t sbuf[];  // kLdsX
  constexpr int kDma = TERN ? kDmaA16X : kDmaX;  // direct loads per wave and k-step

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
  const int S = K / kKbX, G = K / 32;
  // 32-row sub-tiles computed: those holding real rows
  const int nrt = __builtin_amdgcn_readfirstlane((M + 31) >> 5);

  // source row of each tile row; padding rows repeat the first row (never
  // stored).  Kept in ring stage 2 of the activations, which the first loads
  // leave alone (the k-loop's first barrier orders its reuse).
  int* const sTok = reinterpret_cast<int*>(sbuf + 2 * kA16X);
  const int my_src = [&] {
    const int row = row0 + (tid < M ? tid : 0);
    return gather ? (row < Tk ? perm_tok[row] : row - Tk) : row;
  }();
  if (tid < kRowsX) sTok[tid] = my_src;
  __syncthreads();
  // LDS, per ring stage b: the fp16 rows at b * kA16X, row R at R * 256, its
  // 16-byte chunk c (8 k) in slot c ^ (R % 16); the records at
  // 3 * kA16X + b * kA6X, row R at R * 128, the 16-byte half hf of its group g
  // (t = 2g + hf) in slot t ^ ((R / 2) % 8).  A direct-to-LDS load writes 16
  // bytes per lane at consecutive slots, so 16 lanes fill one row's 256 bytes
  // (8 lanes one row's 128 bytes of records) from 2 (1) cache lines; the slot
  // swizzles keep the matrix-core reads (16 rows, one chunk) free of bank
  // conflicts.  Wave w loads rows 16w .. 16w + 15 of both.
  //
  // All global reads of the loop are buffer loads: the compiler's memory
  // counter bookkeeping keeps them in issue order (with the flat-address
  // direct-to-LDS loads it waits for all of them at every use), so that the
  // wait for one step leaves the next step's loads in flight.  Byte offsets
  // are 32-bit (the host bounds the activation arrays).
  const __amdgpu_buffer_rsrc_t rA = __builtin_amdgcn_make_buffer_rsrc((void*)A16, 0, -1, kRsrcX);
  const __amdgpu_buffer_rsrc_t rR = __builtin_amdgcn_make_buffer_rsrc((void*)A6, 0, -1, kRsrcX);
  static_assert(kRowsPerWaveX == 4 * kDmaA16X && kRowsPerWaveX == 8 * kDmaA6X, "row split");
  uint32_t aoffs[kDmaA16X], roffs[kDmaA6X];
#pragma unroll
  for (int i = 0; i < kDmaA16X; ++i) {
    const int R = kRowsPerWaveX * wave + 4 * i + (lane >> 4);
    aoffs[i] = (uint32_t)sTok[R] * (uint32_t)(2 * K) + (((lane & 15) ^ (R & 15)) << 4);
  }
#pragma unroll
  for (int i = 0; i < kDmaA6X; ++i) {
    const int R = kRowsPerWaveX * wave + 8 * i + (lane >> 3);
    roffs[i] = (uint32_t)sTok[R] * (uint32_t)(G * kRecX) + (((lane & 7) ^ ((R >> 1) & 7)) << 4);
  }
  // matrix-core reads: fp16 chunk c = 4 GB + 2h + hl (group GB of the k-step)
  // of row rt * 32 + l32 at l32 * 256 + (((4 GB + 2h) ^ ya) << 4) + rt * 8192;
  // record half hf of group 2 gp + hl of that row at
  // l32 * 128 + (((4 gp + hf) ^ zr) << 4) + rt * 4096
  // (the lane's parts: the XOR terms occupy bits 4..7, which no other term
  // of an address touches, so a step's base takes them once and each read
  // XORs in its chunk)
  const uint32_t la16 = (uint32_t)(l32 * 256) | ((uint32_t)(hl ^ (l32 & 15)) << 4);
  const uint32_t lr16 =
      (uint32_t)(kStagesX * kA16X + l32 * 128) | ((uint32_t)((2 * hl) ^ ((l32 >> 1) & 7)) << 4);

  MainK mv = mk;
  TernK tv = tk;
  if constexpr (TERN) {
#pragma unroll
    for (int D = 0; D < 4; ++D) tv.base[D] = lane_copy(tk.base[D]);
    tv.base8 = lane_copy(tk.base8);
  } else {
#pragma unroll
    for (int v = 1; v < 4; ++v) mv.base[v] = lane_copy(mk.base[v]);
    mv.base8 = lane_copy(mk.base8);
  }

  const int cw = col * kWavesX + wave;
  const int KT = K / 128;  // packed tiles along K
  // packed weights, one buffer over the expert: the lane's two code words of
  // column tile ct and k-half h at wu[ct] + 256 h + wl and its column's four
  // scales at su[ct] + sl, plus 512 (resp. 128) per tile along K; the parts
  // wu, su are the same for the whole wave (scalar offsets), wl, sl the
  // lane's (one vector register each)
  const __amdgpu_buffer_rsrc_t rB = __builtin_amdgcn_make_buffer_rsrc((void*)blob, 0, -1, kRsrcX);
  const uint32_t wl = (uint32_t)((l32 >> 4) * KT * 512 + (16 * hl + r) * 8);
  const uint32_t sl = (uint32_t)((l32 >> 4) * KT * 128 + r * 8);
  uint32_t wu[2], su[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const bool sec = NMAT == 2 && ct == 1;
    const uint32_t ntl = (uint32_t)(NMAT == 2 ? cw * 2 : cw * 4 + 2 * ct);
    wu[ct] = (uint32_t)(sec ? pb.off : pa.off) + ntl * KT * 512;
    su[ct] = (uint32_t)(sec ? pb.off + pb.scales : pa.off + pa.scales) + ntl * KT * 128;
  }

  f32x16 acc[kRtX][2];
#pragma unroll
  for (int rt = 0; rt < kRtX; ++rt)
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[rt][ct][i] = 0.f;

#define BQX_ISSUE(S_, BUF_)                                                                    \
  {                                                                                            \
    _Pragma("unroll") for (int i = 0; i < kDmaA16X; ++i)                                       \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                \
          rA, (lds_void*)(sbuf + (BUF_) * kA16X + (kDmaA16X * wave + i) * 1024), 16, aoffs[i], \
          (S_) * kKbX * 2, 0, 0);                                                              \
    _Pragma("unroll") for (int i = 0; i < (TERN ? 0 : kDmaA6X); ++i)                           \
      __builtin_amdgcn_raw_ptr_buffer_load_lds(                                                \
          rR, (lds_void*)(sbuf + kStagesX * kA16X + (BUF_) * kA6X + (kDmaA6X * wave + i) * 1024), \
          16, roffs[i], (S_) * 4 * kRecX, 0, 0);                                               \
  }
#define BQX_LOADB(S_, W_, SC_)                                                                 \
  {                                                                                            \
    _Pragma("unroll") for (int ct = 0; ct < 2; ++ct) {                                         \
      _Pragma("unroll") for (int h = 0; h < 2; ++h) W_[ct][h] =                                \
          __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(                      \
                                        rB, (int)wl, (int)(wu[ct] + 256 * h + (S_) * 512), 0)); \
      SC_[ct] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(                \
                                              rB, (int)sl, (int)(su[ct] + (S_) * 128), 0));    \
    }                                                                                          \
  }

  // The k-loop over k-steps of 128 (one packed tile along K) for NRT
  // computed 32-row sub-tiles (a compile-time count, so that the body is
  // straight-line code).  The activations and records go through a ring of
  // three LDS stages with direct-to-LDS loads two steps ahead; the packed
  // words and scales go into registers one step ahead.  Per step a wave issues
  // the words of step s + 1 and then the kDma direct loads of step s + 2; the
  // memory counter counts in issue order, so at the top of step s a wait down
  // to kDma outstanding loads leaves step s + 1's activations in flight.
  // Loads beyond the last step repeat it (in bounds, into a stage no wave
  // reads any more), so that the step has no branch.  Unrolled by two, the
  // words of step s sit in one register set while those of step s + 1 load
  // into the other.
  //
  // A step is two halves gp (groups 2gp, 2gp + 1), each software-pipelined
  // over its four sub-steps q = (group P, k-half h) and the correction: while
  // the matrix-core ops of one sub-step run, the wave reads the next
  // sub-step's activations from LDS and builds its weight operands
  // (scheduling groups interleave them); during q1 it also builds the half's
  // correction operands, and during q3 the next half's first weight operands.
  struct Ops {
    i32x8 b4[2];  // fp4 tau/2 operands of the correction, per column tile
    int sb[2];    // their E8M0 scales
  };
  typedef u32x2 Words[2][2];
  typedef u32x2 Scales[2];
  struct Split {
    uint32_t a0, b0, a1, b1;  // tau_split of the column tile's two words
  };
  // the correction operands of column tile ct in two parts (split, then
  // exchange, sign and scale), spread over the half's sub-steps
  auto corr_split = [&](auto gpc, auto ctc, const Words& w, Split& sp)
      __attribute__((always_inline)) {
    constexpr int gp = decltype(gpc)::value, ct = decltype(ctc)::value;
    tau_split(w[ct][0][gp], sp.a0, sp.b0);
    tau_split(w[ct][1][gp], sp.a1, sp.b1);
  };
  auto corr_finish = [&](auto gpc, auto ctc, const Scales& sc, const Split& sp, Ops& o)
      __attribute__((always_inline)) {
    constexpr int gp = decltype(gpc)::value, ct = decltype(ctc)::value;
    const uint32_t s16 = (sc[ct][gp] >> (16 * hl)) & 0xFFFFu;  // this lane's group is 2gp + hl
    uint32_t e8, sgn, keep;
    corr_scale(s16, e8, sgn, keep);
    o.b4[ct] = tau_operand(sp.a0, sp.b0, sp.a1, sp.b1, sgn, keep);
    o.sb[ct] = (int)e8;
  };
  auto bmain = [&](auto gpc, auto qc, const Words& w, const Scales& sc, u32x4 (&bm)[2])
      __attribute__((always_inline)) {
    constexpr int gp = decltype(gpc)::value;
    constexpr int P = decltype(qc)::value >> 1, h = decltype(qc)::value & 1;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const uint32_t sh = (sc[ct][gp] >> (16 * P)) & 0xFFFFu;
      if constexpr (TERN)
        bm[ct] = build_tern<P>(w[ct][h][gp], sh | (sh << 16), tv);
      else
        bm[ct] = main_operand<P>(w[ct][h][gp], sh | (sh << 16), mv);
    }
  };
  auto kloop = [&](auto nrt_c) {
  constexpr int NRT = decltype(nrt_c)::value;
  using G0 = std::integral_constant<int, 0>;
  using G1 = std::integral_constant<int, 1>;
  using Q0 = std::integral_constant<int, 0>;
  using Q1 = std::integral_constant<int, 1>;
  using Q2 = std::integral_constant<int, 2>;
  using Q3 = std::integral_constant<int, 3>;
  // interleave the region's 2 NRT matrix-core ops with V vector ops and D LDS reads each
  auto pattern = [&](auto vc, auto dc) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < 2 * NRT; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, decltype(vc)::value, 0);
      __builtin_amdgcn_sched_group_barrier(0x100, decltype(dc)::value, 0);
    }
  };
  // aS: the step's base of the lane's fp16 reads (la16 plus the stage);
  // c2 = 4 GB + 2h
  auto loadA = [&](const uint32_t aS, const uint32_t c2, u32x4 (&a)[kRtX])
      __attribute__((always_inline)) {
    const uint8_t* p = sbuf + (aS ^ (c2 << 4));
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt) a[rt] = *reinterpret_cast<const u32x4*>(p + rt * 8192);
  };
  auto mfmas = [&](const u32x4 (&a)[kRtX], const u32x4 (&bm)[2]) __attribute__((always_inline)) {
#pragma unroll
    for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) acc[rt][ct] = mfma_f16x(a[rt], bm[ct], acc[rt][ct]);
  };
  // half gp of a step: wc/sc its words, (wn, sn, gpn) those of the next half
  // (the same step's half 1, or the next step's half 0); bm0 and sp hold the
  // half's first weight operands and its code splits on entry, and the next
  // half's on exit.  A0 holds the first sub-step's activations on entry when
  // PRE; with NEXT the half reads the next half's (same stage) into it during
  // its correction ops.
  auto half = [&](auto gpc, auto gpnc, auto prec, auto nextc, const uint32_t sA,
                  const uint32_t sR, const Words& wc, const Scales& sc, const Words& wn,
                  const Scales& sn, u32x4 (&bm0)[2], Split (&sp)[2], u32x4 (&A0)[kRtX])
      __attribute__((always_inline)) {
    constexpr int gp = decltype(gpc)::value, gpn = decltype(gpnc)::value;
    u32x4 A1[kRtX], bmx[2], bmy[2];
    Ops oc;
    if constexpr (!decltype(prec)::value) {
      loadA(sA, 8 * gp, A0);
      __builtin_amdgcn_sched_barrier(0);
    }
    // q0 (P 0, h 0): read q1, build q1
    loadA(sA, 8 * gp + 2, A1);
    bmain(gpc, Q1{}, wc, sc, bmx);
    mfmas(A0, bm0);
    pattern(std::integral_constant<int, 4>{}, std::integral_constant<int, 1>{});
    __builtin_amdgcn_sched_barrier(0);
    // q1 (P 0, h 1): read q2, build q2 and column tile 0's correction operand
    loadA(sA, 8 * gp + 4, A0);
    bmain(gpc, Q2{}, wc, sc, bmy);
    if constexpr (!TERN) corr_finish(gpc, G0{}, sc, sp[0], oc);
    mfmas(A1, bmx);
    pattern(std::integral_constant<int, 6>{}, std::integral_constant<int, 1>{});
    __builtin_amdgcn_sched_barrier(0);
    // q2 (P 1, h 0): read q3, build q3 and column tile 1's correction operand
    loadA(sA, 8 * gp + 6, A1);
    bmain(gpc, Q3{}, wc, sc, bmx);
    if constexpr (!TERN) corr_finish(gpc, G1{}, sc, sp[1], oc);
    mfmas(A0, bmy);
    pattern(std::integral_constant<int, 6>{}, std::integral_constant<int, 1>{});
    __builtin_amdgcn_sched_barrier(0);
    // q3 (P 1, h 1): read the records (group 2 gp + hl of each sub-tile),
    // build the next half's first weight operands
    // (codes 0..15, codes 16..31 and the scale byte as three reads, so
    // that the codes land in one register tuple)
    i32x6 R6[kRtX];
    uint32_t RS[kRtX];
#pragma unroll
    for (int rt = 0; rt < (TERN ? 0 : NRT); ++rt) {
      const i32x4 c0 = *reinterpret_cast<const i32x4*>(sbuf + (sR ^ ((4u * gp) << 4)) + rt * 4096);
      const uint8_t* p1 = sbuf + (sR ^ ((4u * gp + 1) << 4)) + rt * 4096;
      const i32x2 c1 = *reinterpret_cast<const i32x2*>(p1);
      R6[rt] = __builtin_shufflevector(c0, __builtin_shufflevector(c1, c1, 0, 1, -1, -1), 0, 1, 2,
                                       3, 4, 5);
      RS[rt] = *reinterpret_cast<const uint32_t*>(p1 + 8);
    }
    bmain(gpnc, Q0{}, wn, sn, bm0);
    mfmas(A1, bmx);
    pattern(std::integral_constant<int, 4>{}, std::integral_constant<int, 2>{});
    __builtin_amdgcn_sched_barrier(0);
    // the correction; meanwhile the next half's code splits and, with NEXT,
    // its first activations
    if constexpr (decltype(nextc)::value) loadA(sA, 8 * gpn, A0);
    if constexpr (!TERN) {
      corr_split(gpnc, G0{}, wn, sp[0]);
      corr_split(gpnc, G1{}, wn, sp[1]);
    }
#pragma unroll
    for (int rt = 0; rt < (TERN ? 0 : NRT); ++rt) {
      const i32x8 a6 = __builtin_shufflevector(R6[rt], i32x6{0, 0, 0, 0, 0, 0}, 0, 1, 2, 3, 4, 5,
                                               6, 7);
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
        acc[rt][ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
            a6, oc.b4[ct], acc[rt][ct], 2, 4, 0, (int)RS[rt], 0, oc.sb[ct]);
    }
    pattern(std::integral_constant<int, 6>{}, std::integral_constant<int, 1>{});
    __builtin_amdgcn_sched_barrier(0);
  };
  Words wa, wb;
  Scales sa, sb2;
  u32x4 bm0[2], A0[kRtX];
  Split sp[2];
  using F = std::false_type;
  using T = std::true_type;
  BQX_ISSUE(0, 0)
  BQX_LOADB(0, wa, sa)
  BQX_ISSUE(min(1, S - 1), 1)
  bmain(G0{}, Q0{}, wa, sa, bm0);
  if constexpr (!TERN) {
    corr_split(G0{}, G0{}, wa, sp[0]);
    corr_split(G0{}, G1{}, wa, sp[1]);
  }
  int st = 0;  // ring stage of step s
  auto step = [&](const int s, const Words& cw_, const Scales& cs_, Words& nw_, Scales& ns_)
      __attribute__((always_inline)) {
    // k-step s is in LDS for every wave (the direct loads of step s + 1 may
    // remain in flight), and every wave is done reading the stage of step
    // s - 1, which the loads of step s + 2 overwrite: vmcnt(kDma)
    // lgkmcnt(0), then the barrier without a fence
    __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm(kDma, 0));
    __builtin_amdgcn_s_barrier();
    // the first sub-step's activations are read before the loads are
    // issued, so that the issue covers their latency
    const int st2 = st == 0 ? 2 : st - 1;  // (s + 2) % 3
    const uint32_t sA = la16 + (uint32_t)(st * kA16X);
    const uint32_t sR = lr16 + (uint32_t)(st * kA6X);
    loadA(sA, 0, A0);
    __builtin_amdgcn_sched_barrier(0);
    BQX_LOADB(min(s + 1, S - 1), nw_, ns_)
    BQX_ISSUE(min(s + 2, S - 1), st2)
    __builtin_amdgcn_sched_barrier(0);
    half(G0{}, G1{}, T{}, T{}, sA, sR, cw_, cs_, cw_, cs_, bm0, sp, A0);
    half(G1{}, G0{}, T{}, F{}, sA, sR, cw_, cs_, nw_, ns_, bm0, sp, A0);
    st = st == 2 ? 0 : st + 1;
  };
  for (int s = 0; s < S; s += 2) {  // S is even
    step(s, wa, sa, wb, sb2);
    step(s + 1, wb, sb2, wa, sa);
  }
  __builtin_amdgcn_s_waitcnt(waitcnt_vm_lgkm(0, 0));  // the repeated last loads have landed
  };
  switch (nrt) {
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    default: kloop(std::integral_constant<int, 4>{}); break;
  }
#undef BQX_ISSUE
#undef BQX_LOADB

  // the rows' activation scales, in LDS now free
  __syncthreads();
  float* const sScale = reinterpret_cast<float*>(sbuf);
  if (tid < kRowsX) sScale[tid] = rscale[my_src];
  __syncthreads();

  // acc[rt][ct][i] is row rt*32 + 8(i/4) + 4(lane/32) + i%4, column l32 of
  // column tile ct, in units of half the product (the operand was s c / 2);
  // the row's 2^e undoes the activation scale
#pragma unroll
  for (int rt = 0; rt < kRtX; ++rt)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int m = rt * 32 + 8 * (i >> 2) + 4 * hl + (i & 3);
      if (m < M) {
        const float sc = (TERN ? 1.0f : 2.0f) * sScale[m];
        if constexpr (NMAT == 2) {
          // gate and up of the same column of I: h = bf16(SiLU(g) * u)
          const float g = acc[rt][0][i] * sc, u = acc[rt][1][i] * sc;
          out[(size_t)(row0 + m) * N + cw * 32 + l32] = (uint16_t)f32_to_bf16(silu_x(g) * u);
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
bool prefill_x2_shape(const moe_layer* L) {
  return L->inter % (32 * kWavesX) == 0 && L->d % (64 * kWavesX) == 0;
}

bool prefill_x2(const moe_layer* L) {
  return L->q_gate == MOE_Q_INT2 && L->q_up == MOE_Q_INT2 && L->q_down == MOE_Q_INT2 &&
         prefill_x2_shape(L);
}

int prefill_x2_tile_rows() { return kRowsX;
}

// dynamic LDS above 64 KB, once per process, for every instantiation
static bool pfx_lds_attributes() {
  static bool attr_set = false;
  if (!attr_set) {
    const void* fns[4] = {(const void*)k_pfx<2>, (const void*)k_pfx<1>, (const void*)k_pfx<2, true>,
                          (const void*)k_pfx<1, true>};
    for (const void* f : fns)
      if (hipFuncSetAttribute(f, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsX) != hipSuccess)
        return false;
    attr_set = true;
  }
  return true;
}

static MainK main_constants() {
  // per pair v (field at bit q = 2, 2, 4, 6 after the shifts of main_operand):
  // the field's mask, the fp16 base 2^(10 - q) and -(base / 2 + 0.75), in both
  // halves: 256, 256, 64, 16 and -128.75, -128.75, -32.75, -8.75
  MainK k{};
  const uint32_t m[4] = {0x000C000Cu, 0x000C000Cu, 0x00300030u, 0x00C000C0u};
  const uint32_t b[4] = {0x5C005C00u, 0x5C005C00u, 0x54005400u, 0x4C004C00u};
  const uint32_t o[4] = {0xD806D806u, 0xD806D806u, 0xD018D018u, 0xC860C860u};
  for (int v = 0; v < 4; ++v) {
    k.msk[v] = m[v];
    k.base[v] = b[v];
    k.off[v] = o[v];
  }
  k.msk8 = 0x03000300u;  // parity 1's pair 0 at bits 8-9 of each half
  k.base8 = 0x40004000u;  // 2.0: the field adds u / 2
  k.off8 = 0xC180C180u;   // -2.75
  return k;
}

// The stages of a 2-bit layer after routing (x staging, gate/up, down).  The
// workspace areas hold: xs the fp16 rows of x, xsum their scales, x6 their
// records; h the bf16 h and then (by the end of the gate/up stage) its fp16
// rows, hsum their scales, h6 their records.
int launch_prefill_x2(const moe_layer* L, const uint16_t* x, int T, moe_routing* R, uint8_t* ws,
                      const PrefillWs& P, void* stream, uint32_t mask) {
  hipStream_t s = (hipStream_t)stream;
  const int k = L->top_k, d = L->d, I = L->inter;
  const int Tk = T * k;
  const int rows = Tk + (L->n_shared ? T : 0);
  uint16_t* xs = (uint16_t*)(ws + P.xs);
  float* xscale = (float*)(ws + P.xsum);
  uint8_t* x6 = ws + P.x6;
  uint16_t* hs = (uint16_t*)(ws + P.h);
  float* hscale = (float*)(ws + P.hsum);
  uint8_t* h6 = ws + P.h6;
  uint16_t* y = (uint16_t*)(ws + P.y);
  const int32_t* tiles = (const int32_t*)(ws + P.tiles);
  const int32_t* ctrl = (const int32_t*)(ws + P.ctrl);
  const uint8_t* experts = (const uint8_t*)L->experts;
  const uint8_t* shared = (const uint8_t*)L->shared;
  const PackedLayout lg = packed_layout(MOE_Q_INT2, d, I);
  const PackedLayout ld = packed_layout(MOE_Q_INT2, I, d);
  ProjDesc pg{}, pu{}, pdn{};
  pg.off = 0;
  pu.off = lg.total;
  pdn.off = 2 * lg.total;
  pg.scales = pu.scales = lg.scales;
  pdn.scales = ld.scales;
  pg.qtype = pu.qtype = pdn.qtype = MOE_Q_INT2;
  pg.K = pu.K = d;
  pg.N = pu.N = I;
  pdn.K = I;
  pdn.N = d;
  const MainK mk = main_constants();
  const size_t lds = (size_t)kLdsX;
  if (!pfx_lds_attributes()) return (int)hipErrorInvalidConfiguration;
  if (mask & MOE_PREFILL_STAGE_STAGE_X)
    hipLaunchKernelGGL(k_stage_x2, dim3((T + 3) / 4), dim3(256), 0, s, x, T, d, xs, xscale, x6);
  if (mask & MOE_PREFILL_STAGE_GATEUP) {
    const int ncol = I / (32 * kWavesX);
    const dim3 g1((unsigned)(((long)P.max_tiles * ncol + 7) / 8 * 8));
    hipLaunchKernelGGL(k_pfx<2>, g1, dim3(64 * kWavesX), lds, s, experts, L->expert_stride,
                       shared, pg, pu, tiles, ctrl, R->perm_tok, Tk, 1, xs, xscale, x6, d, I, hs,
                       ncol, mk, TernK{});
    // h to fp16 rows (in place) and records, within this stage, so that every
    // stage can be re-run
    hipLaunchKernelGGL(k_stage_x2, dim3((rows + 3) / 4), dim3(256), 0, s, hs, rows, I, hs,
                       hscale, h6);
  }
  if (mask & MOE_PREFILL_STAGE_DOWN) {
    const int ncol = d / (64 * kWavesX);
    const dim3 g2((unsigned)(((long)P.max_tiles * ncol + 7) / 8 * 8));
    hipLaunchKernelGGL(k_pfx<1>, g2, dim3(64 * kWavesX), lds, s, experts, L->expert_stride,
                       shared, pdn, pdn, tiles, ctrl, R->perm_tok, Tk, 0, hs, hscale, h6, I, d, y,
                       ncol, mk, TernK{});
  }
  return (int)hipGetLastError();
}

// The GEMMs of an all-ternary layer on this kernel (prefill_x2_shape): the
// staged fp16 rows of x (xs, xsum) or h (h, hsum) come from the ternary
// staging kernel; gate/up writes bf16 h, down the rows of y.
int launch_pfx_tern(const moe_layer* L, int T, moe_routing* R, uint8_t* ws, const PrefillWs& P,
                    void* stream, bool gateup) {
  hipStream_t s = (hipStream_t)stream;
  const int k = L->top_k, d = L->d, I = L->inter;
  const int Tk = T * k;
  if (!pfx_lds_attributes()) return (int)hipErrorInvalidConfiguration;
  const int32_t* tiles = (const int32_t*)(ws + P.tiles);
  const int32_t* ctrl = (const int32_t*)(ws + P.ctrl);
  const uint8_t* experts = (const uint8_t*)L->experts;
  const uint8_t* shared = (const uint8_t*)L->shared;
  const PackedLayout lg = packed_layout(MOE_Q_TERNARY, d, I);
  const PackedLayout ld = packed_layout(MOE_Q_TERNARY, I, d);
  ProjDesc pg{}, pu{}, pdn{};
  pg.off = 0;
  pu.off = lg.total;
  pdn.off = 2 * lg.total;
  pg.scales = pu.scales = lg.scales;
  pdn.scales = ld.scales;
  pg.qtype = pu.qtype = pdn.qtype = MOE_Q_TERNARY;
  pg.K = pu.K = d;
  pg.N = pu.N = I;
  pdn.K = I;
  pdn.N = d;
  const TernK tk = tern_constants();
  if (gateup) {
    const int ncol = I / (32 * kWavesX);
    const dim3 g1((unsigned)(((long)P.max_tiles * ncol + 7) / 8 * 8));
    hipLaunchKernelGGL((k_pfx<2, true>), g1, dim3(64 * kWavesX), kLdsX, s, experts,
                       L->expert_stride, shared, pg, pu, tiles, ctrl, R->perm_tok, Tk, 1,
                       (const uint16_t*)(ws + P.xs), (const float*)(ws + P.xsum), nullptr, d, I,
                       (uint16_t*)(ws + P.h), ncol, MainK{}, tk);
  } else {
    const int ncol = d / (64 * kWavesX);
    const dim3 g2((unsigned)(((long)P.max_tiles * ncol + 7) / 8 * 8));
    hipLaunchKernelGGL((k_pfx<1, true>), g2, dim3(64 * kWavesX), kLdsX, s, experts,
                       L->expert_stride, shared, pdn, pdn, tiles, ctrl, R->perm_tok, Tk, 0,
                       (const uint16_t*)(ws + P.h), (const float*)(ws + P.hsum), nullptr, I, d,
                       (uint16_t*)(ws + P.y), ncol, MainK{}, tk);
  }
  return (int)hipGetLastError();
}

}  // namespace bqmoe
