// Internal declarations shared by the host dispatch and the HIP kernels.
#pragma once
#include <cstddef>
#include <cstdint>

#include "../../include/moe.h"

namespace bqmoe {

inline int qtype_levels(int q) {
  return q == MOE_Q_TERNARY ? 3 : q == MOE_Q_INT2 ? 4 : q == MOE_Q_INT3 ? 8 : 0;
}
inline float qtype_offset(int q) {
  return q == MOE_Q_TERNARY ? 1.0f : q == MOE_Q_INT2 ? 1.5f : 3.5f;
}

// Byte offsets of the regions of one packed projection.
struct PackedLayout {
  size_t plane0, plane1, scales, total;
};
bool format_shape_ok(int qtype, int64_t K, int64_t N);
PackedLayout packed_layout(int qtype, int64_t K, int64_t N);

// One projection as the kernels see it: byte offset inside an expert blob plus
// the region offsets relative to the start of the projection.
struct ProjDesc {
  uint64_t off;      // from the start of the expert blob
  uint64_t plane1;   // relative to off (3-bit only)
  uint64_t scales;   // relative to off
  int32_t qtype;
  int32_t K, N;
};

// Operand encoding used by the kernels: a level u becomes an exact bf16 value
// base + 16u (base 2048, 512 or 128 by k-slot, see unpack2 / unpack3),
// activations are pre-scaled by 1/16, and the per-group term
// sum_k x_k * (base_k / 16 + offset) is removed by a second matrix-core op on
// staged sums (W = sum x_k * base_k / 16, S = sum x_k).
// Decode slot list: a 16-int header (n_slots first), then one 16-int record per
// slot: expert (-1 = shared), first permuted row, row count M, unused, and the
// token of each of the M rows.  All max_slots records are written; those past
// the last slot have M == 0.
constexpr int kSlotRec = 16;
constexpr int kSlotTok = 4;
constexpr int kDecodeMaxRoutedRows = 64;  // T*k for the decode path
constexpr int kDecodeMaxRows = 72;        // T*(k + n_shared) for the decode path
constexpr int kDecodeMaxDim = 8192;       // d and inter for the decode path

// Workspace layouts (byte offsets from the workspace base).
struct DecodeWs {
  size_t slots;     // int32 [16 * (1 + max_slots)]: header, then one record per slot
  size_t xs;        // bf16 [T][d]        x / 16
  size_t xsum;      // bf16 [T][d/32][8]  staged sums (W, S) of each 32-group of x
  size_t hs;        // bf16 [rows][I]     h / 16
  size_t hsum;      // fp32 [rows][I/16][2] (W, S) sums of h over each 16 columns
  size_t y;         // bf16 [rows][d]
  size_t total;
  int max_slots, rows;
};

struct PrefillWs {
  size_t hist;      // int32 [nblk][E]   per-block expert counts
  size_t lrank;     // int32 [T*k]       rank of each row among its block's rows of that expert
  size_t tiles;     // int32 [max_tiles][4] (expert|-1, row0, rows, 0) + int32 count (at ctrl)
  size_t ctrl;      // int32 [16] counters
  size_t xs;        // bf16 [T][d]        x / 16
  size_t xsum;      // bf16 [T][d/32][8]  staged sums (W, S) of each 32-group of x
  size_t h;         // bf16 [rows][I]     h / 16
  size_t hsum;      // bf16 [rows][I/32][8] staged sums of h
  size_t y;         // bf16 [rows][d]
  size_t x6;        // 2-bit layers: [T][d/32] 32-byte fp6 records of x's fp16 rows
  size_t h6;        // 2-bit layers: [rows][I/32] 32-byte fp6 records of h's fp16 rows
  size_t total;
  int nblk, max_tiles, rows;
};

constexpr int kHistTokensPerBlock = 256;  // tokens per histogram block
constexpr int kPrefillTileM = 64;         // rows per grouped-GEMM tile (bf16-operand path)

DecodeWs decode_ws_layout(const moe_layer* L, int T);
PrefillWs prefill_ws_layout(const moe_layer* L, int T);

// ---------------------------------------------------------------- launchers
// All return hipSuccess (0) or the launch error code.
int launch_route_generic(const moe_layer* L, const uint16_t* x, int T, uint32_t flags,
                         moe_routing* R, uint8_t* ws, const PrefillWs& P, void* stream);
// `mask` selects the kernels to enqueue (bit i = stage i, see moe.h); ~0u runs all.
// Whether the decode kernels take this layer for T tokens (LDS and register
// limits of their launch shapes).
bool decode_shape_ok(const moe_layer* L, int T);
int launch_decode(const moe_layer* L, const uint16_t* x, int T, uint32_t flags, moe_routing* R,
                  uint8_t* ws, const DecodeWs& W, uint16_t* out, void* stream, uint32_t mask);
int launch_prefill(const moe_layer* L, const uint16_t* x, int T, uint32_t flags, moe_routing* R,
                   uint8_t* ws, const PrefillWs& P, uint16_t* out, void* stream, uint32_t mask);
// Prefill on exact fp16 terms (all projections ternary): the stages after routing
// (x staging, gate/up, down), on 128-row tiles of the tile list.
bool prefill_exact16(const moe_layer* L);
int prefill_tile_rows(const moe_layer* L);
int launch_prefill16(const moe_layer* L, const uint16_t* x, int T, moe_routing* R, uint8_t* ws,
                     const PrefillWs& P, void* stream, uint32_t mask);
// Prefill of 2-bit layers on fp16 terms plus the fp6 x fp4 correction: the
// stages after routing, on 128-row tiles of the tile list.
bool prefill_x2(const moe_layer* L);
struct TernK;
TernK tern_constants();
// the 8-wave fp16-term GEMMs (prefill2x.hip) on an all-ternary layer, where
// its shape allows (prefill_x2_shape); gate/up (mask bit GATEUP) or down
int launch_pfx_tern(const moe_layer* L, int T, moe_routing* R, uint8_t* ws, const PrefillWs& P,
                    void* stream, bool gateup);
bool prefill_x2_shape(const moe_layer* L);
int prefill_x2_tile_rows();
int launch_prefill_x2(const moe_layer* L, const uint16_t* x, int T, moe_routing* R, uint8_t* ws,
                      const PrefillWs& P, void* stream, uint32_t mask);
// moe_forward_decode's validation and dispatch; with decode_ws_only the workspace need only
// hold decode_ws_layout(L, T) (the no-allocation entry point's fixed array).
moe_status decode_call(const moe_layer* L, const uint16_t* x, int32_t T, uint32_t flags,
                       moe_routing* R, void* ws, size_t ws_bytes, uint16_t* out, uint32_t mask,
                       void* stream, bool decode_ws_only);
// out[t] = bf16([x[t]] + sum_j w[t][j] * y[inv_row[t][j]] + [y[T*k + t]]) for all T tokens
int launch_combine(const uint16_t* y, int T, int d, int k, int n_shared, const int32_t* inv_row,
                   const float* w, const uint16_t* x, int residual, uint16_t* out, void* stream);

}  // namespace bqmoe
