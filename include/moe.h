/*
 * moe.h -- C ABI of libbqmoe.so, a quantized mixture-of-experts expert layer
 * for AMD Instinct MI355X (gfx950).
 *
 * What the layer computes.  The pages on the Xolotl engine ("Xolotl"
 * repository card, README section "How it works, in one paragraph") describe
 * the idea: a mixture-of-experts model runs only the few experts each token's
 * router asks for.  Their "Quick start" section names the expert weights'
 * code families (mixed ternary / 2-bit / 3-bit) and "Fast mode" says decode
 * speed is set by the expert bytes moved per token.  The pages give no
 * formula; this library's definition is:
 *
 *   logits[t][e] = fp32( sum_i x[t][i] * Wr[e][i] + bias[e] )
 *   ids[t][0..k)  = the k largest logits, descending, lower index first on ties
 *   w[t][j]       = softmax over the k selected logits (fp32, sums to 1)
 *   for each selected expert e and the shared expert (weight 1):
 *       h = bf16( SiLU(x.Wg_e) * (x.Wu_e) ),   y_e = bf16( h.Wd_e )
 *   out[t] = bf16( [x[t]] + sum_j w[t][j] * y_{ids[t][j]}[t] + y_shared[t] )
 *
 * Weights: W[k][n] = fp16 scale[n][k/32] * (level[n][k] - offset), with
 * ternary levels 0..2 (offset 1: values -1, 0, +1), 2-bit levels 0..3
 * (offset 1.5: -1.5 .. +1.5) and 3-bit levels 0..7 (offset 3.5: -3.5 .. +3.5).
 * Products and sums are fp32 on the GPU; h, y and out are rounded to bf16.
 *
 * Conventions for every call below
 *   - bf16 and fp16 values travel as uint16_t bit patterns.
 *   - Device pointers are HIP device addresses; the caller owns and allocates
 *     every buffer (inputs, outputs and the workspace).  The library allocates
 *     nothing, keeps no pointer after returning and has no mutable global
 *     state; calls are thread-safe.  The one exception is
 *     moe_forward_decode_noalloc, whose workspace is a static device array
 *     of the library (see its comment).
 *   - `stream` is a hipStream_t (NULL = the null stream).  Calls enqueue work
 *     on it and return without synchronising; argument errors are returned
 *     before anything is enqueued.  A failed launch returns MOE_ERR_DEVICE.
 *     Device faults surface at the caller's next synchronisation.
 *   - T == 0 is a no-op returning MOE_OK.
 *   - Results are deterministic: the same inputs give bitwise-identical
 *     outputs (no floating-point atomics).
 */
#ifndef BQMOE_MOE_H
#define BQMOE_MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, bad range, aliasing, misalignment */
  MOE_ERR_UNSUPPORTED = 2, /* shape outside what the kernels handle */
  MOE_ERR_WORKSPACE = 3,   /* workspace smaller than moe_workspace_bytes() */
  MOE_ERR_BAD_CODES = 4,   /* a level index outside its alphabet (moe_pack_weights) */
  MOE_ERR_DEVICE = 5       /* a HIP launch or runtime call failed */
} moe_status;

typedef enum { MOE_Q_TERNARY = 1, MOE_Q_INT2 = 2, MOE_Q_INT3 = 3 } moe_qtype;

enum {
  MOE_LOGITS_GIVEN = 1u, /* routing->logits is an input; the router matrix is not used */
  MOE_ADD_RESIDUAL = 2u  /* out = x + MoE(x) */
};

/* Limits of this implementation (anything else returns MOE_ERR_UNSUPPORTED). */
enum {
  MOE_MAX_EXPERTS = 1024,
  MOE_MAX_TOPK = 32,
  MOE_MAX_DECODE_TOKENS = 8,
  MOE_MAX_DIM = 65536 /* d and inter: multiples of 128 up to this */
};

/* ------------------------------------------------------------ packed format
 * Packed format v2 of one projection W[K][N] (K % 128 == 0, N % 16 == 0).
 * NT = N/16 n-tiles, KB = K/128 k-blocks.  For code (n, k): r = n%16,
 * kk = k%128, gb = kk/32, j = kk%32, q = j/8, s = j%8, lane chunk L = 16q + r.
 *   plane 0 (level & 3): tile (n/16, k/128) at ((n/16)*KB + k/128)*512 B;
 *     chunk L at L*8 holds two little-endian 32-bit words; the code sits in
 *     word gb/2 at bit 16*(s%2) + 2*(4*(gb%2) + s/2).
 *   plane 1 (3-bit only, level >> 2): from the next 256-B boundary, 256 B
 *     per tile, chunk L is one 32-bit word at L*4; with v = s/2 the bit is
 *     16*(s%2) + 2v + 2 + {0,1,6,7}[gb] for v < 3 and 16*(s%2) + {0,1,14,15}[gb]
 *     for v == 3 (v1 used 16*(s%2) + 4*gb + v).
 *   scales: from the next 256-B boundary, 128 B per (n-tile, k-block) block,
 *     fp16 scale[16*nt + r][4*kb + gb] at index r*4 + gb.
 *   The size is rounded up to a multiple of 256 B.
 * Each lane chunk of a tile is exactly what one lane of a 64-wide wavefront
 * needs for a 16 x 32 bf16 matrix-core operand, so a wave reads a tile as
 * one coalesced 512-B request.
 */

/* Bytes of one packed projection, or 0 if (qtype, K, N) is not supported. */
size_t moe_packed_bytes(int qtype, int64_t K, int64_t N);

/* Bytes of one packed expert: gate (K=d, N=inter), then up (same shape), then
 * down (K=inter, N=d), each starting at a 256-B aligned offset.  0 if invalid. */
size_t moe_expert_bytes(int q_gate, int q_up, int q_down, int64_t d, int64_t inter);

/* Pack one projection on the host.
 * Source: the "Xolotl" repository card, README "Quick start" ("Get a model"),
 * names the experts' code families (a mixed ternary / 2-bit / 3-bit
 * quantisation); the pages give no storage layout, so the packed format
 * above is this library's own, laid out for the matrix-core operands.
 *   codes  : host, [N][K] level indices (row n holds k = 0..K-1)
 *   scales : host, [N][K/32] fp16 bit patterns
 *   out    : host buffer of out_bytes >= moe_packed_bytes(qtype, K, N); the
 *            caller copies it to device memory.
 * Returns MOE_ERR_UNSUPPORTED for a bad shape or qtype, MOE_ERR_BAD_CODES if
 * a level is outside the alphabet (e.g. 3 in a ternary matrix), and
 * MOE_ERR_INVALID_ARG for null pointers or a short buffer. */
moe_status moe_pack_weights(int qtype, int64_t K, int64_t N, const uint8_t* codes,
                            const uint16_t* scales, void* out, size_t out_bytes);

/* Round-to-nearest quantisation of float weights into the code alphabet of
 * qtype, the input moe_pack_weights takes.  Per column n and 32-group g
 * along K, the scale is s = fp16(max |w| / cmax), rounded to nearest even,
 * where cmax = (levels - 1) - offset is the largest level magnitude (ternary
 * 1, int2 1.5, int3 3.5); each code is u = round-half-even(w / s + offset),
 * clamped to 0..levels-1 (u = round-half-even(offset) when s == 0).
 * Arithmetic in double.  The "Xolotl" README's "Quick start" names the code
 * families but no quantiser; this is the plain round-to-nearest route from
 * float weights onto them (the pages' calibrated quantiser is not
 * reproduced).
 *   w      : host, [N][K] fp32 (row n holds k = 0..K-1), finite
 *   codes  : host, [N][K] level indices (output)
 *   scales : host, [N][K/32] fp16 bit patterns (output)
 * Returns MOE_ERR_UNSUPPORTED for an unknown qtype or K % 32 != 0,
 * MOE_ERR_INVALID_ARG for null pointers, a non-finite weight, or a group
 * whose scale would exceed the largest fp16 value. */
moe_status moe_quantize_rtn(int qtype, int64_t K, int64_t N, const float* w, uint8_t* codes,
                            uint16_t* scales);

/* A packed projection in another code family: every weight of src (qtype
 * q_src) is decoded to s * (u - offset), exactly, and quantised to q_dst by
 * the rule of moe_quantize_rtn, then packed.  The "Xolotl" README's "Fast
 * mode" section describes keeping a lower-bit copy of the largest experts
 * and reading it instead of them when speed matters more than the last bit
 * of fidelity; with this call a 2-bit shadow of 3-bit experts is built once
 * on the host, and a second moe_layer pointing at the shadow blobs selects
 * it at run time, per call (the kernels see an ordinary 2-bit layer).
 *   src : host, src_bytes >= moe_packed_bytes(q_src, K, N)
 *   dst : host, dst_bytes >= moe_packed_bytes(q_dst, K, N) (output)
 * Returns MOE_ERR_UNSUPPORTED for a bad shape or qtype, MOE_ERR_BAD_CODES if
 * src holds a level outside its alphabet, and MOE_ERR_INVALID_ARG for null
 * pointers, short buffers, a non-finite scale in src, or a group whose new
 * scale would exceed the largest fp16 value. */
moe_status moe_requantize(int q_src, int q_dst, int64_t K, int64_t N, const void* src,
                          size_t src_bytes, void* dst, size_t dst_bytes);

/* ------------------------------------------------------------------ layer */
typedef struct {
  int32_t d;          /* hidden size, multiple of 128 */
  int32_t inter;      /* expert intermediate size, multiple of 128 */
  int32_t n_experts;  /* routed experts E, 1..1024 */
  int32_t top_k;      /* k, 1..min(E, 32) */
  int32_t n_shared;   /* 0 or 1 shared expert (weight 1, every token) */
  int32_t q_gate, q_up, q_down; /* moe_qtype of each projection (shared expert too) */
  const float* router_w;    /* device fp32 [E][d] (row e = expert e's router column);
                               may be NULL only with MOE_LOGITS_GIVEN */
  const float* router_bias; /* device fp32 [E] added to the logits, or NULL */
  const void* experts;      /* device: expert e's packed blob at experts + e*expert_stride,
                               256-B aligned (gate | up | down, see moe_expert_bytes) */
  size_t expert_stride;     /* >= moe_expert_bytes(...), multiple of 256 */
  const void* shared;       /* device packed shared expert (same layout), or NULL if none */
  /* Per-expert mixed precision (decode).  The "Xolotl" README's "Fast mode"
   * section keeps a lower-bit copy of the largest experts and reads it in
   * their place.  Here a second copy of the routed experts may be given in
   * other code families; alt_select picks, per expert, the copy that decode
   * calls read.  alt_experts == NULL: no second copy (the fields below are
   * then ignored).  Prefill calls on a layer with a second copy return
   * MOE_ERR_UNSUPPORTED.  The shared expert always comes from `shared`.
   * Errors: an unknown q_alt_* gives MOE_ERR_UNSUPPORTED; a NULL alt_select,
   * a short or unaligned alt_stride or an unaligned alt_experts gives
   * MOE_ERR_INVALID_ARG. */
  const void* alt_experts;  /* device: expert e's blob at alt_experts + e*alt_stride,
                               in the families q_alt_* (layout as `experts`) */
  size_t alt_stride;        /* >= moe_expert_bytes(q_alt_*), multiple of 256 */
  int32_t q_alt_gate, q_alt_up, q_alt_down;
  const uint8_t* alt_select; /* device [n_experts]: nonzero = expert e is read from the
                                second copy */
} moe_layer;

typedef struct {           /* caller-allocated device buffers, written by the calls below */
  float* logits;           /* [T][E]; an input under MOE_LOGITS_GIVEN */
  int32_t* topk_ids;       /* [T][k] */
  float* topk_w;           /* [T][k] */
  int32_t* counts;         /* [E] rows routed to each expert (shared expert not counted) */
  int32_t* offsets;        /* [E+1] exclusive prefix sum of counts; offsets[E] == T*k */
  int32_t* perm_tok;       /* [T*k] token of permuted row r (rows grouped by expert, tokens
                              ascending within an expert) */
  int32_t* inv_row;        /* [T][k] permuted row of (t, j) */
} moe_routing;

/* Device workspace needed by moe_route_topk / moe_forward_decode /
 * moe_forward_prefill for T tokens (the largest of the three).  0 if the
 * layer description is invalid. */
size_t moe_workspace_bytes(const moe_layer* L, int32_t T);

/* Router, top-k, weights and permutation only (the first steps of the layer).
 * Source: the "Xolotl" repository card, README "How it works, in one
 * paragraph": a token's router asks for a few experts and only those are
 * used.  The pages give no scoring function, normalisation or tie rule; the
 * definition at the top of this header (fp32 logits, k largest with the lower
 * index first on ties, softmax over the k selected, permutation stable in
 * token order) is this library's reading.
 *   x   : device bf16 [T][d] (ignored under MOE_LOGITS_GIVEN)
 *   R   : all fields required; logits is written unless MOE_LOGITS_GIVEN
 *   ws  : device workspace of ws_bytes >= moe_workspace_bytes(L, T) */
moe_status moe_route_topk(const moe_layer* L, const uint16_t* x, int32_t T, uint32_t flags,
                          moe_routing* R, void* ws, size_t ws_bytes, void* stream);

/* The whole layer for 1..8 tokens (decode), bandwidth-bound kernels that
 * stream each selected expert's packed bytes once for all its tokens.
 * Source: the "Xolotl" repository card, README "Latest" (an expert decoded
 * once for all the tokens that chose it, at 4-8 tokens) and "Fast mode
 * (DeepSeek-V4.1)" (decode speed is set by the expert bytes read per token).
 *   x   : device bf16 [T][d];  out : device bf16 [T][d], must not overlap x
 *   R   : routing outputs as in moe_route_topk
 * T outside 1..8 returns MOE_ERR_INVALID_ARG. */
moe_status moe_forward_decode(const moe_layer* L, const uint16_t* x, int32_t T, uint32_t flags,
                              moe_routing* R, void* ws, size_t ws_bytes, uint16_t* out,
                              void* stream);

/* The whole layer for any T >= 1 (prefill): matrix-core grouped GEMMs over
 * the permuted rows.  Arguments as for moe_forward_decode.  d must be a
 * multiple of 256 (MOE_ERR_UNSUPPORTED otherwise).  For a layer whose
 * three projections are all 2-bit or all ternary,
 * T * (top_k + n_shared) * max(d, inter) * 2 must not exceed 2^32 - 1
 * (MOE_ERR_UNSUPPORTED otherwise).
 * Source: the "Xolotl" repository card, README "What one PC can do" (prefill
 * throughput over prompts of thousands of tokens, where every expert sees many
 * rows); the grouped-GEMM form is this library's design, not the pages'. */
moe_status moe_forward_prefill(const moe_layer* L, const uint16_t* x, int32_t T, uint32_t flags,
                               moe_routing* R, void* ws, size_t ws_bytes, uint16_t* out,
                               void* stream);

/* ---------------------------------------------------------------- stages
 * Each forward call above enqueues a fixed sequence of kernels.  The _stages
 * variants enqueue only the kernels whose bit is set in stage_mask, with the
 * same arguments and validation; a stage reads what the earlier stages of the
 * same call left in the workspace (and in R), so a stage may be run alone only
 * after the earlier stages have run on that workspace with the same inputs.
 * This is the hook used to time one kernel with events or a profiler, and
 * running the stages in order one call at a time is equivalent to the full
 * call.  No stage overwrites what it reads, so a stage may also be run again
 * on the same workspace with the same result.  For a single token, at most
 * 256 experts and no second expert copy, the decode gate/up stage
 * makes the expert selection itself, from R->logits, and writes everything
 * the select stage writes (same values). A call whose mask holds both SELECT
 * and GATEUP then launches no separate select kernel.  An empty or unknown
 * mask returns MOE_ERR_INVALID_ARG. */
enum {
  MOE_DECODE_STAGE_ROUTE = 1u,   /* router logits + activation staging */
  MOE_DECODE_STAGE_SELECT = 2u,  /* top-k, weights, permutation, active-expert list */
  MOE_DECODE_STAGE_GATEUP = 4u,  /* gate/up projections + SiLU gating */
  MOE_DECODE_STAGE_DOWN = 8u,    /* down projection + weighted combine */
  MOE_DECODE_STAGES_ALL = 15u
};
enum {
  MOE_PREFILL_STAGE_ROUTE = 1u,    /* logits (unless given), top-k, permutation, tile list */
  MOE_PREFILL_STAGE_STAGE_X = 2u,  /* activation staging */
  MOE_PREFILL_STAGE_GATEUP = 4u,   /* grouped GEMM gate/up + SiLU gating (all-ternary
                                      layers: then h staged as scaled fp16 rows) */
  MOE_PREFILL_STAGE_DOWN = 8u,     /* grouped GEMM down */
  MOE_PREFILL_STAGE_COMBINE = 16u, /* unpermute + weighted combine */
  MOE_PREFILL_STAGES_ALL = 31u
};
moe_status moe_forward_decode_stages(const moe_layer* L, const uint16_t* x, int32_t T,
                                     uint32_t flags, moe_routing* R, void* ws, size_t ws_bytes,
                                     uint16_t* out, uint32_t stage_mask, void* stream);
moe_status moe_forward_prefill_stages(const moe_layer* L, const uint16_t* x, int32_t T,
                                      uint32_t flags, moe_routing* R, void* ws, size_t ws_bytes,
                                      uint16_t* out, uint32_t stage_mask, void* stream);

/* ---------------------------------------------------------- no allocation
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops and harnesses that forbid hipMalloc): the same layer
 * as moe_forward_decode, same kernels, arguments, validation and results,
 * without the workspace argument.  The workspace is a static device array of
 * MOE_NOALLOC_SCRATCH_BYTES inside the library; each GPU the library runs on
 * holds its own copy until the process ends, and its address is looked up
 * once per device, on the first call on that device.  The call allocates
 * nothing (no hipMalloc, no allocating library routine).
 * Every call on one GPU uses that GPU's array: calls on one stream are
 * ordered and safe, but calls whose work overlaps on one GPU (other streams,
 * other host threads) race on it and must not be issued.  No kernel needs the
 * array cleared between calls; each call writes all it reads.
 * Errors: as moe_forward_decode; MOE_ERR_WORKSPACE if the decode workspace of
 * (L, T) exceeds the array (no shape the decode path accepts does: d and
 * inter <= 8192, T*k <= 64 need at most about 2.9 MB); MOE_ERR_DEVICE if the
 * array's device address cannot be found. */
enum { MOE_NOALLOC_SCRATCH_BYTES = 4 << 20 };
moe_status moe_forward_decode_noalloc(const moe_layer* L, const uint16_t* x, int32_t T,
                                      uint32_t flags, moe_routing* R, uint16_t* out,
                                      void* stream);

/* Human-readable name of a status code (static string). */
const char* moe_status_string(moe_status s);

/* ABI version of this header: 3 (2 added the second expert copy to moe_layer,
 * 3 added moe_forward_decode_noalloc). */
int moe_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BQMOE_MOE_H */
