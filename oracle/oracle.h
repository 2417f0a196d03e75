/*
 * CPU oracle for the quantized MoE expert layer -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this library.  The GPU library never links or calls it, and it
 * shares no code, header, table or helper with the GPU library.
 *
 * Everything is plain, slow, single-threaded C: weights are rebuilt from
 * their level codes and fp16 group scales, every dot product is accumulated
 * in double precision, and the layer's bf16 rounding points are applied with
 * this file's own round-to-nearest-even conversion.
 *
 * Status codes: 0 = ok, -1 = invalid argument (bad shape, code out of range,
 * NaN logit, buffer too small).
 */
#ifndef MOE_ORACLE_H
#define MOE_ORACLE_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* number formats */
double oracle_bf16_to_f64(uint16_t b);
uint16_t oracle_f64_to_bf16(double v);
double oracle_f16_to_f64(uint16_t h);

/* qtype: 1 ternary (levels 0..2, offset 1), 2 int2 (0..3, 1.5), 3 int3 (0..7, 3.5) */
double oracle_code_offset(int qtype);
int oracle_code_levels(int qtype);

/* Round-to-nearest quantisation of float weights w[N][K] into codes[N][K] and
 * fp16 scales[N][K/32] (the reading stated in moe.h); 0, or -1 on bad input. */
int oracle_quantize_rtn(int qtype, int64_t K, int64_t N, const float* w, uint8_t* codes,
                        uint16_t* scales);

/* Packed format v2: decode a blob back to canonical codes [N][K] and scales [N][K/32]. */
size_t oracle_packed_bytes(int qtype, int64_t K, int64_t N);
int oracle_unpack(int qtype, int64_t K, int64_t N, const uint8_t* blob, size_t blob_bytes,
                  uint8_t* codes, uint16_t* scales);

/* Dense weights W[K][N] (double) of one projection, from codes [N][K] + scales [N][K/32]. */
int oracle_dequant(int qtype, int64_t K, int64_t N, const uint8_t* codes, const uint16_t* scales,
                   double* W);

/* logits[t][e] = fp32( sum_i x[t][i] * Wr[e][i] + bias[e] ), sum in double. Wr stored [E][d]. */
int oracle_router_logits(int T, int d, int E, const uint16_t* x, const float* Wr, const float* bias,
                         float* logits);

/* top-k by (descending logit, ascending index); weights = softmax over the k selected. */
int oracle_topk_softmax(int T, int E, int k, const float* logits, int32_t* ids, float* w);

/* stable counting sort of the T*k (token, slot) rows by expert id. */
int oracle_permute(int T, int E, int k, const int32_t* ids, int32_t* counts, int32_t* offsets,
                   int32_t* perm_tok, int32_t* inv_row);

/* One expert's SwiGLU FFN on M rows (bf16 bits [M][d]).  h = bf16(SiLU(x.Wg) * (x.Wu)) [M][I],
 * y = bf16(h.Wd) [M][d].  Weights given as codes+scales per projection.  h_out may be NULL.
 * g_out / u_out (double [M][I], may be NULL) receive the unrounded projections, and
 * y_pre (double [M][d], may be NULL) the unrounded down projection. */
int oracle_expert_rows(int d, int I, int qg, int qu, int qd,
                       const uint8_t* cg, const uint16_t* sg,
                       const uint8_t* cu, const uint16_t* su,
                       const uint8_t* cd, const uint16_t* sd,
                       int M, const uint16_t* x_rows, uint16_t* h_out, uint16_t* y_out,
                       double* g_out, double* u_out, double* y_pre);

/* out[t] = bf16( [x[t]] + sum_j w[t][j] * y[inv_row[t][j]] + [y_shared[t]] ), in double.
 * y: bf16 [T*k][d] in permuted-row order; y_shared: bf16 [T][d] or NULL; x used iff residual. */
int oracle_combine(int T, int d, int k, const float* w, const int32_t* inv_row, const uint16_t* y,
                   const uint16_t* y_shared, const uint16_t* x, int residual, uint16_t* out,
                   double* out_pre);

/* The whole layer.  experts_codes[e*3+m] / experts_scales[e*3+m] for e < E (+1 shared), m =
 * gate, up, down.  If logits_given, `logits` is an input; else it is written from x and Wr.
 * Routing arrays are outputs. */
int oracle_moe_layer(int T, int d, int E, int k, int I, int n_shared, int qg, int qu, int qd,
                     const uint16_t* x, const float* Wr, const float* bias, int logits_given,
                     float* logits, const uint8_t* const* experts_codes,
                     const uint16_t* const* experts_scales, int residual, int32_t* ids, float* w,
                     int32_t* counts, int32_t* offsets, int32_t* perm_tok, int32_t* inv_row,
                     uint16_t* out);

#ifdef __cplusplus
}
#endif
#endif
