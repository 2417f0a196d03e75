/*
 * CPU oracle for the quantized MoE expert layer -- TEST INFRASTRUCTURE ONLY.
 * (Loaded only by the tests, the smoke check and the benchmark's CPU-baseline
 * leg; the GPU library neither links nor calls it.)
 *
 * What the layer computes, and where it comes from
 * -------------------------------------------------
 * Sources are the pages on the Xolotl engine:
 *   [HOW]   "Xolotl" repository card (ossradar.top), README section "How it
 *           works, in one paragraph": a mixture-of-experts model uses only a
 *           few experts per token, and each token's router asks for them.
 *   [QUANT] same page, README "Quick start" (model list): the experts are a
 *           mixed ternary / 2-bit / 3-bit quantisation.
 *   [FAST]  same page, README "Fast mode": decode speed is set by the expert
 *           bytes moved per token.
 * The pages name the ideas only: they print no formula, shape, bit layout,
 * scoring function or tie rule.  Everything else below is this library's
 * stated reading, marked "Reading:".
 *
 *  1. Weights (Reading, from [QUANT]'s three code families): a projection is
 *     a logical matrix W[K][N] applied as y = x . W.  Codes u[n][k] are level
 *     indices; groups are 32 consecutive k for one n, each with an fp16 scale
 *     s[n][k/32].  W[k][n] = s[n][k/32] * (u[n][k] - off), off = 1 (ternary,
 *     u in 0..2), 1.5 (2-bit, u in 0..3), 3.5 (3-bit, u in 0..7).
 *  2. Router ([HOW]): logits[t][e] = sum_i x[t][i] * Wr[i][e] (+ bias[e]),
 *     rounded to fp32.
 *  3. Selection (Reading): the k largest logits, ordered by descending value,
 *     lower expert index first on equal values (IEEE ==, so +0 == -0).
 *  4. Weights (Reading): softmax over the k selected logits (sums to 1).
 *  5. Permutation (Reading): counting sort of the T*k (token, slot) rows by
 *     expert, stable in token order; counts, exclusive offsets, perm_tok
 *     (token of each permuted row), inv_row (permuted row of each (t, j)).
 *  6. Expert FFN (Reading, SwiGLU): g = x.Wg, u = x.Wu, h = bf16(SiLU(g)*u),
 *     y = bf16(h.Wd).  The shared expert (if any) runs on every token with
 *     weight 1 and is not counted in `counts`.
 *  7. Combine ([HOW]'s per-token gather): out[t] = bf16([x[t]] +
 *     sum_j w[t][j] * y(t, j) + y_shared[t]); x is added only for a residual
 *     layer.
 * Rounding points (Reading): h, y and out are bf16 (round to nearest even
 * from the exact double value); logits and weights are fp32; all sums are in
 * double.
 *
 * Packed format v2 (the decoder below; written from the format definition):
 *   K % 128 == 0 and N % 16 == 0.  NT = N/16 n-tiles, KB = K/128 k-blocks.
 *   plane 0 (u & 3): NT*KB tiles of 512 B, tile (nt,kb) at (nt*KB+kb)*512;
 *     inside, 64 chunks of 8 B (chunk L at L*8) = two little-endian 32-bit
 *     words.  For code (n, k): r = n%16, kk = k%128, gb = kk/32, j = kk%32,
 *     q = j/8, s = j%8; chunk L = 16q + r; word gb/2; 2-bit field at bit
 *     16*(s%2) + 2*(4*(gb%2) + s/2).
 *   plane 1 (3-bit only, u >> 2): starts at the next 256-B boundary; NT*KB
 *     tiles of 256 B; chunk L (one 32-bit word) at L*4; with v = s/2, bit
 *     16*(s%2) + 2v + 2 + {0,1,6,7}[gb] if v < 3, else 16*(s%2) + {0,1,14,15}[gb].
 *   scales: start at the next 256-B boundary; NT*KB blocks of 128 B; block
 *     (nt,kb) holds fp16 scale s[16nt+r][4kb+gb] at index r*4 + gb.
 *   The blob size is rounded up to a multiple of 256 B.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------ numbers */

double oracle_bf16_to_f64(uint16_t b) {
  uint32_t bits = (uint32_t)b << 16;
  float f;
  memcpy(&f, &bits, 4);
  return (double)f;
}

/* bf16 has fp32's exponent range and 8 significant bits.  Round the exact
 * double to the nearest bf16 value, ties to even, in one step. */
uint16_t oracle_f64_to_bf16(double v) {
  if (isnan(v)) return 0x7FC0;
  uint16_t sign = signbit(v) ? 0x8000 : 0;
  double a = fabs(v);
  if (a == 0.0) return sign;
  if (isinf(a)) return (uint16_t)(sign | 0x7F80);
  int e;
  frexp(a, &e);              /* a = m * 2^e with m in [0.5, 1) */
  int ulp_e = e - 8;         /* spacing of 8-significant-bit values at this binade */
  if (ulp_e < -133) ulp_e = -133; /* bf16 subnormal spacing 2^-133 */
  double q = nearbyint(ldexp(a, -ulp_e)); /* default rounding mode: ties to even */
  double r = ldexp(q, ulp_e);
  if (r >= ldexp(1.0, 128)) return (uint16_t)(sign | 0x7F80); /* overflow to infinity */
  float f = (float)r; /* exact: r is a bf16 value, hence an fp32 value */
  uint32_t bits;
  memcpy(&bits, &f, 4);
  return (uint16_t)(sign | (bits >> 16));
}

double oracle_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int ex = (h >> 10) & 0x1F;
  int man = h & 0x3FF;
  double v;
  if (ex == 0)
    v = ldexp((double)man, -24);
  else if (ex == 31)
    v = man ? NAN : INFINITY;
  else
    v = ldexp((double)(man + 1024), ex - 25);
  return sign ? -v : v;
}

double oracle_code_offset(int qtype) {
  switch (qtype) {
    case 1: return 1.0;
    case 2: return 1.5;
    case 3: return 3.5;
  }
  return NAN;
}

int oracle_code_levels(int qtype) {
  switch (qtype) {
    case 1: return 3;
    case 2: return 4;
    case 3: return 8;
  }
  return 0;
}

/* ------------------------------------------------------------ packed format */

static size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

static int shape_ok(int qtype, int64_t K, int64_t N) {
  return oracle_code_levels(qtype) > 0 && K > 0 && N > 0 && K % 128 == 0 && N % 16 == 0;
}

size_t oracle_packed_bytes(int qtype, int64_t K, int64_t N) {
  if (!shape_ok(qtype, K, N)) return 0;
  size_t tiles = (size_t)(N / 16) * (size_t)(K / 128);
  size_t off = round256(tiles * 512);
  if (qtype == 3) off = round256(off + tiles * 256);
  return round256(off + tiles * 128);
}

static uint32_t rd32(const uint8_t* p) {
  return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
}

int oracle_unpack(int qtype, int64_t K, int64_t N, const uint8_t* blob, size_t blob_bytes,
                  uint8_t* codes, uint16_t* scales) {
  size_t need = oracle_packed_bytes(qtype, K, N);
  if (!need || blob_bytes < need || !blob || !codes || !scales) return -1;
  int64_t KB = K / 128, NT = N / 16;
  size_t tiles = (size_t)NT * (size_t)KB;
  size_t p1 = round256(tiles * 512);
  size_t ps = qtype == 3 ? round256(p1 + tiles * 256) : p1;
  int levels = oracle_code_levels(qtype);
  for (int64_t n = 0; n < N; ++n) {
    int64_t nt = n / 16, r = n % 16;
    for (int64_t k = 0; k < K; ++k) {
      int64_t kb = k / 128, kk = k % 128, gb = kk / 32, j = kk % 32, q = j / 8, s = j % 8;
      int64_t L = 16 * q + r;
      size_t tile = (size_t)(nt * KB + kb);
      const uint8_t* chunk0 = blob + tile * 512 + (size_t)L * 8;
      uint32_t w0 = rd32(chunk0 + 4 * (gb / 2));
      int bit0 = (int)(16 * (s % 2) + 2 * (4 * (gb % 2) + s / 2));
      unsigned u = (w0 >> bit0) & 3u;
      if (qtype == 3) {
        uint32_t w1 = rd32(blob + p1 + tile * 256 + (size_t)L * 4);
        static const int below3[4] = {0, 1, 6, 7}, third[4] = {0, 1, 14, 15};
        int v = (int)(s / 2);
        int bit1 = (int)(16 * (s % 2)) + (v < 3 ? 2 * v + 2 + below3[gb] : third[gb]);
        u |= ((w1 >> bit1) & 1u) << 2;
      }
      if ((int)u >= levels) return -1; /* e.g. level 3 in a ternary matrix */
      codes[n * K + k] = (uint8_t)u;
    }
    for (int64_t g = 0; g < K / 32; ++g) {
      int64_t kb = g / 4, gb = g % 4;
      const uint8_t* p = blob + ps + (size_t)(nt * KB + kb) * 128 + (size_t)(r * 4 + gb) * 2;
      scales[n * (K / 32) + g] = (uint16_t)(p[0] | (p[1] << 8));
    }
  }
  return 0;
}

/* ------------------------------------------------------- quantise (RTN) */

/* fp16 nearest to a finite v >= 0, ties to even, as bits; 0x7C00 past 65504.
 * Written from the fp16 definition: in the binade [2^e, 2^(e+1)) (e >= -14)
 * the representable values are multiples of 2^(e-10); below 2^-14 they are
 * multiples of 2^-24.  Take the two neighbours and keep the nearer. */
static uint16_t oracle_f64_to_f16(double v) {
  if (v == 0.0) return 0;
  int e = ilogb(v);
  if (e < -14) e = -14;
  double ulp = ldexp(1.0, e - 10);
  double lo = floor(v / ulp) * ulp, hi = lo + ulp, r;
  if (v - lo < hi - v) r = lo;
  else if (hi - v < v - lo) r = hi;
  else r = fmod(lo / ulp, 2.0) == 0.0 ? lo : hi;   /* tie: even multiple */
  if (r > 65504.0) return 0x7C00;
  if (r < ldexp(1.0, -14)) return (uint16_t)(r / ldexp(1.0, -24));
  int E = ilogb(r);                                 /* r = 1.f * 2^E */
  double frac = r / ldexp(1.0, E) - 1.0;            /* in [0, 1), multiple of 2^-10 */
  return (uint16_t)(((E + 15) << 10) | (int)(frac * 1024.0));
}

/* Round-to-nearest quantisation, the reading in moe.h: per column n and
 * 32-group g, s = fp16(max|w| / cmax) with cmax = (levels-1) - offset, and
 * u = clamp(round-half-even(w / s + offset), 0, levels-1); u = round(offset)
 * when s == 0.  Returns -1 for a bad qtype or shape or a non-finite weight
 * or a scale past the fp16 range. */
int oracle_quantize_rtn(int qtype, int64_t K, int64_t N, const float* w, uint8_t* codes,
                        uint16_t* scales) {
  int levels = oracle_code_levels(qtype);
  if (levels == 0 || K <= 0 || N <= 0 || K % 32) return -1;
  double off = oracle_code_offset(qtype), cmax = (levels - 1) - off;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t g = 0; g < K / 32; ++g) {
      double amax = 0.0;
      for (int64_t k = g * 32; k < g * 32 + 32; ++k) {
        double a = fabs((double)w[n * K + k]);
        if (!isfinite(a)) return -1;
        if (a > amax) amax = a;
      }
      uint16_t sb = oracle_f64_to_f16(amax / cmax);
      if (sb == 0x7C00) return -1;
      scales[n * (K / 32) + g] = sb;
      double s = oracle_f16_to_f64(sb);
      for (int64_t k = g * 32; k < g * 32 + 32; ++k) {
        double u = s > 0.0 ? nearbyint((double)w[n * K + k] / s + off) : nearbyint(off);
        if (u < 0.0) u = 0.0;
        if (u > levels - 1) u = levels - 1;
        codes[n * K + k] = (uint8_t)u;
      }
    }
  }
  return 0;
}

/* -------------------------------------------------------------- dequantise */

int oracle_dequant(int qtype, int64_t K, int64_t N, const uint8_t* codes, const uint16_t* scales,
                   double* W) {
  if (oracle_code_levels(qtype) == 0 || K <= 0 || N <= 0 || K % 32) return -1;
  double off = oracle_code_offset(qtype);
  int levels = oracle_code_levels(qtype);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      uint8_t u = codes[n * K + k];
      if (u >= levels) return -1;
      W[k * N + n] = oracle_f16_to_f64(scales[n * (K / 32) + k / 32]) * ((double)u - off);
    }
  return 0;
}

/* ------------------------------------------------------------------ router */

int oracle_router_logits(int T, int d, int E, const uint16_t* x, const float* Wr, const float* bias,
                         float* logits) {
  if (T < 0 || d <= 0 || E <= 0) return -1;
  for (int t = 0; t < T; ++t)
    for (int e = 0; e < E; ++e) {
      double acc = 0.0;
      for (int i = 0; i < d; ++i)
        acc += oracle_bf16_to_f64(x[(size_t)t * d + i]) * (double)Wr[(size_t)e * d + i];
      if (bias) acc += (double)bias[e];
      logits[(size_t)t * E + e] = (float)acc;
    }
  return 0;
}

/* candidate a ranks before candidate b: larger logit, or equal logit and lower index */
static int ranks_before(float la, int a, float lb, int b) {
  if (la > lb) return 1;
  if (la == lb) return a < b;
  return 0;
}

int oracle_topk_softmax(int T, int E, int k, const float* logits, int32_t* ids, float* w) {
  if (T < 0 || E <= 0 || k <= 0 || k > E) return -1;
  int* order = (int*)malloc(sizeof(int) * (size_t)E);
  if (!order) return -1;
  for (int t = 0; t < T; ++t) {
    const float* L = logits + (size_t)t * E;
    for (int e = 0; e < E; ++e)
      if (isnan(L[e])) {
        free(order);
        return -1;
      }
    /* insertion sort of all candidates by the ranking rule (plain and obviously ordered) */
    for (int e = 0; e < E; ++e) {
      int pos = e;
      while (pos > 0 && ranks_before(L[e], e, L[order[pos - 1]], order[pos - 1])) {
        order[pos] = order[pos - 1];
        --pos;
      }
      order[pos] = e;
    }
    double top = (double)L[order[0]];
    double denom = 0.0;
    for (int j = 0; j < k; ++j) denom += exp((double)L[order[j]] - top);
    for (int j = 0; j < k; ++j) {
      ids[(size_t)t * k + j] = order[j];
      w[(size_t)t * k + j] = (float)(exp((double)L[order[j]] - top) / denom);
    }
  }
  free(order);
  return 0;
}

int oracle_permute(int T, int E, int k, const int32_t* ids, int32_t* counts, int32_t* offsets,
                   int32_t* perm_tok, int32_t* inv_row) {
  if (T < 0 || E <= 0 || k <= 0) return -1;
  for (int e = 0; e < E; ++e) counts[e] = 0;
  for (int r = 0; r < T * k; ++r) {
    if (ids[r] < 0 || ids[r] >= E) return -1;
    counts[ids[r]]++;
  }
  offsets[0] = 0;
  for (int e = 0; e < E; ++e) offsets[e + 1] = offsets[e] + counts[e];
  /* place rows in increasing (t, j) order: each expert's rows come out in token order */
  int32_t* fill = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
  if (!fill) return -1;
  for (int e = 0; e < E; ++e) fill[e] = offsets[e];
  for (int t = 0; t < T; ++t)
    for (int j = 0; j < k; ++j) {
      int e = ids[(size_t)t * k + j];
      int pos = fill[e]++;
      perm_tok[pos] = t;
      inv_row[(size_t)t * k + j] = pos;
    }
  free(fill);
  return 0;
}

/* ------------------------------------------------------------------ expert */

/* SiLU(g) = g / (1 + exp(-g)), evaluated without overflow for any finite g */
static double silu(double g) {
  if (g >= 0) return g / (1.0 + exp(-g));
  double e = exp(g);
  return g * e / (1.0 + e);
}

/* y[n] = sum_k x[k] * W[k][n] for one projection given by codes/scales; x is double[K]. */
static void project(int qtype, int64_t K, int64_t N, const uint8_t* codes, const uint16_t* scales,
                    const double* x, double* y) {
  double off = oracle_code_offset(qtype);
  for (int64_t n = 0; n < N; ++n) {
    double acc = 0.0;
    const uint8_t* cn = codes + n * K;
    const uint16_t* sn = scales + n * (K / 32);
    for (int64_t g = 0; g < K / 32; ++g) {
      const double s = oracle_f16_to_f64(sn[g]); /* the group's scale */
      for (int64_t k = g * 32; k < g * 32 + 32; ++k) {
        double wkn = s * ((double)cn[k] - off);
        acc += x[k] * wkn;
      }
    }
    y[n] = acc;
  }
}

static int codes_in_range(int qtype, int64_t n, const uint8_t* c) {
  int levels = oracle_code_levels(qtype);
  for (int64_t i = 0; i < n; ++i)
    if (c[i] >= levels) return 0;
  return 1;
}

int oracle_expert_rows(int d, int I, int qg, int qu, int qd, const uint8_t* cg, const uint16_t* sg,
                       const uint8_t* cu, const uint16_t* su, const uint8_t* cd, const uint16_t* sd,
                       int M, const uint16_t* x_rows, uint16_t* h_out, uint16_t* y_out,
                       double* g_out, double* u_out, double* y_pre) {
  if (d <= 0 || I <= 0 || M < 0 || d % 32 || I % 32) return -1;
  if (!oracle_code_levels(qg) || !oracle_code_levels(qu) || !oracle_code_levels(qd)) return -1;
  if (!codes_in_range(qg, (int64_t)d * I, cg) || !codes_in_range(qu, (int64_t)d * I, cu) ||
      !codes_in_range(qd, (int64_t)d * I, cd))
    return -1;
  double* xv = (double*)malloc(sizeof(double) * (size_t)d);
  double* g = (double*)malloc(sizeof(double) * (size_t)I);
  double* u = (double*)malloc(sizeof(double) * (size_t)I);
  double* h = (double*)malloc(sizeof(double) * (size_t)I);
  double* y = (double*)malloc(sizeof(double) * (size_t)d);
  if (!xv || !g || !u || !h || !y) {
    free(xv), free(g), free(u), free(h), free(y);
    return -1;
  }
  for (int m = 0; m < M; ++m) {
    for (int i = 0; i < d; ++i) xv[i] = oracle_bf16_to_f64(x_rows[(size_t)m * d + i]);
    project(qg, d, I, cg, sg, xv, g);
    project(qu, d, I, cu, su, xv, u);
    for (int n = 0; n < I; ++n) {
      uint16_t hb = oracle_f64_to_bf16(silu(g[n]) * u[n]);
      h[n] = oracle_bf16_to_f64(hb);
      if (h_out) h_out[(size_t)m * I + n] = hb;
      if (g_out) g_out[(size_t)m * I + n] = g[n];
      if (u_out) u_out[(size_t)m * I + n] = u[n];
    }
    project(qd, I, d, cd, sd, h, y);
    for (int n = 0; n < d; ++n) {
      y_out[(size_t)m * d + n] = oracle_f64_to_bf16(y[n]);
      if (y_pre) y_pre[(size_t)m * d + n] = y[n];
    }
  }
  free(xv), free(g), free(u), free(h), free(y);
  return 0;
}

/* ----------------------------------------------------------------- combine */

int oracle_combine(int T, int d, int k, const float* w, const int32_t* inv_row, const uint16_t* y,
                   const uint16_t* y_shared, const uint16_t* x, int residual, uint16_t* out,
                   double* out_pre) {
  if (T < 0 || d <= 0 || k <= 0) return -1;
  for (int t = 0; t < T; ++t)
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      if (residual) acc += oracle_bf16_to_f64(x[(size_t)t * d + c]);
      for (int j = 0; j < k; ++j) {
        int row = inv_row[(size_t)t * k + j];
        acc += (double)w[(size_t)t * k + j] * oracle_bf16_to_f64(y[(size_t)row * d + c]);
      }
      if (y_shared) acc += oracle_bf16_to_f64(y_shared[(size_t)t * d + c]);
      out[(size_t)t * d + c] = oracle_f64_to_bf16(acc);
      if (out_pre) out_pre[(size_t)t * d + c] = acc;
    }
  return 0;
}

/* ------------------------------------------------------------- whole layer */

int oracle_moe_layer(int T, int d, int E, int k, int I, int n_shared, int qg, int qu, int qd,
                     const uint16_t* x, const float* Wr, const float* bias, int logits_given,
                     float* logits, const uint8_t* const* ec, const uint16_t* const* es,
                     int residual, int32_t* ids, float* w, int32_t* counts, int32_t* offsets,
                     int32_t* perm_tok, int32_t* inv_row, uint16_t* out) {
  if (T < 0 || d <= 0 || E <= 0 || k <= 0 || k > E || I <= 0 || n_shared < 0 || n_shared > 1)
    return -1;
  if (!logits_given && oracle_router_logits(T, d, E, x, Wr, bias, logits)) return -1;
  if (oracle_topk_softmax(T, E, k, logits, ids, w)) return -1;
  if (oracle_permute(T, E, k, ids, counts, offsets, perm_tok, inv_row)) return -1;
  size_t rows = (size_t)T * k;
  uint16_t* xr = (uint16_t*)malloc(sizeof(uint16_t) * (rows ? rows : 1) * d);
  uint16_t* y = (uint16_t*)malloc(sizeof(uint16_t) * (rows ? rows : 1) * d);
  uint16_t* ysh = n_shared ? (uint16_t*)malloc(sizeof(uint16_t) * (T ? T : 1) * (size_t)d) : NULL;
  int rc = 0;
  if (!xr || !y || (n_shared && !ysh)) rc = -1;
  /* gather the rows of each expert (permuted order), run the expert once for all of them */
  for (size_t r = 0; !rc && r < rows; ++r)
    memcpy(xr + r * d, x + (size_t)perm_tok[r] * d, sizeof(uint16_t) * d);
  for (int e = 0; !rc && e < E; ++e) {
    int M = counts[e];
    if (!M) continue;
    size_t r0 = (size_t)offsets[e];
    rc = oracle_expert_rows(d, I, qg, qu, qd, ec[e * 3 + 0], es[e * 3 + 0], ec[e * 3 + 1],
                            es[e * 3 + 1], ec[e * 3 + 2], es[e * 3 + 2], M, xr + r0 * d, NULL,
                            y + r0 * d, NULL, NULL, NULL);
  }
  if (!rc && n_shared)
    rc = oracle_expert_rows(d, I, qg, qu, qd, ec[E * 3 + 0], es[E * 3 + 0], ec[E * 3 + 1],
                            es[E * 3 + 1], ec[E * 3 + 2], es[E * 3 + 2], T, x, NULL, ysh, NULL,
                            NULL, NULL);
  if (!rc) rc = oracle_combine(T, d, k, w, inv_row, y, ysh, x, residual, out, NULL);
  free(xr), free(y), free(ysh);
  return rc;
}
