/*
 * Seeded, counter-based generators for synthetic MoE-layer inputs.
 *
 * This module draws random numbers and stores them in the input dtypes
 * (bf16, fp16, fp32, small integer codes).  It holds none of the MoE
 * layer's arithmetic: no routing, no dequantisation, no products.  Both the
 * CPU oracle's tests and the GPU path's tests / benchmark take their inputs
 * from here, so that the two sides see identical bytes.
 *
 * Counter-based stream: element i of stream (seed, stream) is
 *     mix64(key + (i + 1) * GAMMA),  key = mix64(seed * GAMMA ^ mix64(stream + GAMMA))
 * where mix64 is the SplitMix64 output finaliser (Steele, Lea & Flood,
 * "Fast splittable pseudorandom number generators", OOPSLA 2014) and GAMMA
 * its golden-ratio increment.  Any element can be regenerated on its own,
 * so a large tensor never has to be held whole by a checker.
 *
 * Normals use the Box-Muller transform on two uniforms taken from counters
 * 2i and 2i+1 of the same stream.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

#define GAMMA 0x9E3779B97F4A7C15ULL

static inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

static inline uint64_t stream_key(uint64_t seed, uint64_t stream) {
  return mix64((seed * GAMMA) ^ mix64(stream + GAMMA));
}

static inline uint64_t draw(uint64_t key, uint64_t i) { return mix64(key + (i + 1) * GAMMA); }

/* uniform in (0, 1]: 53 random bits, never zero (safe for log). */
static inline double unif(uint64_t key, uint64_t i) {
  return ((double)(draw(key, i) >> 11) + 1.0) * (1.0 / 9007199254740992.0);
}

static inline double normal(uint64_t key, uint64_t i) {
  const double two_pi = 6.283185307179586476925286766559;
  double u1 = unif(key, 2 * i), u2 = unif(key, 2 * i + 1);
  return sqrt(-2.0 * log(u1)) * cos(two_pi * u2);
}

/* float -> bf16 bits, round to nearest even (input storage only). */
static inline uint16_t f32_to_bf16_bits(float f) {
  uint32_t b;
  memcpy(&b, &f, 4);
  if ((b & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((b >> 16) | 0x40u);
  uint32_t r = 0x7FFFu + ((b >> 16) & 1u);
  return (uint16_t)((b + r) >> 16);
}

/* non-negative finite double -> fp16 bits, round to nearest even. */
static inline uint16_t pos_f64_to_f16_bits(double a) {
  if (!(a > 0.0)) return 0;
  if (a >= 65520.0) return 0x7C00; /* rounds to infinity */
  int e;
  frexp(a, &e);               /* a = m * 2^e, m in [0.5, 1) */
  int ulp_e = e - 11;         /* fp16 keeps 11 significant bits */
  if (ulp_e < -24) ulp_e = -24; /* subnormal spacing 2^-24 */
  double q = nearbyint(ldexp(a, -ulp_e));
  double v = ldexp(q, ulp_e);
  /* v is an fp16 value: encode it */
  if (v < ldexp(1.0, -14)) return (uint16_t)ldexp(v, 24);
  int ev;
  double mv = frexp(v, &ev);  /* v = mv * 2^ev, mv in [0.5,1) */
  uint16_t mant = (uint16_t)(ldexp(mv, 11) - 1024.0);
  uint16_t expo = (uint16_t)(ev - 1 + 15);
  return (uint16_t)((expo << 10) | mant);
}

void synth_u64(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, uint64_t* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = draw(key, start + (uint64_t)i);
}

void synth_normal_f64(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, double mean,
                      double sigma, double* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = mean + sigma * normal(key, start + (uint64_t)i);
}

void synth_normal_f32(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, double mean,
                      double sigma, float* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = (float)(mean + sigma * normal(key, start + (uint64_t)i));
}

void synth_normal_bf16(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, double mean,
                       double sigma, uint16_t* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i)
    out[i] = f32_to_bf16_bits((float)(mean + sigma * normal(key, start + (uint64_t)i)));
}

/* fp16 bits of |N(0, sigma)| (group scales). */
void synth_absnormal_f16(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, double sigma,
                         uint16_t* out) {
  uint64_t key = stream_key(seed, stream);
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n; ++i) out[i] = pos_f64_to_f16_bits(fabs(sigma * normal(key, start + (uint64_t)i)));
}

/* Uniform level indices over an alphabet of `levels` values (2, 3, 4 or 8). */
void synth_codes(uint64_t seed, uint64_t stream, uint64_t start, int64_t n, int levels,
                 uint8_t* out) {
  uint64_t key = stream_key(seed, stream);
  if (levels == 4 || levels == 8 || levels == 2) {
    uint64_t mask = (uint64_t)levels - 1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)(draw(key, start + (uint64_t)i) & mask);
  } else {
    /* multiply-shift of the top 32 bits onto [0, levels) */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i)
      out[i] = (uint8_t)(((draw(key, start + (uint64_t)i) >> 32) * (uint64_t)levels) >> 32);
  }
}
