// Host-side packing of one projection into packed format v2 (see moe.h).
//
// The format is laid out for the decode kernels: a 512-B tile holds a 16 (n)
// x 128 (k) block of 2-bit fields, and lane chunk L = 16q + r of a tile is
// what wavefront lane L feeds to the matrix core for output column r and the
// k-slots 8q..8q+7 of each 32-wide group.  Inside a lane's 32-bit word the two
// 16-bit halves carry adjacent k-slots (s even / odd) of the same group, so a
// single mask-and-or turns a pair of fields into a pair of bf16 operands.
// Bit 2 of a 3-bit level (plane 1) is placed so that one shift lines up pairs
// 0..2 of a group just above their low bits and another shift pair 3.
#include <cmath>
#include <cstring>
#include <vector>

#include "moe_internal.h"

namespace bqmoe {

static size_t round256(size_t x) { return (x + 255) & ~size_t(255); }

// Plane-1 bit of pair v (k-slots 2v, 2v+1) of group gb, half h (slot parity).
static int plane1_bit(int gb, int h, int v) {
  static const int lo3[4] = {0, 1, 6, 7}, pair3[4] = {0, 1, 14, 15};
  return 16 * h + (v < 3 ? 2 * v + 2 + lo3[gb] : pair3[gb]);
}

bool format_shape_ok(int qtype, int64_t K, int64_t N) {
  return qtype_levels(qtype) > 0 && K > 0 && N > 0 && K % 128 == 0 && N % 16 == 0 &&
         K <= (int64_t(1) << 24) && N <= (int64_t(1) << 24);
}

PackedLayout packed_layout(int qtype, int64_t K, int64_t N) {
  PackedLayout p{};
  if (!format_shape_ok(qtype, K, N)) return p;
  size_t tiles = size_t(N / 16) * size_t(K / 128);
  p.plane0 = 0;
  size_t end = round256(tiles * 512);
  p.plane1 = end;
  if (qtype == MOE_Q_INT3) end = round256(end + tiles * 256);
  p.scales = end;
  p.total = round256(end + tiles * 128);
  return p;
}

}  // namespace bqmoe

using namespace bqmoe;

extern "C" size_t moe_packed_bytes(int qtype, int64_t K, int64_t N) {
  return packed_layout(qtype, K, N).total;
}

extern "C" size_t moe_expert_bytes(int qg, int qu, int qd, int64_t d, int64_t inter) {
  size_t g = moe_packed_bytes(qg, d, inter), u = moe_packed_bytes(qu, d, inter),
         dn = moe_packed_bytes(qd, inter, d);
  if (!g || !u || !dn) return 0;
  return g + u + dn;  // each is a multiple of 256
}

// Nearest fp16 value of a finite, non-negative double, ties to even (fp16:
// 11 significant bits, smallest subnormal 2^-24, largest finite 65504);
// returns 0x7C00 (infinity) past the largest finite value.
static uint16_t round_to_f16(double v) {
  if (v == 0.0) return 0;
  int e;
  std::frexp(v, &e);             // v = m * 2^e, m in [0.5, 1)
  int q = e - 11;                // unit in the last place of an 11-bit significand
  if (q < -24) q = -24;          // subnormal spacing
  const double units = std::nearbyint(std::ldexp(v, -q));  // ties to even (default mode)
  const double r = std::ldexp(units, q);
  if (r > 65504.0) return 0x7C00;
  if (r < 0x1p-14) return (uint16_t)units;  // subnormal: the significand is the code
  int re;
  const double rm = std::frexp(r, &re);      // r = rm * 2^re, rm in [0.5, 1)
  const uint32_t mant = (uint32_t)std::ldexp(rm, 11) - 1024u;  // 10 fraction bits
  return (uint16_t)(((re - 1 + 15) << 10) | mant);
}

static double f16_value(uint16_t h) {
  const int ex = (h >> 10) & 31, man = h & 1023;
  return ex == 0 ? std::ldexp((double)man, -24) : std::ldexp((double)(man | 1024), ex - 25);
}

extern "C" moe_status moe_quantize_rtn(int qtype, int64_t K, int64_t N, const float* w,
                                       uint8_t* codes, uint16_t* scales) {
  const int levels = qtype_levels(qtype);
  if (levels == 0 || K <= 0 || N <= 0 || K % 32) return MOE_ERR_UNSUPPORTED;
  if (!w || !codes || !scales) return MOE_ERR_INVALID_ARG;
  const double off = qtype_offset(qtype), cmax = (levels - 1) - off;
  for (int64_t i = 0; i < K * N; ++i)
    if (!std::isfinite(w[i])) return MOE_ERR_INVALID_ARG;
  for (int64_t n = 0; n < N; ++n) {
    for (int64_t g = 0; g < K / 32; ++g) {
      const float* wg = w + n * K + g * 32;
      double amax = 0.0;
      for (int j = 0; j < 32; ++j) amax = std::fmax(amax, std::fabs((double)wg[j]));
      const uint16_t sh = round_to_f16(amax / cmax);
      if (sh == 0x7C00) return MOE_ERR_INVALID_ARG;
      scales[n * (K / 32) + g] = sh;
      const double s = f16_value(sh);
      for (int j = 0; j < 32; ++j) {
        double u = s > 0.0 ? std::nearbyint((double)wg[j] / s + off) : std::nearbyint(off);
        u = std::fmin(std::fmax(u, 0.0), (double)(levels - 1));
        codes[n * K + g * 32 + j] = (uint8_t)u;
      }
    }
  }
  return MOE_OK;
}

extern "C" moe_status moe_pack_weights(int qtype, int64_t K, int64_t N, const uint8_t* codes,
                                       const uint16_t* scales, void* out, size_t out_bytes) {
  if (!format_shape_ok(qtype, K, N)) return MOE_ERR_UNSUPPORTED;
  if (!codes || !scales || !out) return MOE_ERR_INVALID_ARG;
  PackedLayout lay = packed_layout(qtype, K, N);
  if (out_bytes < lay.total) return MOE_ERR_INVALID_ARG;
  const int levels = qtype_levels(qtype);
  for (int64_t i = 0; i < K * N; ++i)
    if (codes[i] >= levels) return MOE_ERR_BAD_CODES;

  uint8_t* base = static_cast<uint8_t*>(out);
  std::memset(base, 0, lay.total);
  const int64_t NT = N / 16, KB = K / 128;
  for (int64_t nt = 0; nt < NT; ++nt) {
    for (int64_t kb = 0; kb < KB; ++kb) {
      const size_t tile = size_t(nt * KB + kb);
      uint32_t* p0 = reinterpret_cast<uint32_t*>(base + lay.plane0 + tile * 512);
      uint32_t* p1 = reinterpret_cast<uint32_t*>(base + lay.plane1 + tile * 256);
      uint16_t* ps = reinterpret_cast<uint16_t*>(base + lay.scales + tile * 128);
      for (int lane = 0; lane < 64; ++lane) {
        const int q = lane >> 4, r = lane & 15;
        const int64_t n = nt * 16 + r;
        const uint8_t* row = codes + n * K + kb * 128;
        uint32_t w0[2] = {0, 0}, hi = 0;
        for (int gb = 0; gb < 4; ++gb) {      // group inside the k-block
          for (int s = 0; s < 8; ++s) {       // k-slot inside the lane's 8
            const int kk = gb * 32 + q * 8 + s;
            const uint32_t u = row[kk];
            const int half = s & 1, pair = s >> 1;
            const int field = 4 * (gb & 1) + pair;
            w0[gb >> 1] |= (u & 3u) << (16 * half + 2 * field);
            hi |= (u >> 2) << plane1_bit(gb, half, pair);
          }
        }
        p0[lane * 2 + 0] = w0[0];
        p0[lane * 2 + 1] = w0[1];
        if (qtype == MOE_Q_INT3) p1[lane] = hi;
      }
      for (int r = 0; r < 16; ++r)
        for (int gb = 0; gb < 4; ++gb)
          ps[r * 4 + gb] = scales[(nt * 16 + r) * (K / 32) + kb * 4 + gb];
    }
  }
  return MOE_OK;
}

// Inverse of moe_pack_weights: the codes and scales of a packed projection.
static moe_status unpack_weights(int qtype, int64_t K, int64_t N, const uint8_t* base,
                                 uint8_t* codes, uint16_t* scales) {
  const PackedLayout lay = packed_layout(qtype, K, N);
  const int64_t NT = N / 16, KB = K / 128;
  const int levels = qtype_levels(qtype);
  for (int64_t nt = 0; nt < NT; ++nt) {
    for (int64_t kb = 0; kb < KB; ++kb) {
      const size_t tile = size_t(nt * KB + kb);
      const uint32_t* p0 = reinterpret_cast<const uint32_t*>(base + lay.plane0 + tile * 512);
      const uint32_t* p1 = reinterpret_cast<const uint32_t*>(base + lay.plane1 + tile * 256);
      const uint16_t* ps = reinterpret_cast<const uint16_t*>(base + lay.scales + tile * 128);
      for (int lane = 0; lane < 64; ++lane) {
        const int q = lane >> 4, r = lane & 15;
        const int64_t n = nt * 16 + r;
        uint8_t* row = codes + n * K + kb * 128;
        const uint32_t hi = qtype == MOE_Q_INT3 ? p1[lane] : 0u;
        for (int gb = 0; gb < 4; ++gb) {
          for (int s = 0; s < 8; ++s) {
            const int half = s & 1, pair = s >> 1;
            const int field = 4 * (gb & 1) + pair;
            uint32_t u = (p0[lane * 2 + (gb >> 1)] >> (16 * half + 2 * field)) & 3u;
            u |= ((hi >> plane1_bit(gb, half, pair)) & 1u) << 2;
            if ((int)u >= levels) return MOE_ERR_BAD_CODES;
            row[gb * 32 + q * 8 + s] = (uint8_t)u;
          }
        }
      }
      for (int r = 0; r < 16; ++r)
        for (int gb = 0; gb < 4; ++gb)
          scales[(nt * 16 + r) * (K / 32) + kb * 4 + gb] = ps[r * 4 + gb];
    }
  }
  return MOE_OK;
}

extern "C" moe_status moe_requantize(int q_src, int q_dst, int64_t K, int64_t N, const void* src,
                                     size_t src_bytes, void* dst, size_t dst_bytes) {
  if (!format_shape_ok(q_src, K, N) || !format_shape_ok(q_dst, K, N)) return MOE_ERR_UNSUPPORTED;
  if (!src || !dst) return MOE_ERR_INVALID_ARG;
  if (src_bytes < packed_layout(q_src, K, N).total || dst_bytes < packed_layout(q_dst, K, N).total)
    return MOE_ERR_INVALID_ARG;
  std::vector<uint8_t> codes(size_t(K * N));
  std::vector<uint16_t> scales(size_t(N * (K / 32)));
  moe_status st = unpack_weights(q_src, K, N, static_cast<const uint8_t*>(src), codes.data(),
                                 scales.data());
  if (st != MOE_OK) return st;
  for (uint16_t sh : scales)
    if ((sh & 0x7C00u) == 0x7C00u) return MOE_ERR_INVALID_ARG;  // infinite or NaN scale
  // every weight s * (u - offset) is exact in fp32 (an 11-bit scale times a half-integer <= 3.5)
  const double off = qtype_offset(q_src);
  std::vector<float> w(size_t(K * N));
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k)
      w[n * K + k] = (float)(f16_value(scales[n * (K / 32) + k / 32]) * ((double)codes[n * K + k] - off));
  std::vector<uint8_t> codes2(size_t(K * N));
  std::vector<uint16_t> scales2(size_t(N * (K / 32)));
  st = moe_quantize_rtn(q_dst, K, N, w.data(), codes2.data(), scales2.data());
  if (st != MOE_OK) return st;
  return moe_pack_weights(q_dst, K, N, codes2.data(), scales2.data(), dst, dst_bytes);
}
