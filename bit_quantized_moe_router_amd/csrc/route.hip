// Routing kernels: router logits, top-k with softmax weights, and the stable
// expert permutation (histogram / prefix sum / scatter with wavefront ballots).
//
// The pages ("Xolotl" card, README "How it works, in one paragraph") say only
// that each token's router asks for a few experts.  The rule implemented here
// (Reading): the k largest fp32 logits, descending, lower expert index first on
// equal values (IEEE ==), weights = softmax over the selected k; rows are
// grouped by expert with tokens ascending inside each expert.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "moe_internal.h"
#include "topk_common.h"

namespace bqmoe {

// ------------------------------------------------------------------ logits
// Wave per expert, up to 8 tokens per block row (grid.y tiles the tokens).
// Router weights are stored [E][d] so a wave streams one contiguous row.
__global__ __launch_bounds__(256) void k_router_logits(const uint16_t* __restrict__ x, int T, int d,
                                                       int E, const float* __restrict__ Wr,
                                                       const float* __restrict__ bias,
                                                       float* __restrict__ logits) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.y * 8;
  const int nt = min(8, T - t0);
  const int e = blockIdx.x * 4 + wave;
  if (e >= E) return;
  // rows past the last token re-read the last token (their sums are not
  // stored), so that every load of a step is unconditional
  const uint16_t* xr[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) xr[t] = x + (size_t)(t0 + min(t, nt - 1)) * d;
  float acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = 0.f;
  const float* w = Wr + (size_t)e * d;
  for (int i = lane * 4; i < d; i += 256) {
    const float4 wv = *reinterpret_cast<const float4*>(w + i);
    uint2 xv[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) xv[t] = *reinterpret_cast<const uint2*>(xr[t] + i);
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      acc[t] = fmaf(bf16_to_f32(xv[t].x & 0xFFFFu), wv.x, acc[t]);
      acc[t] = fmaf(bf16_to_f32(xv[t].x >> 16), wv.y, acc[t]);
      acc[t] = fmaf(bf16_to_f32(xv[t].y & 0xFFFFu), wv.z, acc[t]);
      acc[t] = fmaf(bf16_to_f32(xv[t].y >> 16), wv.w, acc[t]);
    }
  }
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const float s = wave_sum(acc[t]);
    if (t < nt && lane == 0) logits[(size_t)(t0 + t) * E + e] = s + b;
  }
}

// Decode router logits (TT = T <= 8 tokens, a compile-time count so that
// every load of a step is unconditional and all of them are in flight
// together): block per expert, its 4 waves split d; the router row is read
// once for all T tokens and the partial sums meet in LDS.  The blocks after
// the E logit blocks stage x for the expert kernels: xs = x/16 (exact) and, per 32-group, the
// staged sums of the correction term (see stage_sums in device_common.h).
template <int TT>
__global__ __launch_bounds__(256) void k_dec_logits(const uint16_t* __restrict__ x, int T, int d,
                                                    int E, const float* __restrict__ Wr,
                                                    const float* __restrict__ bias,
                                                    float* __restrict__ logits, int do_logits,
                                                    uint16_t* __restrict__ xs,
                                                    uint16_t* __restrict__ xsum) {
  __shared__ float s_part[4][TT];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int e = blockIdx.x;
  const int nlog = do_logits ? E : 0;  // blocks [0, nlog): one logit each; the rest stage x
  if (e < nlog) {
    float acc[TT];
#pragma unroll
    for (int t = 0; t < TT; ++t) acc[t] = 0.f;
    const float* w = Wr + (size_t)e * d;
    // 8 consecutive entries per lane and step (d is a multiple of 128)
#pragma unroll 2
    for (int i = tid * 8; i < d; i += 2048) {
      const float4 w0 = *reinterpret_cast<const float4*>(w + i);
      const float4 w1 = *reinterpret_cast<const float4*>(w + i + 4);
      uint4 xv[TT];
#pragma unroll
      for (int t = 0; t < TT; ++t) xv[t] = *reinterpret_cast<const uint4*>(x + (size_t)t * d + i);
#pragma unroll
      for (int t = 0; t < TT; ++t) {
        acc[t] = fmaf(bf16_to_f32(xv[t].x & 0xFFFFu), w0.x, acc[t]);
        acc[t] = fmaf(bf16_to_f32(xv[t].x >> 16), w0.y, acc[t]);
        acc[t] = fmaf(bf16_to_f32(xv[t].y & 0xFFFFu), w0.z, acc[t]);
        acc[t] = fmaf(bf16_to_f32(xv[t].y >> 16), w0.w, acc[t]);
        acc[t] = fmaf(bf16_to_f32(xv[t].z & 0xFFFFu), w1.x, acc[t]);
        acc[t] = fmaf(bf16_to_f32(xv[t].z >> 16), w1.y, acc[t]);
        acc[t] = fmaf(bf16_to_f32(xv[t].w & 0xFFFFu), w1.z, acc[t]);
        acc[t] = fmaf(bf16_to_f32(xv[t].w >> 16), w1.w, acc[t]);
      }
    }
#pragma unroll
    for (int t = 0; t < TT; ++t) {
      const float s = wave_sum_lanes(acc[t]);
      if (lane == 0) s_part[wave][t] = s;
    }
    __syncthreads();
    if (tid < TT) {
      const float s = ((s_part[0][tid] + s_part[1][tid]) + s_part[2][tid]) + s_part[3][tid];
      logits[(size_t)tid * E + e] = s + (bias ? bias[e] : 0.f);
    }
  }
  // staging: one 32-lane half-wave per (token, group), on blocks of their own so
  // that it runs beside the logits instead of after them
  if (e < nlog) return;
  const int G = d / 32;
  const int pairs = T * G;
  const int half = tid >> 5, j = tid & 31;
  for (int p = (e - nlog) * 8 + half; p < pairs; p += (gridDim.x - nlog) * 8) {
    const int t = p / G, g = p % G;
    const uint32_t xb = x[(size_t)t * d + g * 32 + j];
    const float xf = bf16_to_f32(xb);
    xs[(size_t)t * d + g * 32 + j] = (uint16_t)f32_to_bf16(xf * 0.0625f);
    float sw = xf * slot_weight(j), sm = xf;
#pragma unroll
    for (int o = 16; o > 0; o >>= 1) {
      sw += __shfl_xor(sw, o, 32);
      sm += __shfl_xor(sm, o, 32);
    }
    if (j == 0) *reinterpret_cast<uint4*>(xsum + ((size_t)t * G + g) * 8) = stage_sums(sw, sm);
  }
}

// Generic top-k: wave per token.
template <int PER>
__global__ __launch_bounds__(256) void k_topk(const float* __restrict__ logits, int T, int E, int k,
                                              int32_t* __restrict__ ids, float* __restrict__ w) {
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (t >= T) return;
  int id;
  float wt;
  wave_topk<PER>(logits + (size_t)t * E, E, k, lane, id, wt);
  if (lane < k) {
    ids[(size_t)t * k + lane] = id;
    w[(size_t)t * k + lane] = wt;
  }
}

// Lanes whose `key` (< 2^bits) equals this lane's, among `active` lanes.
__device__ __forceinline__ uint64_t match_peers(int key, int bits, uint64_t active) {
  uint64_t peers = active;
  for (int b = 0; b < bits; ++b) {
    const uint64_t m = __ballot((key >> b) & 1);
    peers &= ((key >> b) & 1) ? m : ~m;
  }
  return peers;
}

__device__ __forceinline__ int expert_bits(int E) {
  int b = 0;
  while ((1 << b) < E) ++b;
  return b ? b : 1;
}

// Block-wide exclusive scan of n <= 2*blockDim.x ints in LDS (in place).
// Returns the total.  blockDim.x must be a multiple of 64, at most 1024.
__device__ int block_exclusive_scan(int* a, int n, int* wave_tot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nw = blockDim.x >> 6;
  const int i0 = 2 * tid, i1 = 2 * tid + 1;
  const int v0 = i0 < n ? a[i0] : 0, v1 = i1 < n ? a[i1] : 0;
  int s = v0 + v1;
  // inclusive scan inside the wave
  int incl = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  if (tid == 0) {
    int run = 0;
    for (int w = 0; w < nw; ++w) {
      const int t = wave_tot[w];
      wave_tot[w] = run;
      run += t;
    }
    wave_tot[nw] = run;
  }
  __syncthreads();
  const int excl = incl - s + wave_tot[wave];
  if (i0 < n) a[i0] = excl;
  if (i1 < n) a[i1] = excl + v0;
  const int total = wave_tot[nw];
  __syncthreads();
  return total;
}

// ------------------------------------------------- decode: select + permute
// One block of 8 waves for T <= 8 tokens (T*k <= 64 rows):
//   1. wave t selects token t's top-k (k rounds of a wave maximum) and its
//      softmax weights;
//   2. the <= 64 selected rows sit one per lane of wave 0, which derives each
//      row's in-expert rank, permuted position and slot from ~log2(E)
//      ballots over the expert-id bits;
//   3. meanwhile, on waves 1..7, every expert's count and offset is a count
//      over the rows, held in registers.
// Slots list the active experts in ascending id, then the shared expert.
constexpr int kSelThreads = 512;  // one wave per decode token

template <int PER>
__global__ __launch_bounds__(kSelThreads) void k_dec_select(
    const float* __restrict__ logits, int T, int E, int k, int n_shared,
    int32_t* __restrict__ ids, float* __restrict__ wts, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm_tok, int32_t* __restrict__ inv_row,
    int32_t* __restrict__ slots, int max_slots, const uint8_t* __restrict__ alt_select) {
  __shared__ __attribute__((aligned(16))) int s_row[kDecodeMaxRoutedRows];  // expert of row t*k + j
  __shared__ int s_nact;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rows = T * k;
  // 1. top-k and weights, wave t for token t (same order and softmax as the
  //    generic top-k kernel)
  if (wave < T) {
    int id;
    float w;
    wave_topk<PER>(logits + (size_t)wave * E, E, k, lane, id, w);
    if (lane < k) {
      ids[wave * k + lane] = id;
      wts[wave * k + lane] = w;
      s_row[wave * k + lane] = id;
    }
  }
  __syncthreads();
  // 2. rows (wave 0): rank among the rows of the same expert, permuted
  //     position and slot, from ballots over the expert-id bits
  if (wave == 0) {
    const bool act = lane < rows;
    const int id = act ? s_row[lane] : 0;
    const uint64_t active = __ballot(act);
    uint64_t eq = active, less = 0;  // rows with the same id / a smaller id
    for (int b = expert_bits(E) - 1; b >= 0; --b) {
      const int bit = (id >> b) & 1;
      const uint64_t m1 = __ballot(act && bit);
      if (bit) {
        less |= eq & ~m1;
        eq &= m1;
      } else {
        eq &= ~m1;
      }
    }
    const uint64_t below = lane ? (~0ull >> (64 - lane)) : 0ull;
    const int rk = __popcll(eq & below);
    const uint64_t first = __ballot(act && rk == 0);
    const int off = __popcll(less), slot = __popcll(less & first);
    const int n_active = __popcll(first);
    if (act) {
      const int pos = off + rk;
      perm_tok[pos] = lane / k;
      inv_row[lane] = pos;
      int32_t* rec = slots + kSlotRec * (1 + slot);
      rec[kSlotTok + rk] = lane / k;
      if (rk == 0) {
        rec[0] = id;
        rec[1] = off;
        rec[2] = __popcll(eq);
        rec[3] = alt_select && alt_select[id] ? 1 : 0;  // read from the second expert copy
      }
    }
    if (n_shared && lane < T) {  // shared slot: rows T*k + t, token t
      int32_t* rec = slots + kSlotRec * (1 + n_active);
      if (lane == 0) {
        rec[0] = -1;
        rec[1] = rows;
        rec[2] = T;
        rec[3] = 0;
      }
      rec[kSlotTok + lane] = lane;
    }
    if (lane == 0) {
      slots[0] = n_active + (n_shared ? 1 : 0);
      offsets[E] = rows;
      s_nact = n_active;
    }
  } else {
    // 3. meanwhile, on the other waves: every expert's count and offset, the
    //    row ids in registers
    int rid[kDecodeMaxRoutedRows];
#pragma unroll
    for (int q4 = 0; q4 < kDecodeMaxRoutedRows / 4; ++q4) {
      const int4 v = *reinterpret_cast<const int4*>(s_row + 4 * q4);
      rid[4 * q4] = 4 * q4 < rows ? v.x : 0x7FFFFFFF;
      rid[4 * q4 + 1] = 4 * q4 + 1 < rows ? v.y : 0x7FFFFFFF;
      rid[4 * q4 + 2] = 4 * q4 + 2 < rows ? v.z : 0x7FFFFFFF;
      rid[4 * q4 + 3] = 4 * q4 + 3 < rows ? v.w : 0x7FFFFFFF;
    }
    for (int e = tid - 64; e < E; e += kSelThreads - 64) {
      int cnt = 0, off = 0;
#pragma unroll
      for (int r = 0; r < kDecodeMaxRoutedRows; ++r) {
        cnt += rid[r] == e;
        off += rid[r] < e;
      }
      counts[e] = cnt;
      offsets[e] = off;
    }
  }
  __syncthreads();
  // records past the last slot: no rows (a decode block reads only its own
  // record and stops on M == 0)
  const int n_slots = s_nact + (n_shared ? 1 : 0);
  for (int sidx = n_slots + tid; sidx < max_slots; sidx += kSelThreads) {
    int32_t* rec = slots + kSlotRec * (1 + sidx);
    rec[0] = 0;
    rec[1] = 0;
    rec[2] = 0;
    rec[3] = 0;
  }
}

// ------------------------------------------------ generic permutation (any T)
// Block b handles tokens [b*256, b*256+256), i.e. rows [b*256*k, ...).  Each
// wave takes a contiguous quarter of the block's rows in 64-row chunks; lanes
// with equal experts are matched with ballots, so every row gets its rank
// among the block's earlier rows of the same expert without atomics.
__global__ __launch_bounds__(256) void k_hist(const int32_t* __restrict__ ids, int T, int E, int k,
                                              int32_t* __restrict__ hist,
                                              int32_t* __restrict__ lrank) {
  __shared__ int cnt[4][MOE_MAX_EXPERTS];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  for (int i = tid; i < 4 * E; i += 256) cnt[i / E][i % E] = 0;
  __syncthreads();
  const int r_begin = blockIdx.x * kHistTokensPerBlock * k;
  const int r_end = min(T * k, r_begin + kHistTokensPerBlock * k);
  const int nrows = r_end - r_begin;
  const int nchunk = (nrows + 63) / 64;
  const int per = (nchunk + 3) / 4;
  const int c0 = wave * per, c1 = min(nchunk, c0 + per);
  const int bits = expert_bits(E);
  for (int c = c0; c < c1; ++c) {
    const int r = r_begin + c * 64 + lane;
    const bool act = r < r_end;
    const int e = act ? ids[r] : 0;
    const uint64_t active = __ballot(act);
    const uint64_t peers = match_peers(e, bits, active);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    // One LDS read instruction for all lanes, then the group leaders' write: a
    // wave's LDS accesses complete in program order, so no barrier is needed.
    int base = 0;
    if (act) base = cnt[wave][e];
    if (act) lrank[r] = base + __popcll(peers & lt);
    if (act && (peers & lt) == 0) cnt[wave][e] = base + __popcll(peers);
  }
  __syncthreads();
  // per-wave bases (prefix over waves) and the block histogram
  for (int e = tid; e < E; e += 256) {
    int run = 0;
    for (int w = 0; w < 4; ++w) {
      const int c = cnt[w][e];
      cnt[w][e] = run;
      run += c;
    }
    hist[(size_t)blockIdx.x * E + e] = run;
  }
  __syncthreads();
  for (int c = c0; c < c1; ++c) {
    const int r = r_begin + c * 64 + lane;
    if (r < r_end) lrank[r] += cnt[wave][ids[r]];
  }
}

// Single block: per-expert exclusive scan over blocks (in place), counts,
// offsets, and the grouped-GEMM tile list of tm-row tiles (routed experts in id order, then
// the shared expert).
__global__ __launch_bounds__(1024) void k_scan(int32_t* __restrict__ hist, int nblk, int E, int T,
                                               int k, int n_shared, int tm,
                                               int32_t* __restrict__ counts,
                                               int32_t* __restrict__ offsets,
                                               int32_t* __restrict__ tiles,
                                               int32_t* __restrict__ ctrl) {
  __shared__ int s_cnt[MOE_MAX_EXPERTS];
  __shared__ int s_off[MOE_MAX_EXPERTS];
  __shared__ int s_nt[MOE_MAX_EXPERTS];
  __shared__ int s_tot[17];
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += blockDim.x) {
    int run = 0;
    for (int b = 0; b < nblk; ++b) {
      const size_t i = (size_t)b * E + e;
      const int c = hist[i];
      hist[i] = run;
      run += c;
    }
    s_cnt[e] = run;
    s_off[e] = run;
    s_nt[e] = (run + tm - 1) / tm;
  }
  __syncthreads();
  const int total = block_exclusive_scan(s_off, E, s_tot);
  const int ntiles = block_exclusive_scan(s_nt, E, s_tot);
  for (int e = tid; e < E; e += blockDim.x) {
    counts[e] = s_cnt[e];
    offsets[e] = s_off[e];
    const int n = (s_cnt[e] + tm - 1) / tm;
    for (int i = 0; i < n; ++i) {
      int32_t* t = tiles + 4 * (s_nt[e] + i);
      t[0] = e;
      t[1] = s_off[e] + i * tm;
      t[2] = min(tm, s_cnt[e] - i * tm);
      t[3] = 0;
    }
  }
  int nsh = 0;
  if (n_shared) {
    nsh = (T + tm - 1) / tm;
    for (int i = tid; i < nsh; i += blockDim.x) {
      int32_t* t = tiles + 4 * (ntiles + i);
      t[0] = -1;
      t[1] = T * k + i * tm;
      t[2] = min(tm, T - i * tm);
      t[3] = 0;
    }
  }
  if (tid == 0) {
    offsets[E] = total;
    ctrl[0] = ntiles + nsh;
  }
}

__global__ __launch_bounds__(256) void k_scatter(const int32_t* __restrict__ ids, int T, int E,
                                                 int k, const int32_t* __restrict__ blkbase,
                                                 const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ lrank,
                                                 int32_t* __restrict__ perm_tok,
                                                 int32_t* __restrict__ inv_row) {
  const int r = blockIdx.x * 256 + threadIdx.x;
  if (r >= T * k) return;
  const int e = ids[r];
  const int t = r / k;
  const int b = t / kHistTokensPerBlock;
  const int pos = offsets[e] + blkbase[(size_t)b * E + e] + lrank[r];
  perm_tok[pos] = t;
  inv_row[r] = pos;
}

// ------------------------------------------------------------------ launch
int launch_route_generic(const moe_layer* L, const uint16_t* x, int T, uint32_t flags,
                         moe_routing* R, uint8_t* ws, const PrefillWs& P, void* stream) {
  hipStream_t s = (hipStream_t)stream;
  const int E = L->n_experts, k = L->top_k, d = L->d;
  if (!(flags & MOE_LOGITS_GIVEN)) {
    dim3 grid((E + 3) / 4, (T + 7) / 8);
    hipLaunchKernelGGL(k_router_logits, grid, dim3(256), 0, s, x, T, d, E, L->router_w,
                       L->router_bias, R->logits);
  }
#define BQ_TK(PER)                                                                              \
  hipLaunchKernelGGL(k_topk<PER>, dim3((T + 3) / 4), dim3(256), 0, s, R->logits, T, E, k,      \
                     R->topk_ids, R->topk_w)
  if (E <= 64)
    BQ_TK(1);
  else if (E <= 128)
    BQ_TK(2);
  else if (E <= 256)
    BQ_TK(4);
  else if (E <= 512)
    BQ_TK(8);
  else
    BQ_TK(16);
#undef BQ_TK
  int32_t* hist = (int32_t*)(ws + P.hist);
  int32_t* lrank = (int32_t*)(ws + P.lrank);
  hipLaunchKernelGGL(k_hist, dim3(P.nblk), dim3(256), 0, s, R->topk_ids, T, E, k, hist, lrank);
  hipLaunchKernelGGL(k_scan, dim3(1), dim3(1024), 0, s, hist, P.nblk, E, T, k, L->n_shared,
                     prefill_tile_rows(L),
                     R->counts, R->offsets, (int32_t*)(ws + P.tiles), (int32_t*)(ws + P.ctrl));
  hipLaunchKernelGGL(k_scatter, dim3((T * k + 255) / 256), dim3(256), 0, s, R->topk_ids, T, E, k,
                     hist, R->offsets, lrank, R->perm_tok, R->inv_row);
  return (int)hipGetLastError();
}

// decode routing: logits + staging, then select (2 launches)
int launch_decode_route(const moe_layer* L, const uint16_t* x, int T, uint32_t flags,
                        moe_routing* R, uint8_t* ws, const DecodeWs& W, void* stream,
                        uint32_t mask) {
  hipStream_t s = (hipStream_t)stream;
  const int E = L->n_experts, k = L->top_k, d = L->d;
  const int do_logits = !(flags & MOE_LOGITS_GIVEN);
  if (mask & MOE_DECODE_STAGE_ROUTE) {
    const int G = d / 32;
    dim3 grid((do_logits ? E : 0) + (T * G + 7) / 8);
#define BQ_LG(TT)                                                                             \
  case TT:                                                                                    \
    hipLaunchKernelGGL(k_dec_logits<TT>, grid, dim3(256), 0, s, x, T, d, E, L->router_w,      \
                       L->router_bias, R->logits, do_logits, (uint16_t*)(ws + W.xs),          \
                       (uint16_t*)(ws + W.xsum));                                             \
    break
    switch (T) {
      BQ_LG(1); BQ_LG(2); BQ_LG(3); BQ_LG(4); BQ_LG(5); BQ_LG(6); BQ_LG(7); BQ_LG(8);
      default: return (int)hipErrorInvalidValue;
    }
#undef BQ_LG
  }
  if (mask & MOE_DECODE_STAGE_SELECT) {
#define BQ_SEL(PER)                                                                               \
  hipLaunchKernelGGL(k_dec_select<PER>, dim3(1), dim3(kSelThreads), 0, s, R->logits, T, E, k,    \
                     L->n_shared, R->topk_ids, R->topk_w, R->counts, R->offsets, R->perm_tok,    \
                     R->inv_row, (int32_t*)(ws + W.slots), W.max_slots,                          \
                     L->alt_experts ? L->alt_select : nullptr)
    if (E <= 64)
      BQ_SEL(1);
    else if (E <= 128)
      BQ_SEL(2);
    else if (E <= 256)
      BQ_SEL(4);
    else if (E <= 512)
      BQ_SEL(8);
    else
      BQ_SEL(16);
#undef BQ_SEL
  }
  return (int)hipGetLastError();
}

}  // namespace bqmoe
