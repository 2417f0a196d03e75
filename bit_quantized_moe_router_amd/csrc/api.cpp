// C ABI entry points: argument validation, workspace layout, dispatch.
// Every check below happens before anything is enqueued on the stream.
#include <cstdint>
#include <cstring>

#include "moe_internal.h"

namespace bqmoe {

static size_t al256(size_t x) { return (x + 255) & ~size_t(255); }

static bool layer_ok(const moe_layer* L) {
  if (!L) return false;
  if (L->d <= 0 || L->inter <= 0 || L->d % 128 || L->inter % 128 || L->d > MOE_MAX_DIM ||
      L->inter > MOE_MAX_DIM)
    return false;
  if (L->n_experts < 1 || L->n_experts > MOE_MAX_EXPERTS) return false;
  if (L->top_k < 1 || L->top_k > MOE_MAX_TOPK || L->top_k > L->n_experts) return false;
  if (L->n_shared < 0 || L->n_shared > 1) return false;
  if (!qtype_levels(L->q_gate) || !qtype_levels(L->q_up) || !qtype_levels(L->q_down)) return false;
  return true;
}

DecodeWs decode_ws_layout(const moe_layer* L, int T) {
  DecodeWs w{};
  const int k = L->top_k, d = L->d, I = L->inter, S = L->n_shared;
  w.max_slots = (T * k < L->n_experts ? T * k : L->n_experts) + S;
  w.rows = T * k + T * S;
  size_t o = 0;
  w.slots = o;
  o = al256(o + sizeof(int32_t) * kSlotRec * (1 + (size_t)w.max_slots));
  w.xs = o;
  o = al256(o + 2 * (size_t)T * d);
  w.xsum = o;
  o = al256(o + 16 * (size_t)T * (d / 32));
  w.hs = o;
  o = al256(o + 2 * (size_t)w.rows * I);
  w.hsum = o;
  o = al256(o + 16 * (size_t)w.rows * (I / 32));
  w.y = o;
  o = al256(o + 2 * (size_t)w.rows * d);
  w.total = o;
  return w;
}

PrefillWs prefill_ws_layout(const moe_layer* L, int T) {
  PrefillWs p{};
  const int k = L->top_k, d = L->d, I = L->inter, S = L->n_shared, E = L->n_experts;
  p.nblk = (T + kHistTokensPerBlock - 1) / kHistTokensPerBlock;
  const size_t rows_routed = (size_t)T * k;
  p.rows = (int)(rows_routed + (size_t)T * S);
  const size_t tm = (size_t)prefill_tile_rows(L);
  p.max_tiles = (int)(rows_routed / tm + (size_t)E + (S ? ((size_t)T + tm - 1) / tm : 0));
  size_t o = 0;
  p.ctrl = o;
  o = al256(o + 64);
  p.hist = o;
  o = al256(o + sizeof(int32_t) * (size_t)p.nblk * E);
  p.lrank = o;
  o = al256(o + sizeof(int32_t) * rows_routed);
  p.tiles = o;
  o = al256(o + sizeof(int32_t) * 4 * (size_t)p.max_tiles);
  p.xs = o;
  o = al256(o + 2 * (size_t)T * d);
  p.xsum = o;
  o = al256(o + 16 * (size_t)T * (d / 32));
  p.h = o;
  o = al256(o + 2 * (size_t)p.rows * I);
  p.hsum = o;
  o = al256(o + 16 * (size_t)p.rows * (I / 32));
  p.y = o;
  o = al256(o + 2 * (size_t)p.rows * d);
  p.x6 = o;
  o = al256(o + (size_t)T * d);
  p.h6 = o;
  o = al256(o + (size_t)p.rows * I);
  p.total = o;
  return p;
}

static bool overlaps(const void* a, size_t na, const void* b, size_t nb) {
  const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
  return x < y + nb && y < x + na;
}

static bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// shared checks for the calls that take routing buffers
// (ws_need: the workspace bytes the call requires; 0 = moe_workspace_bytes(L, T))
static moe_status check_common(const moe_layer* L, const uint16_t* x, int32_t T, uint32_t flags,
                               const moe_routing* R, const void* ws, size_t ws_bytes,
                               bool need_experts, size_t ws_need = 0) {
  if (!layer_ok(L)) {
    if (!L) return MOE_ERR_INVALID_ARG;
    // distinguish plain invalid values from unsupported-but-meaningful shapes
    if (L->d <= 0 || L->inter <= 0 || L->n_experts <= 0 || L->top_k <= 0 ||
        L->top_k > L->n_experts || L->n_shared < 0 || L->n_shared > 1)
      return MOE_ERR_INVALID_ARG;
    return MOE_ERR_UNSUPPORTED;
  }
  if (T < 0) return MOE_ERR_INVALID_ARG;
  if (flags & ~(uint32_t)(MOE_LOGITS_GIVEN | MOE_ADD_RESIDUAL)) return MOE_ERR_INVALID_ARG;
  if ((int64_t)T * L->top_k > (int64_t)1 << 30) return MOE_ERR_UNSUPPORTED;
  if (!R || !R->logits || !R->topk_ids || !R->topk_w || !R->counts || !R->offsets ||
      !R->perm_tok || !R->inv_row)
    return MOE_ERR_INVALID_ARG;
  if (!(flags & MOE_LOGITS_GIVEN)) {
    if (!L->router_w || !x) return MOE_ERR_INVALID_ARG;
  }
  if (need_experts) {
    const size_t eb = moe_expert_bytes(L->q_gate, L->q_up, L->q_down, L->d, L->inter);
    if (!x || !L->experts || L->expert_stride < eb || L->expert_stride % 256 ||
        !aligned(L->experts, 256))
      return MOE_ERR_INVALID_ARG;
    if (L->n_shared && (!L->shared || !aligned(L->shared, 256))) return MOE_ERR_INVALID_ARG;
    if (!aligned(x, 16)) return MOE_ERR_INVALID_ARG;
    if (L->alt_experts) {  // the second copy of the routed experts
      const size_t ab =
          moe_expert_bytes(L->q_alt_gate, L->q_alt_up, L->q_alt_down, L->d, L->inter);
      if (!ab) return MOE_ERR_UNSUPPORTED;  // a code family outside the three
      if (!L->alt_select || L->alt_stride < ab || L->alt_stride % 256 ||
          !aligned(L->alt_experts, 256))
        return MOE_ERR_INVALID_ARG;
    }
  }
  if (!ws || ws_bytes < (ws_need ? ws_need : moe_workspace_bytes(L, T))) return MOE_ERR_WORKSPACE;
  if (!aligned(ws, 256)) return MOE_ERR_INVALID_ARG;
  return MOE_OK;
}

}  // namespace bqmoe

using namespace bqmoe;

extern "C" size_t moe_workspace_bytes(const moe_layer* L, int32_t T) {
  if (!layer_ok(L) || T < 0) return 0;
  if (T == 0) return 256;
  size_t b = prefill_ws_layout(L, T).total;
  if (T <= MOE_MAX_DECODE_TOKENS) {
    const size_t dcd = decode_ws_layout(L, T).total;
    if (dcd > b) b = dcd;
  }
  return b;
}

extern "C" moe_status moe_route_topk(const moe_layer* L, const uint16_t* x, int32_t T,
                                     uint32_t flags, moe_routing* R, void* ws, size_t ws_bytes,
                                     void* stream) {
  if (T == 0 && L && R) return MOE_OK;
  moe_status st = check_common(L, x, T, flags, R, ws, ws_bytes, false);
  if (st != MOE_OK) return st;
  const PrefillWs P = prefill_ws_layout(L, T);
  return launch_route_generic(L, x, T, flags, R, (uint8_t*)ws, P, stream) ? MOE_ERR_DEVICE
                                                                         : MOE_OK;
}

namespace bqmoe {
// decode_ws_only: the workspace need only hold the decode layout (the
// no-allocation entry point's fixed array), not moe_workspace_bytes
moe_status decode_call(const moe_layer* L, const uint16_t* x, int32_t T, uint32_t flags,
                       moe_routing* R, void* ws, size_t ws_bytes, uint16_t* out, uint32_t mask,
                       void* stream, bool decode_ws_only) {
  if (T < 1 || T > MOE_MAX_DECODE_TOKENS) return MOE_ERR_INVALID_ARG;
  if (decode_ws_only && !layer_ok(L)) return L ? MOE_ERR_UNSUPPORTED : MOE_ERR_INVALID_ARG;
  const size_t need = decode_ws_only ? decode_ws_layout(L, T).total : 0;
  moe_status st = check_common(L, x, T, flags, R, ws, ws_bytes, true, need);
  if (st != MOE_OK) return st;
  if (T * L->top_k > kDecodeMaxRoutedRows || T * (L->top_k + L->n_shared) > kDecodeMaxRows ||
      L->d > kDecodeMaxDim || L->inter > kDecodeMaxDim || !decode_shape_ok(L, T))
    return MOE_ERR_UNSUPPORTED;
  if (!out || !aligned(out, 16)) return MOE_ERR_INVALID_ARG;
  const size_t bytes = (size_t)T * L->d * 2;
  if (overlaps(x, bytes, out, bytes)) return MOE_ERR_INVALID_ARG;
  const DecodeWs W = decode_ws_layout(L, T);
  return launch_decode(L, x, T, flags, R, (uint8_t*)ws, W, out, stream, mask) ? MOE_ERR_DEVICE
                                                                            : MOE_OK;
}
}  // namespace bqmoe

static moe_status decode_impl(const moe_layer* L, const uint16_t* x, int32_t T, uint32_t flags,
                              moe_routing* R, void* ws, size_t ws_bytes, uint16_t* out,
                              uint32_t mask, void* stream) {
  return decode_call(L, x, T, flags, R, ws, ws_bytes, out, mask, stream, false);
}

static moe_status prefill_impl(const moe_layer* L, const uint16_t* x, int32_t T, uint32_t flags,
                               moe_routing* R, void* ws, size_t ws_bytes, uint16_t* out,
                               uint32_t mask, void* stream) {
  if (T == 0 && L && R) return MOE_OK;
  moe_status st = check_common(L, x, T, flags, R, ws, ws_bytes, true);
  if (st != MOE_OK) return st;
  if (L->alt_experts) return MOE_ERR_UNSUPPORTED;  // the second expert copy is read by decode
  if (L->d % 256) return MOE_ERR_UNSUPPORTED;  // the down GEMMs cover 256 columns per block
  if (!out || !aligned(out, 16)) return MOE_ERR_INVALID_ARG;
  const size_t bytes = (size_t)T * L->d * 2;
  if (overlaps(x, bytes, out, bytes)) return MOE_ERR_INVALID_ARG;
  const PrefillWs P = prefill_ws_layout(L, T);
  // the 2-bit and ternary kernels address their activation rows with 32-bit byte offsets
  if ((prefill_x2(L) || prefill_exact16(L)) && (size_t)P.rows * (size_t)(L->d > L->inter ? L->d : L->inter) * 2 >
                           (size_t)UINT32_MAX)
    return MOE_ERR_UNSUPPORTED;
  return launch_prefill(L, x, T, flags, R, (uint8_t*)ws, P, out, stream, mask) ? MOE_ERR_DEVICE
                                                                             : MOE_OK;
}

extern "C" moe_status moe_forward_decode(const moe_layer* L, const uint16_t* x, int32_t T,
                                         uint32_t flags, moe_routing* R, void* ws,
                                         size_t ws_bytes, uint16_t* out, void* stream) {
  return decode_impl(L, x, T, flags, R, ws, ws_bytes, out, ~0u, stream);
}

extern "C" moe_status moe_forward_prefill(const moe_layer* L, const uint16_t* x, int32_t T,
                                          uint32_t flags, moe_routing* R, void* ws,
                                          size_t ws_bytes, uint16_t* out, void* stream) {
  return prefill_impl(L, x, T, flags, R, ws, ws_bytes, out, ~0u, stream);
}

extern "C" moe_status moe_forward_decode_stages(const moe_layer* L, const uint16_t* x, int32_t T,
                                                uint32_t flags, moe_routing* R, void* ws,
                                                size_t ws_bytes, uint16_t* out,
                                                uint32_t stage_mask, void* stream) {
  if (stage_mask == 0 || (stage_mask & ~(uint32_t)MOE_DECODE_STAGES_ALL)) return MOE_ERR_INVALID_ARG;
  return decode_impl(L, x, T, flags, R, ws, ws_bytes, out, stage_mask, stream);
}

extern "C" moe_status moe_forward_prefill_stages(const moe_layer* L, const uint16_t* x, int32_t T,
                                                 uint32_t flags, moe_routing* R, void* ws,
                                                 size_t ws_bytes, uint16_t* out,
                                                 uint32_t stage_mask, void* stream) {
  if (stage_mask == 0 || (stage_mask & ~(uint32_t)MOE_PREFILL_STAGES_ALL)) return MOE_ERR_INVALID_ARG;
  return prefill_impl(L, x, T, flags, R, ws, ws_bytes, out, stage_mask, stream);
}

extern "C" const char* moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape or type";
    case MOE_ERR_WORKSPACE: return "workspace too small";
    case MOE_ERR_BAD_CODES: return "level index outside its alphabet";
    case MOE_ERR_DEVICE: return "HIP launch or runtime error";
  }
  return "unknown status";
}

extern "C" int moe_abi_version(void) { return 3; }
