"""Quantized mixture-of-experts expert layer for AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libbqmoe.so`` (C ABI declared in ``include/moe.h``).
Every step of the layer runs in the library's HIP kernels; this module only
marshals arguments: torch tensors provide device memory and the stream.  If
the library is missing the import fails loudly -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import numpy as np
import torch  # load torch's HIP runtime first: libbqmoe.so binds to the same one

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbqmoe.so")
ABI_VERSION = 3  # moe_abi_version() of the include/moe.h this binding follows

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_BAD_CODES, \
    MOE_ERR_DEVICE = range(6)
MOE_Q_TERNARY, MOE_Q_INT2, MOE_Q_INT3 = 1, 2, 3
MOE_LOGITS_GIVEN, MOE_ADD_RESIDUAL = 1, 2
MOE_MAX_DECODE_TOKENS = 8
MOE_DECODE_STAGE_ROUTE, MOE_DECODE_STAGE_SELECT, MOE_DECODE_STAGE_GATEUP, MOE_DECODE_STAGE_DOWN = \
    1, 2, 4, 8
MOE_DECODE_STAGES_ALL = 15
MOE_PREFILL_STAGE_ROUTE, MOE_PREFILL_STAGE_STAGE_X, MOE_PREFILL_STAGE_GATEUP, \
    MOE_PREFILL_STAGE_DOWN, MOE_PREFILL_STAGE_COMBINE = 1, 2, 4, 8, 16
MOE_PREFILL_STAGES_ALL = 31
MOE_NOALLOC_SCRATCH_BYTES = 4 << 20

EXPORTED = ("moe_packed_bytes", "moe_expert_bytes", "moe_pack_weights", "moe_quantize_rtn",
            "moe_requantize", "moe_workspace_bytes",
            "moe_route_topk", "moe_forward_decode", "moe_forward_prefill",
            "moe_forward_decode_stages", "moe_forward_prefill_stages",
            "moe_forward_decode_noalloc", "moe_status_string", "moe_abi_version")


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


class moe_layer(ctypes.Structure):
    _fields_ = [("d", ctypes.c_int32), ("inter", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_shared", ctypes.c_int32), ("q_gate", ctypes.c_int32),
                ("q_up", ctypes.c_int32), ("q_down", ctypes.c_int32),
                ("router_w", ctypes.c_void_p), ("router_bias", ctypes.c_void_p),
                ("experts", ctypes.c_void_p), ("expert_stride", ctypes.c_size_t),
                ("shared", ctypes.c_void_p),
                ("alt_experts", ctypes.c_void_p), ("alt_stride", ctypes.c_size_t),
                ("q_alt_gate", ctypes.c_int32), ("q_alt_up", ctypes.c_int32),
                ("q_alt_down", ctypes.c_int32), ("alt_select", ctypes.c_void_p)]


class moe_routing(ctypes.Structure):
    _fields_ = [("logits", ctypes.c_void_p), ("topk_ids", ctypes.c_void_p),
                ("topk_w", ctypes.c_void_p), ("counts", ctypes.c_void_p),
                ("offsets", ctypes.c_void_p), ("perm_tok", ctypes.c_void_p),
                ("inv_row", ctypes.c_void_p)]


_lib = None


def load():
    """Load libbqmoe.so (built in-tree by ``build.py``); raise if it is absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it first (python -c "
                          "'import __graft_entry__ as g; g.build()').  There is no CPU fallback.")
    if torch.cuda.is_available():
        # bring the HIP runtime up before the library registers its code objects
        torch.cuda.init()
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32, i64, u32 = (ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int64,
                             ctypes.c_uint32)
    L, R = ctypes.POINTER(moe_layer), ctypes.POINTER(moe_routing)
    lib.moe_packed_bytes.argtypes, lib.moe_packed_bytes.restype = [i32, i64, i64], sz
    lib.moe_expert_bytes.argtypes, lib.moe_expert_bytes.restype = [i32, i32, i32, i64, i64], sz
    lib.moe_pack_weights.argtypes, lib.moe_pack_weights.restype = [i32, i64, i64, vp, vp, vp,
                                                                   sz], i32
    lib.moe_quantize_rtn.argtypes, lib.moe_quantize_rtn.restype = [i32, i64, i64, vp, vp, vp], i32
    lib.moe_requantize.argtypes = [i32, i32, i64, i64, vp, sz, vp, sz]
    lib.moe_requantize.restype = i32
    lib.moe_workspace_bytes.argtypes, lib.moe_workspace_bytes.restype = [L, ctypes.c_int32], sz
    lib.moe_route_topk.argtypes = [L, vp, ctypes.c_int32, u32, R, vp, sz, vp]
    lib.moe_forward_decode.argtypes = [L, vp, ctypes.c_int32, u32, R, vp, sz, vp, vp]
    lib.moe_forward_prefill.argtypes = [L, vp, ctypes.c_int32, u32, R, vp, sz, vp, vp]
    lib.moe_forward_decode_stages.argtypes = [L, vp, ctypes.c_int32, u32, R, vp, sz, vp, u32, vp]
    lib.moe_forward_prefill_stages.argtypes = [L, vp, ctypes.c_int32, u32, R, vp, sz, vp, u32, vp]
    lib.moe_forward_decode_noalloc.argtypes = [L, vp, ctypes.c_int32, u32, R, vp, vp]
    for f in (lib.moe_route_topk, lib.moe_forward_decode, lib.moe_forward_prefill,
              lib.moe_forward_decode_stages, lib.moe_forward_prefill_stages,
              lib.moe_forward_decode_noalloc):
        f.restype = i32
    lib.moe_status_string.argtypes, lib.moe_status_string.restype = [i32], ctypes.c_char_p
    lib.moe_abi_version.argtypes, lib.moe_abi_version.restype = [], i32
    if lib.moe_abi_version() != ABI_VERSION:
        # moe_layer's layout depends on it: a stale build would misread every layer
        raise ImportError(f"{LIB_PATH}: ABI version {lib.moe_abi_version()}, this binding needs "
                          f"{ABI_VERSION}; rebuild the library")
    _lib = lib
    return lib


def status_string(status: int) -> str:
    try:
        return load().moe_status_string(int(status)).decode()
    except ImportError:
        return "unknown"


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if isinstance(t, np.ndarray):
        return t.ctypes.data
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return ctypes.c_void_p(stream.cuda_stream)
    return ctypes.c_void_p(int(stream))


def _check(status, what):
    if status != MOE_OK:
        raise MoeError(int(status), what)


# ------------------------------------------------------------- format
def moe_packed_bytes(qtype: int, K: int, N: int) -> int:
    return int(load().moe_packed_bytes(qtype, K, N))


def moe_expert_bytes(q_gate: int, q_up: int, q_down: int, d: int, inter: int) -> int:
    return int(load().moe_expert_bytes(q_gate, q_up, q_down, d, inter))


def moe_pack_weights(qtype: int, codes: np.ndarray, scales: np.ndarray,
                     out: np.ndarray | None = None) -> np.ndarray:
    """Pack one projection (codes [N][K] uint8 levels, scales [N][K/32] fp16 bits) on the host."""
    codes = np.ascontiguousarray(codes, np.uint8)
    scales = np.ascontiguousarray(scales, np.uint16)
    N, K = codes.shape
    nbytes = moe_packed_bytes(qtype, K, N)
    if out is None:
        out = np.empty(max(nbytes, 1), np.uint8)
    st = load().moe_pack_weights(qtype, K, N, _ptr(codes), _ptr(scales), _ptr(out), out.nbytes)
    _check(st, "moe_pack_weights")
    return out[:nbytes]


def moe_quantize_rtn(qtype: int, w: np.ndarray):
    """Round-to-nearest codes [N][K] (uint8) and fp16 scale bits [N][K/32] of float weights
    w[N][K] on the host (moe_quantize_rtn)."""
    w = np.ascontiguousarray(w, np.float32)
    N, K = w.shape
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((N, max(K // 32, 1)), np.uint16)
    st = load().moe_quantize_rtn(qtype, K, N, _ptr(w), _ptr(codes), _ptr(scales))
    _check(st, "moe_quantize_rtn")
    return codes, scales[:, : K // 32]


def moe_requantize(q_src: int, q_dst: int, K: int, N: int, blob: np.ndarray) -> np.ndarray:
    """The packed projection `blob` (q_src, K x N) re-quantised to q_dst, on the host
    (moe_requantize); returns the new packed bytes."""
    blob = np.ascontiguousarray(blob, np.uint8)
    out = np.zeros(moe_packed_bytes(q_dst, K, N), np.uint8)
    st = load().moe_requantize(q_src, q_dst, K, N, _ptr(blob), blob.nbytes, _ptr(out), out.nbytes)
    _check(st, "moe_requantize")
    return out


# -------------------------------------------------------------- layer
@dataclass
class Layer:
    """A moe_layer plus the tensors it points into (kept alive here)."""
    c: moe_layer
    tensors: tuple


def make_layer(d, inter, n_experts, top_k, n_shared, qtypes, experts, expert_stride,
               shared=None, router_w=None, router_bias=None, alt=None) -> Layer:
    """alt = (alt_experts, alt_stride, alt_qtypes, alt_select): a second copy of the routed
    experts in other code families and the device byte mask [E] choosing it per expert."""
    qg, qu, qd = qtypes
    ae, astride, aq, asel = alt if alt is not None else (None, 0, (0, 0, 0), None)
    c = moe_layer(d, inter, n_experts, top_k, n_shared, qg, qu, qd, _ptr(router_w),
                  _ptr(router_bias), _ptr(experts), expert_stride, _ptr(shared),
                  _ptr(ae), astride, aq[0], aq[1], aq[2], _ptr(asel))
    return Layer(c, (experts, shared, router_w, router_bias, ae, asel))


@dataclass
class Routing:
    c: moe_routing
    logits: torch.Tensor
    topk_ids: torch.Tensor
    topk_w: torch.Tensor
    counts: torch.Tensor
    offsets: torch.Tensor
    perm_tok: torch.Tensor
    inv_row: torch.Tensor


def alloc_routing(T: int, E: int, k: int, device="cuda", logits: torch.Tensor | None = None) -> Routing:
    """Device buffers for the routing outputs (logits may be given as an input)."""
    f32, i32 = torch.float32, torch.int32
    lg = logits if logits is not None else torch.empty((T, E), dtype=f32, device=device)
    ids = torch.empty((T, k), dtype=i32, device=device)
    w = torch.empty((T, k), dtype=f32, device=device)
    counts = torch.empty(E, dtype=i32, device=device)
    offsets = torch.empty(E + 1, dtype=i32, device=device)
    perm = torch.empty(max(T * k, 1), dtype=i32, device=device)
    inv = torch.empty((T, k), dtype=i32, device=device)
    c = moe_routing(_ptr(lg), _ptr(ids), _ptr(w), _ptr(counts), _ptr(offsets), _ptr(perm),
                    _ptr(inv))
    return Routing(c, lg, ids, w, counts, offsets, perm, inv)


def moe_workspace_bytes(layer: Layer, T: int) -> int:
    return int(load().moe_workspace_bytes(ctypes.byref(layer.c), T))


def alloc_workspace(layer: Layer, T: int, device="cuda") -> torch.Tensor:
    n = moe_workspace_bytes(layer, T)
    if n == 0:
        raise MoeError(MOE_ERR_INVALID_ARG, "moe_workspace_bytes")
    return torch.empty(n, dtype=torch.uint8, device=device)


def moe_route_topk(layer: Layer, x, T: int, flags: int, routing: Routing, ws, stream=None):
    st = load().moe_route_topk(ctypes.byref(layer.c), _ptr(x), T, flags, ctypes.byref(routing.c),
                               _ptr(ws), 0 if ws is None else ws.numel(), _stream(stream))
    _check(st, "moe_route_topk")


def moe_forward_decode(layer: Layer, x, T: int, flags: int, routing: Routing, ws, out,
                       stream=None):
    st = load().moe_forward_decode(ctypes.byref(layer.c), _ptr(x), T, flags,
                                   ctypes.byref(routing.c), _ptr(ws),
                                   0 if ws is None else ws.numel(), _ptr(out), _stream(stream))
    _check(st, "moe_forward_decode")


def moe_forward_decode_noalloc(layer: Layer, x, T: int, flags: int, routing: Routing, out,
                               stream=None):
    """moe_forward_decode with the library's static device workspace (no ws argument)."""
    st = load().moe_forward_decode_noalloc(ctypes.byref(layer.c), _ptr(x), T, flags,
                                           ctypes.byref(routing.c), _ptr(out), _stream(stream))
    _check(st, "moe_forward_decode_noalloc")


def moe_forward_prefill(layer: Layer, x, T: int, flags: int, routing: Routing, ws, out,
                        stream=None):
    st = load().moe_forward_prefill(ctypes.byref(layer.c), _ptr(x), T, flags,
                                    ctypes.byref(routing.c), _ptr(ws),
                                    0 if ws is None else ws.numel(), _ptr(out), _stream(stream))
    _check(st, "moe_forward_prefill")


def moe_forward_decode_stages(layer: Layer, x, T: int, flags: int, routing: Routing, ws, out,
                              stage_mask: int, stream=None):
    st = load().moe_forward_decode_stages(ctypes.byref(layer.c), _ptr(x), T, flags,
                                          ctypes.byref(routing.c), _ptr(ws),
                                          0 if ws is None else ws.numel(), _ptr(out), stage_mask,
                                          _stream(stream))
    _check(st, "moe_forward_decode_stages")


def moe_forward_prefill_stages(layer: Layer, x, T: int, flags: int, routing: Routing, ws, out,
                               stage_mask: int, stream=None):
    st = load().moe_forward_prefill_stages(ctypes.byref(layer.c), _ptr(x), T, flags,
                                           ctypes.byref(routing.c), _ptr(ws),
                                           0 if ws is None else ws.numel(), _ptr(out),
                                           stage_mask, _stream(stream))
    _check(st, "moe_forward_prefill_stages")


def moe_abi_version() -> int:
    return int(load().moe_abi_version())
