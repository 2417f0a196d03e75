"""CPU oracle for the quantized MoE expert layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The GPU library never uses it.

This is a thin numpy/ctypes wrapper over ``oracle.c`` (plain C, double
precision); see that file's header for what each function computes and the
passage it follows.  Parity status of every function is recorded in the
tests that pin it (``tests/test_oracle_*.py``); none is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None

QT_TERNARY, QT_INT2, QT_INT3 = 1, 2, 3


def build(verbose: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math).  Always recompiles."""
    src = os.path.join(_HERE, "oracle.c")
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11",
           src, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    p, i32, i64, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_size_t
    lib.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_bf16_to_f64.restype = ctypes.c_double
    lib.oracle_f64_to_bf16.argtypes = [ctypes.c_double]
    lib.oracle_f64_to_bf16.restype = ctypes.c_uint16
    lib.oracle_f16_to_f64.argtypes = [ctypes.c_uint16]
    lib.oracle_f16_to_f64.restype = ctypes.c_double
    lib.oracle_packed_bytes.argtypes = [i32, i64, i64]
    lib.oracle_packed_bytes.restype = sz
    lib.oracle_unpack.argtypes = [i32, i64, i64, p, sz, p, p]
    lib.oracle_dequant.argtypes = [i32, i64, i64, p, p, p]
    lib.oracle_quantize_rtn.argtypes = [i32, i64, i64, p, p, p]
    lib.oracle_router_logits.argtypes = [i32, i32, i32, p, p, p, p]
    lib.oracle_topk_softmax.argtypes = [i32, i32, i32, p, p, p]
    lib.oracle_permute.argtypes = [i32, i32, i32, p, p, p, p, p]
    lib.oracle_expert_rows.argtypes = [i32, i32, i32, i32, i32, p, p, p, p, p, p, i32, p, p, p,
                                       p, p, p]
    lib.oracle_combine.argtypes = [i32, i32, i32, p, p, p, p, p, i32, p, p]
    lib.oracle_moe_layer.argtypes = [i32] * 9 + [p, p, p, i32, p, p, p, i32, p, p, p, p, p, p, p]
    for name in ("oracle_unpack", "oracle_dequant", "oracle_quantize_rtn", "oracle_router_logits",
                 "oracle_topk_softmax",
                 "oracle_permute", "oracle_expert_rows", "oracle_combine", "oracle_moe_layer"):
        getattr(lib, name).restype = ctypes.c_int
    _lib = lib
    return lib


def _p(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    pass


def _ok(rc, what):
    if rc != 0:
        raise OracleError(f"{what} rejected its input (status {rc})")


# ------------------------------------------------------------------ numbers
def bf16_to_f64(bits):
    bits = np.asarray(bits, np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def f64_to_bf16(v):
    """Round-to-nearest-even bf16 of each double (the oracle's converter)."""
    lib = _load()
    v = np.asarray(v, np.float64)
    out = np.empty(v.shape, np.uint16)
    flat_in, flat_out = v.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = lib.oracle_f64_to_bf16(float(flat_in[i]))
    return out


def f16_to_f64(bits):
    lib = _load()
    bits = np.asarray(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    fi, fo = bits.reshape(-1), out.reshape(-1)
    for i in range(fi.size):
        fo[i] = lib.oracle_f16_to_f64(int(fi[i]))
    return out


# ------------------------------------------------------------ packed format
def packed_bytes(qtype, K, N):
    return int(_load().oracle_packed_bytes(qtype, K, N))


def unpack(qtype, K, N, blob):
    blob = _c(np.frombuffer(bytes(blob), np.uint8) if not isinstance(blob, np.ndarray) else blob,
              np.uint8)
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((N, K // 32), np.uint16)
    _ok(_load().oracle_unpack(qtype, K, N, _p(blob), blob.nbytes, _p(codes), _p(scales)), "unpack")
    return codes, scales


def quantize_rtn(qtype, w):
    """Round-to-nearest codes [N][K] and fp16 scale bits [N][K/32] of float weights w[N][K]."""
    w = _c(w, np.float32)
    N, K = w.shape
    codes = np.empty((N, K), np.uint8)
    scales = np.empty((N, K // 32), np.uint16)
    _ok(_load().oracle_quantize_rtn(qtype, K, N, _p(w), _p(codes), _p(scales)), "quantize_rtn")
    return codes, scales


def dequant(qtype, codes, scales):
    codes = _c(codes, np.uint8)
    scales = _c(scales, np.uint16)
    N, K = codes.shape
    W = np.empty((K, N), np.float64)
    _ok(_load().oracle_dequant(qtype, K, N, _p(codes), _p(scales), _p(W)), "dequant")
    return W


def requantize(q_src, q_dst, K, N, blob):
    """Codes [N][K] and fp16 scale bits [N][K/32] of the packed projection `blob` (q_src)
    re-quantised to q_dst: the oracle's own decoder, dequantisation (exact in fp32) and
    round-to-nearest quantiser."""
    codes, scales = unpack(q_src, K, N, blob)
    w = np.ascontiguousarray(dequant(q_src, codes, scales).T)  # [N][K]
    w32 = w.astype(np.float32)
    assert np.array_equal(w32.astype(np.float64), w)
    return quantize_rtn(q_dst, w32)


# ------------------------------------------------------------------ routing

def router_logits(x_bf16, Wr, bias=None):
    x = _c(x_bf16, np.uint16)
    Wr = _c(Wr, np.float32)
    T, d = x.shape
    E = Wr.shape[0]
    b = None if bias is None else _c(bias, np.float32)
    out = np.empty((T, E), np.float32)
    _ok(_load().oracle_router_logits(T, d, E, _p(x), _p(Wr), _p(b), _p(out)), "router_logits")
    return out


def topk_softmax(logits, k):
    L = _c(logits, np.float32)
    T, E = L.shape
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    _ok(_load().oracle_topk_softmax(T, E, k, _p(L), _p(ids), _p(w)), "topk_softmax")
    return ids, w


def permute(ids, E):
    ids = _c(ids, np.int32)
    T, k = ids.shape
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm_tok = np.empty(T * k, np.int32)
    inv_row = np.empty((T, k), np.int32)
    _ok(_load().oracle_permute(T, E, k, _p(ids), _p(counts), _p(offsets), _p(perm_tok),
                               _p(inv_row)), "permute")
    return counts, offsets, perm_tok, inv_row


# ------------------------------------------------------------------- expert
def expert_rows(qtypes, mats, x_rows, want_pre=False):
    """mats = ((codes_g, scales_g), (codes_u, scales_u), (codes_d, scales_d)).

    Returns (h bf16 [M][I], y bf16 [M][d]) and, with want_pre, also the
    unrounded g, u [M][I] and y [M][d] in double.
    """
    (cg, sg), (cu, su), (cd, sd) = mats
    cg, cu, cd = _c(cg, np.uint8), _c(cu, np.uint8), _c(cd, np.uint8)
    sg, su, sd = _c(sg, np.uint16), _c(su, np.uint16), _c(sd, np.uint16)
    I, d = cg.shape
    x = _c(x_rows, np.uint16).reshape(-1, d)
    M = x.shape[0]
    h = np.empty((M, I), np.uint16)
    y = np.empty((M, d), np.uint16)
    g_pre = np.empty((M, I), np.float64) if want_pre else None
    u_pre = np.empty((M, I), np.float64) if want_pre else None
    y_pre = np.empty((M, d), np.float64) if want_pre else None
    qg, qu, qd = qtypes
    _ok(_load().oracle_expert_rows(d, I, qg, qu, qd, _p(cg), _p(sg), _p(cu), _p(su), _p(cd),
                                   _p(sd), M, _p(x), _p(h), _p(y), _p(g_pre), _p(u_pre),
                                   _p(y_pre)), "expert_rows")
    if want_pre:
        return h, y, g_pre, u_pre, y_pre
    return h, y


def combine(w, inv_row, y, y_shared, x, residual, want_pre=False):
    w = _c(w, np.float32)
    inv = _c(inv_row, np.int32)
    T, k = w.shape
    y = _c(y, np.uint16)
    d = y.shape[-1]
    ysh = None if y_shared is None else _c(y_shared, np.uint16)
    xx = None if x is None else _c(x, np.uint16)
    out = np.empty((T, d), np.uint16)
    pre = np.empty((T, d), np.float64) if want_pre else None
    _ok(_load().oracle_combine(T, d, k, _p(w), _p(inv), _p(y), _p(ysh), _p(xx), int(residual),
                               _p(out), _p(pre)), "combine")
    return (out, pre) if want_pre else out


def moe_layer(cfg_shape, x, experts, Wr=None, bias=None, logits=None, residual=False):
    """The whole layer on the CPU.

    cfg_shape = (E, k, inter, n_shared, (qg, qu, qd)); experts = list of
    ((cg, sg), (cu, su), (cd, sd)) for expert 0..E-1 and then the shared one.
    Returns dict with logits, ids, w, counts, offsets, perm_tok, inv_row, out.
    """
    E, k, I, S, (qg, qu, qd) = cfg_shape
    x = _c(x, np.uint16)
    T, d = x.shape
    given = logits is not None
    L = _c(logits, np.float32).copy() if given else np.empty((T, E), np.float32)
    Wr_c = None if Wr is None else _c(Wr, np.float32)
    b = None if bias is None else _c(bias, np.float32)
    keep = []
    cp = (ctypes.c_void_p * ((E + S) * 3))()
    sp = (ctypes.c_void_p * ((E + S) * 3))()
    for e, mats in enumerate(experts[: E + S]):
        for m, (c, s) in enumerate(mats):
            c = _c(c, np.uint8)
            s = _c(s, np.uint16)
            keep += [c, s]
            cp[e * 3 + m] = c.ctypes.data
            sp[e * 3 + m] = s.ctypes.data
    ids = np.empty((T, k), np.int32)
    w = np.empty((T, k), np.float32)
    counts = np.empty(E, np.int32)
    offsets = np.empty(E + 1, np.int32)
    perm_tok = np.empty(T * k, np.int32)
    inv_row = np.empty((T, k), np.int32)
    out = np.empty((T, d), np.uint16)
    lib = _load()
    rc = lib.oracle_moe_layer(T, d, E, k, I, S, qg, qu, qd, _p(x), _p(Wr_c), _p(b), int(given),
                              _p(L), ctypes.cast(cp, ctypes.c_void_p),
                              ctypes.cast(sp, ctypes.c_void_p), int(residual), _p(ids), _p(w),
                              _p(counts), _p(offsets), _p(perm_tok), _p(inv_row), _p(out))
    _ok(rc, "moe_layer")
    return dict(logits=L, ids=ids, w=w, counts=counts, offsets=offsets, perm_tok=perm_tok,
                inv_row=inv_row, out=out)
