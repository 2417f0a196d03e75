"""Seeded synthetic inputs for the quantized MoE expert layer.

This package only draws random numbers and stores them in the input dtypes; it
holds none of the layer's arithmetic.  The CPU oracle's tests and the GPU
path's tests and benchmark both take their inputs from here.

Every tensor is a counter-based stream identified by ``(seed, stream)``: see
``gen.c`` for the generator.  ``stream_id`` names the tensor (what it is, which
layer, which expert, which projection), so any expert of any layer can be
regenerated on its own.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass, field

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsynth.so")
_lib = None

# tensor kinds used in stream ids
KIND_X = 1
KIND_ROUTER = 2
KIND_CODES = 3
KIND_SCALES = 4
KIND_LOGITS = 5
KIND_ZIPF = 6
KIND_MISC = 7

MAT_GATE, MAT_UP, MAT_DOWN = 0, 1, 2

QT_TERNARY, QT_INT2, QT_INT3 = 1, 2, 3
LEVELS = {QT_TERNARY: 3, QT_INT2: 4, QT_INT3: 8}
QNAME = {QT_TERNARY: "ternary", QT_INT2: "int2", QT_INT3: "int3"}


def build(verbose: bool = False) -> str:
    """Compile gen.c into libsynth.so (gcc, OpenMP).  Always recompiles."""
    src = os.path.join(_HERE, "gen.c")
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", src, "-o", tmp, "-lm"]
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
    u64, i64, p = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
    d = ctypes.c_double
    lib.synth_u64.argtypes = [u64, u64, u64, i64, p]
    lib.synth_normal_f64.argtypes = [u64, u64, u64, i64, d, d, p]
    lib.synth_normal_f32.argtypes = [u64, u64, u64, i64, d, d, p]
    lib.synth_normal_bf16.argtypes = [u64, u64, u64, i64, d, d, p]
    lib.synth_absnormal_f16.argtypes = [u64, u64, u64, i64, d, p]
    lib.synth_codes.argtypes = [u64, u64, u64, i64, ctypes.c_int, p]
    for f in (lib.synth_u64, lib.synth_normal_f64, lib.synth_normal_f32, lib.synth_normal_bf16,
              lib.synth_absnormal_f16, lib.synth_codes):
        f.restype = None
    _lib = lib
    return lib


def stream_id(kind: int, layer: int = 0, expert: int = 0, mat: int = 0) -> int:
    return ((kind * 256 + layer) * 65536 + expert) * 8 + mat


def _ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def u64(seed, stream, n, start=0):
    out = np.empty(n, np.uint64)
    _load().synth_u64(seed, stream, start, n, _ptr(out))
    return out


def normal_f64(seed, stream, n, mean=0.0, sigma=1.0, start=0):
    out = np.empty(n, np.float64)
    _load().synth_normal_f64(seed, stream, start, n, mean, sigma, _ptr(out))
    return out


def normal_f32(seed, stream, n, mean=0.0, sigma=1.0, start=0):
    out = np.empty(n, np.float32)
    _load().synth_normal_f32(seed, stream, start, n, mean, sigma, _ptr(out))
    return out


def normal_bf16(seed, stream, n, mean=0.0, sigma=1.0, start=0):
    """bf16 bit patterns (uint16) of N(mean, sigma)."""
    out = np.empty(n, np.uint16)
    _load().synth_normal_bf16(seed, stream, start, n, mean, sigma, _ptr(out))
    return out


def absnormal_f16(seed, stream, n, sigma, start=0):
    """fp16 bit patterns (uint16) of |N(0, sigma)|."""
    out = np.empty(n, np.uint16)
    _load().synth_absnormal_f16(seed, stream, start, n, sigma, _ptr(out))
    return out


def codes(seed, stream, n, levels, start=0):
    out = np.empty(n, np.uint8)
    _load().synth_codes(seed, stream, start, n, levels, _ptr(out))
    return out


def uniform01(seed, stream, n):
    """Uniform in (0, 1] from the same counter stream (float64)."""
    return ((u64(seed, stream, n) >> np.uint64(11)).astype(np.float64) + 1.0) * (2.0 ** -53)


def seeded_permutation(seed, stream, n):
    """Fisher-Yates shuffle of range(n) driven by counter draws."""
    r = u64(seed, stream, n)
    perm = np.arange(n, dtype=np.int64)
    for i in range(n - 1, 0, -1):
        j = int((int(r[i]) >> 11) % (i + 1))
        perm[i], perm[j] = perm[j], perm[i]
    return perm


def zipf_log_prior(seed, E, s, layer=0):
    """Per-expert additive log-prior ln p_e, p_e proportional to rank_e^-s.

    Ranks are a seeded permutation of the expert ids, so the most popular
    experts are not simply the lowest ids.  Returned as float32.
    """
    perm = seeded_permutation(seed, stream_id(KIND_ZIPF, layer), E)
    rank = np.empty(E, np.float64)
    rank[perm] = np.arange(1, E + 1, dtype=np.float64)
    w = rank ** (-float(s))
    return np.log(w / w.sum()).astype(np.float32)


# --------------------------------------------------------------------------
# Workload configurations (all shapes and distributions of the five cases).
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Config:
    name: str
    T: int
    d: int
    E: int
    k: int
    inter: int
    n_shared: int
    q_gate: int
    q_up: int
    q_down: int
    seed: int
    router: bool            # True: logits from x . W_r; False: logits given
    router_sigma: float = 0.02
    zipf_s: float = 0.0     # 0 = no popularity bias
    layers: int = 1
    residual: bool = False
    scale_sigma: float = 0.05
    note: str = ""

    @property
    def qtypes(self):
        return (self.q_gate, self.q_up, self.q_down)


CONFIGS = {
    "c0": Config("c0_tiny", T=4, d=256, E=8, k=2, inter=128, n_shared=0,
                 q_gate=QT_INT2, q_up=QT_INT2, q_down=QT_INT2, seed=0, router=True,
                 note="tiny layer, oracle-sized"),
    "c1": Config("c1_decode_t1", T=1, d=4096, E=256, k=8, inter=2048, n_shared=1,
                 q_gate=QT_INT2, q_up=QT_INT2, q_down=QT_INT2, seed=1, router=True,
                 note="decode one token, 256 experts top-8 + shared, int2"),
    "c2": Config("c2_decode_t8_zipf", T=8, d=4096, E=256, k=8, inter=2048, n_shared=1,
                 q_gate=QT_INT3, q_up=QT_INT3, q_down=QT_INT2, seed=2, router=True, zipf_s=1.1,
                 note="decode 8 tokens, gate/up int3, down int2, Zipf(1.1) router bias"),
    "c3": Config("c3_prefill_t8192", T=8192, d=4096, E=256, k=8, inter=2048, n_shared=1,
                 q_gate=QT_INT2, q_up=QT_INT2, q_down=QT_INT2, seed=3, router=False,
                 note="prefill 8192 tokens, logits N(0,1) given, int2"),
    "c4": Config("c4_prefill_t16384_4l", T=16384, d=4096, E=256, k=8, inter=2048, n_shared=1,
                 q_gate=QT_TERNARY, q_up=QT_TERNARY, q_down=QT_TERNARY, seed=4, router=False,
                 zipf_s=1.2, layers=4, residual=True,
                 note="prefill 16384 tokens, 4 layers with residual, ternary, logits N(0,1)+Zipf(1.2)"),
}


def expert_index_for_stream(cfg: Config, e: int) -> int:
    """Stream expert index: routed experts 0..E-1, the shared expert is E."""
    return e


def matrix_shape(cfg: Config, mat: int):
    """(K, N) of projection `mat`: gate/up are d -> inter, down is inter -> d."""
    return (cfg.d, cfg.inter) if mat in (MAT_GATE, MAT_UP) else (cfg.inter, cfg.d)


def gen_matrix(cfg: Config, layer: int, expert: int, mat: int, seed: int | None = None):
    """Canonical codes [N][K] (uint8 level index) and scales [N][K/32] (fp16 bits)."""
    seed = cfg.seed if seed is None else seed
    K, N = matrix_shape(cfg, mat)
    q = cfg.qtypes[mat]
    c = codes(seed, stream_id(KIND_CODES, layer, expert, mat), N * K, LEVELS[q]).reshape(N, K)
    s = absnormal_f16(seed, stream_id(KIND_SCALES, layer, expert, mat), N * (K // 32),
                      cfg.scale_sigma).reshape(N, K // 32)
    return c, s


def gen_x(cfg: Config, seed: int | None = None, T: int | None = None):
    seed = cfg.seed if seed is None else seed
    T = cfg.T if T is None else T
    return normal_bf16(seed, stream_id(KIND_X), T * cfg.d).reshape(T, cfg.d)


def gen_router(cfg: Config, layer: int = 0, seed: int | None = None):
    """Router weight, stored [E][d] fp32 (expert e's column of the logical [d][E] matrix)."""
    seed = cfg.seed if seed is None else seed
    return normal_f32(seed, stream_id(KIND_ROUTER, layer), cfg.E * cfg.d, 0.0,
                      cfg.router_sigma).reshape(cfg.E, cfg.d)


def gen_bias(cfg: Config, layer: int = 0, seed: int | None = None):
    """Additive router bias [E] fp32 (Zipf log-prior), or None."""
    if not cfg.zipf_s:
        return None
    seed = cfg.seed if seed is None else seed
    return zipf_log_prior(seed, cfg.E, cfg.zipf_s, layer)


def gen_logits(cfg: Config, layer: int = 0, seed: int | None = None, T: int | None = None):
    """Given logits [T][E] fp32: N(0,1) plus the Zipf log-prior when the config has one."""
    seed = cfg.seed if seed is None else seed
    T = cfg.T if T is None else T
    base = normal_f64(seed, stream_id(KIND_LOGITS, layer), T * cfg.E).reshape(T, cfg.E)
    b = gen_bias(cfg, layer, seed)
    if b is not None:
        base = base + b.astype(np.float64)[None, :]
    return base.astype(np.float32)


def small_config(base: Config, **kw) -> Config:
    """A copy of `base` with some fields replaced (for test cases)."""
    d = dict(base.__dict__)
    d.update(kw)
    return Config(**d)
