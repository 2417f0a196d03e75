"""Inputs on which the whole layer is exact in fp32, so the GPU must equal the
oracle bit for bit (the packed layout read back through the kernels).

Construction (every choice serves exactness; the codes stay the generator's):
  - x[t] = a_t * e_{i_t}: one non-zero entry a_t = +-1 per token, so each gate and
    up output is a single product s * c * a, exact in any precision that holds it;
  - gate scales +-2^8 (sign drawn per group): every gate output g is 0 or has
    |g| >= 128, where SiLU(g) is g itself (g > 0) or rounds to a signed zero
    (g < 0) on both sides, so h = bf16(SiLU(g) * u) is exact;
  - up scales +-2^-1: h is then (2^7 / 4) * m with m a product of two odd code
    values (|m| <= 49), one unit for the whole row;
  - down scales +-2^-2 or +-2^-1 (exponent and sign drawn per group): every
    product, 32-group sum and group-scaled sum of the down projection is a
    multiple of one unit below 2^24 units, so the kernels' fp32 sums are exact
    in any order; y is the bf16 rounding of an exact value on both sides;
  - top-1 routing with a shared expert and no residual: the weight is exactly 1
    and out = bf16(y + y_shared) has a single fp32 rounding, which a following
    bf16 rounding cannot change (fp32 carries more than twice bf16's bits).
check_premise() verifies the numeric conditions on the oracle's own
pre-rounding values.
"""
from __future__ import annotations

import numpy as np

import oracle
import synth

GATE_EXP = 8
UP_EXP = -1
DOWN_EXPS = (-2, -1)


def _pow2_scales(bits: np.ndarray, exps, signed=True) -> np.ndarray:
    """fp16 bits of +-2^e, e and the sign taken from the generator's scale bits."""
    bits = bits.astype(np.uint32)
    e = np.asarray(exps)[(bits >> 3) % len(exps)]
    v = np.exp2(e.astype(np.float64))
    if signed:
        v = np.where((bits >> 1) & 1, -v, v)
    return v.astype(np.float16).view(np.uint16)


def exact_mats(cfg: synth.Config, layer: int = 0):
    """mats(e) for workloads.DeviceLayer / helpers.oracle_outputs."""
    def mats(e):
        out = []
        for m, exps in ((0, (GATE_EXP,)), (1, (UP_EXP,)), (2, DOWN_EXPS)):
            c, s = synth.gen_matrix(cfg, layer, e, m)
            out.append((c, _pow2_scales(s, exps)))
        return out
    return mats


def basis_tokens(d: int, T: int, seed: int, positions=None):
    """x [T][d] bf16 with one entry +-1 per token, and the positions used."""
    rng = np.random.default_rng(seed)
    pos = np.asarray(positions) if positions is not None else rng.integers(0, d, T)
    sign = rng.integers(0, 2, T)
    x = np.zeros((T, d), np.uint16)
    x[np.arange(T), pos] = np.where(sign, 0xBF80, 0x3F80)  # bf16 -1.0 / +1.0
    return x, pos


def top1_logits(experts: np.ndarray, E: int) -> np.ndarray:
    """Given logits that route token t to experts[t] (1.0 there, 0.0 elsewhere)."""
    lg = np.zeros((len(experts), E), np.float32)
    lg[np.arange(len(experts)), experts] = 1.0
    return lg


def check_premise(cfg: synth.Config, mats, x: np.ndarray, experts: np.ndarray):
    """The numeric conditions above, on the oracle's pre-rounding values of every
    (token, expert) pair the routing uses, the shared expert included."""
    pairs = {}
    for t, e in enumerate(experts):
        pairs.setdefault(int(e), []).append(t)
    if cfg.n_shared:
        pairs[cfg.E] = list(range(len(x)))
    for e, toks in pairs.items():
        h, y, g, u, ypre = oracle.expert_rows(cfg.qtypes, mats(e), x[toks], want_pre=True)
        for name, v in (("g", g), ("u", u), ("y", ypre)):
            assert np.array_equal(v.astype(np.float32).astype(np.float64), v), (e, name)
        nz = g[g != 0]
        assert np.all(np.abs(nz) >= 128.0), e
        hv = oracle.bf16_to_f64(h)
        unit = 2.0 ** (GATE_EXP + UP_EXP) / 4
        m = hv / unit
        assert np.array_equal(m, np.round(m)) and np.abs(m).max() <= 49, e
        # h is the exact product (no rounding at the h point)
        silu_g = np.where(g > 0, g, 0.0)
        assert np.array_equal(hv, silu_g * u), e
        # every partial sum of the down projection, in any order, stays below 2^24 of its
        # unit (2^(GATE_EXP + UP_EXP - 2) * 2^(min down exponent) * 0.5)
        cd, sd = mats(e)[2]
        wd = np.abs(oracle.dequant(cfg.qtypes[2], cd, sd))
        unit_y = unit * 2.0 ** min(DOWN_EXPS) * 0.5
        assert (np.abs(hv) @ wd).max() < 2.0 ** 24 * unit_y, e
