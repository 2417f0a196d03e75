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
Variant (odd=...): the named projection's scales become +-2^e * (1 + m/1024)
with m odd, 11 significant bits, so that 0.75 s (the value of a +-1.5 code) is
not an fp16 value: a kernel that builds fp16 weight operands must then restore
the rounding residual exactly.  Then g * u is still exact in fp32 and h is its
single bf16 rounding, and the down projection's sums stay exact (both checked).
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


def _odd_scales(bits: np.ndarray, exps) -> np.ndarray:
    """fp16 bits of +-2^e * (1 + m/1024), m odd in [1, 1023]; e, m and the sign
    taken from the generator's scale bits."""
    bits = bits.astype(np.uint32)
    e = np.asarray(exps)[(bits >> 3) % len(exps)]
    m = 2 * ((bits >> 4) % 512) + 1
    v = np.exp2(e.astype(np.float64)) * (1.0 + m / 1024.0)
    v = np.where((bits >> 1) & 1, -v, v)
    return v.astype(np.float16).view(np.uint16)


PROJ = ("gate", "up", "down")


def exact_mats(cfg: synth.Config, layer: int = 0, odd: str = ""):
    """mats(e) for workloads.DeviceLayer / helpers.oracle_outputs; odd names the
    projection (if any) whose scales carry 11 significant bits."""
    assert odd in ("",) + PROJ, odd

    def mats(e):
        out = []
        for m, exps in ((0, (GATE_EXP,)), (1, (UP_EXP,)), (2, DOWN_EXPS)):
            c, s = synth.gen_matrix(cfg, layer, e, m)
            # odd scales keep one exponent, so that the down projection's sums stay
            # within fp32's exact range at the full shapes
            out.append((c, _odd_scales(s, exps[-1:]) if odd == PROJ[m] else _pow2_scales(s, exps)))
        return out
    return mats


def _valuation(v: np.ndarray) -> np.ndarray:
    """Exponent of the lowest set bit of each non-zero binary fraction."""
    f, ex = np.frexp(np.abs(v))
    m = (f * 2.0 ** 53).astype(np.int64)
    return ex.astype(np.int64) - 53 + np.log2(m & -m).astype(np.int64)


def _e2m3_group_exact(v: np.ndarray) -> bool:
    """Every 32-group of the rows of v, divided by the power of two that puts its
    largest magnitude in [2, 4), consists of fp6 e2m3 values."""
    g = np.abs(v).reshape(v.shape[0], -1, 32)
    mx = g.max(axis=2, keepdims=True)
    ea = np.floor(np.log2(np.where(mx > 0, mx, 1.0))) - 1
    w = g / np.exp2(ea)
    step = np.where(w < 2.0, 8.0, 4.0)
    return bool(np.all(w * step == np.round(w * step)) and np.all(w < 4.0))


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
        # with |g| >= 128, SiLU(g) is g or a signed zero in any precision, so h is the
        # single bf16 rounding of SiLU(g) * u, which is exact in fp32
        prod = np.where(g > 0, g, 0.0) * u
        assert np.array_equal(prod.astype(np.float32).astype(np.float64), prod), e
        # every partial sum of the down projection, in any order, stays below 2^24 of
        # the unit of the products of its row, 2^(lowest set bit of h) * 2^(lowest set
        # bit of W), also where a kernel splits each weight into an fp16 part and a
        # residual (both multiples of that unit, together at most 1 + 2^-11 of |W|)
        cd, sd = mats(e)[2]
        wd = oracle.dequant(cfg.qtypes[2], cd, sd)
        w_unit = _valuation(wd[wd != 0]).min()
        for t in range(len(hv)):
            ht = hv[t]
            if not np.any(ht):
                continue
            unit_t = 2.0 ** (_valuation(ht[ht != 0]).min() + w_unit)
            assert (np.abs(ht) @ np.abs(wd)).max() * (1 + 2.0 ** -10) < 2.0 ** 24 * unit_t, (e, t)
        # where a 2-bit projection has scales whose 0.75 s is not an fp16 value, the fp6
        # copies of its activations (which carry the correction terms) are exact
        for m, act in ((0, oracle.bf16_to_f64(x[toks])), (1, oracle.bf16_to_f64(x[toks])),
                       (2, hv)):
            sc = oracle.f16_to_f64(mats(e)[m][1]) * 0.75
            if cfg.qtypes[m] == 2 and not np.array_equal(sc.astype(np.float16), sc):
                assert _e2m3_group_exact(act), (e, m)
