"""Pins for the oracle's weights, expert FFN, combine and whole layer.

* dequantisation against closed forms (every level, power-of-two, negative,
  subnormal and zero scales) and against numpy's own float16 decode;
* the expert FFN against a dense numpy formulation (weights rebuilt with
  numpy, products by BLAS) before rounding, and after rounding against
  torch's bf16;
* the whole layer against a dense formulation that runs every expert and
  routes with an explicit one-hot weight matrix;
* textbook special cases: one expert (a plain SwiGLU FFN), zero weights,
  exactly representable inputs, and the hand-worked example in
  tests/golden/worked_example.json.
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth

OFF = {1: 1.0, 2: 1.5, 3: 3.5}
LEVELS = {1: 3, 2: 4, 3: 8}
GOLD = os.path.join(os.path.dirname(__file__), "golden", "worked_example.json")


def _bf16(vals):
    t = torch.tensor(np.asarray(vals, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _bf16_of_f64_via_torch(v):
    """Nearest bf16 via fp32; valid only where the fp32 rounding cannot create a tie."""
    return torch.tensor(np.asarray(v, np.float64)).to(torch.float32).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def _dense_np(q, codes, scales):
    """Dense W[K][N] with numpy: fp16 scales decoded by numpy, one scale per 32 k."""
    s = scales.view(np.float16).astype(np.float64)           # [N][K/32]
    s_full = np.repeat(s, 32, axis=1)                        # [N][K]
    return (s_full * (codes.astype(np.float64) - OFF[q])).T  # [K][N]


# ------------------------------------------------------------------ dequant
@pytest.mark.parametrize("q", [1, 2, 3])
def test_dequant_every_level_closed_form(q):
    N, K = 16, 64
    codes = (np.arange(N * K) % LEVELS[q]).astype(np.uint8).reshape(N, K)
    scales = np.full((N, K // 32), 0x3C00, np.uint16)  # 1.0
    scales[:, 1] = 0x3000                               # 0.125
    scales[3, :] = 0xB800                               # -0.5
    scales[4, :] = 0x0001                               # smallest subnormal 2^-24
    scales[5, :] = 0x0000
    W = oracle.dequant(q, codes, scales)
    for n in range(N):
        for k in range(K):
            s = {0x3C00: 1.0, 0x3000: 0.125, 0xB800: -0.5, 0x0001: 2.0 ** -24, 0: 0.0}[
                int(scales[n, k // 32])]
            assert W[k, n] == s * (int(codes[n, k]) - OFF[q])


@pytest.mark.parametrize("q", [1, 2, 3])
def test_dequant_vs_numpy_float16(q):
    N, K = 32, 128
    c = synth.codes(9, 1, N * K, LEVELS[q]).reshape(N, K)
    s = synth.absnormal_f16(9, 2, N * K // 32, 0.05).reshape(N, K // 32)
    assert np.array_equal(oracle.dequant(q, c, s), _dense_np(q, c, s))


def test_dequant_rejects_out_of_range():
    c = np.zeros((16, 32), np.uint8)
    c[3, 4] = 3
    s = np.zeros((16, 1), np.uint16)
    with pytest.raises(oracle.OracleError):
        oracle.dequant(1, c, s)
    c[3, 4] = 8
    with pytest.raises(oracle.OracleError):
        oracle.dequant(3, c, s)


# ------------------------------------------------------------------- expert
def _mats(seed, d, I, qs):
    out = []
    for m, q in enumerate(qs):
        K, N = (d, I) if m < 2 else (I, d)
        c = synth.codes(seed, 10 + m, N * K, LEVELS[q]).reshape(N, K)
        s = synth.absnormal_f16(seed, 20 + m, N * K // 32, 0.05).reshape(N, K // 32)
        out.append((c, s))
    return out


def _silu_np(g):
    return g / (1.0 + np.exp(-g))


@pytest.mark.parametrize("qs", [(2, 2, 2), (3, 3, 2), (1, 1, 1)])
def test_expert_vs_dense_numpy(qs):
    d, I, M = 256, 128, 6
    mats = _mats(5, d, I, qs)
    x = synth.normal_bf16(5, 99, M * d).reshape(M, d)
    h, y, g_pre, u_pre, y_pre = oracle.expert_rows(qs, mats, x, want_pre=True)
    Wg, Wu, Wd = (_dense_np(q, c, s) for q, (c, s) in zip(qs, mats))
    xd = oracle.bf16_to_f64(x)
    g_ref, u_ref = xd @ Wg, xd @ Wu
    assert np.allclose(g_pre, g_ref, rtol=1e-12, atol=1e-12 * np.abs(g_ref).max())
    assert np.allclose(u_pre, u_ref, rtol=1e-12, atol=1e-12 * np.abs(u_ref).max())
    # h: the rounding point after SiLU(g)*u; fp32-exact cases aside, torch agrees bit for bit
    hv = _silu_np(g_pre) * u_pre
    assert np.mean(h == _bf16_of_f64_via_torch(hv)) > 0.999
    y_ref = oracle.bf16_to_f64(h) @ Wd
    assert np.allclose(y_pre, y_ref, rtol=1e-12, atol=1e-12 * np.abs(y_ref).max())
    assert np.mean(y == _bf16_of_f64_via_torch(y_pre)) > 0.999


def test_expert_zero_weights_give_exact_zero():
    d, I = 128, 32
    mats = []
    for m in range(3):
        K, N = (d, I) if m < 2 else (I, d)
        mats.append((np.ones((N, K), np.uint8), synth.absnormal_f16(1, m, N * K // 32, 0.05)
                     .reshape(N, K // 32)))
    x = synth.normal_bf16(1, 7, 3 * d).reshape(3, d)
    h, y = oracle.expert_rows((1, 1, 1), mats, x)
    assert not h.any() or np.all((h & 0x7FFF) == 0)
    assert np.all((y & 0x7FFF) == 0)


def test_expert_exact_inputs_bit_exact():
    # power-of-two scales and small integer activations: every value is exactly representable
    d, I = 128, 32
    rng = np.random.default_rng(6)
    mats = []
    for m in range(3):
        K, N = (d, I) if m < 2 else (I, d)
        c = rng.integers(0, 4, (N, K)).astype(np.uint8)
        s = rng.choice(np.uint16([0x3C00, 0x3800, 0x3400, 0x4000]), (N, K // 32))
        mats.append((c, s))
    xv = rng.integers(-2, 3, (2, d)).astype(np.float32)
    h, y, g_pre, u_pre, y_pre = oracle.expert_rows((2, 2, 2), mats, _bf16(xv), want_pre=True)
    Wg, Wu, Wd = (_dense_np(2, c, s) for c, s in mats)
    assert np.array_equal(g_pre, xv.astype(np.float64) @ Wg)
    assert np.array_equal(u_pre, xv.astype(np.float64) @ Wu)


def test_worked_example():
    ex = json.load(open(GOLD))
    d, I = ex["d"], ex["I"]
    mats = []
    for name in ("gate", "up", "down"):
        K, N = (d, I) if name != "down" else (I, d)
        c = np.ones((N, K), np.uint8)  # ternary level 1 = weight 0
        for n, k, u in ex[name]["codes"]:
            c[n, k] = u
        s = np.full((N, K // 32), ex[name]["scale_bits"], np.uint16)
        mats.append((c, s))
    x = np.zeros((1, d), np.float32)
    for i, v in ex["x"]:
        x[0, i] = v
    h, y = oracle.expert_rows((1, 1, 1), mats, _bf16(x))
    hv = oracle.bf16_to_f64(h)[0]
    yv = oracle.bf16_to_f64(y)[0]
    for n, v in ex["expect_h"]:
        assert hv[n] == v, (n, hv[n], v)
    assert np.count_nonzero(hv) == len(ex["expect_h"])
    for n, v in ex["expect_y"]:
        assert yv[n] == v, (n, yv[n], v)
    assert np.count_nonzero(yv) == len(ex["expect_y"])


# ------------------------------------------------------------------ combine
def test_combine_hand_values():
    # one token, k=2, d=2: out = x + 0.75*y0 + 0.25*y1 + ysh
    w = np.float32([[0.75, 0.25]])
    inv = np.int32([[1, 0]])
    y = _bf16([[2.0, -4.0], [8.0, 1.0]])  # row 0 is slot 1's output, row 1 slot 0's
    ysh = _bf16([[0.5, 0.5]])
    x = _bf16([[1.0, 1.0]])
    out = oracle.combine(w, inv, y, ysh, x, residual=True)
    assert oracle.bf16_to_f64(out).tolist() == [[1 + 6 + 0.5 + 0.5, 1 + 0.75 - 1 + 0.5]]
    out = oracle.combine(w, inv, y, None, x, residual=False)
    assert oracle.bf16_to_f64(out).tolist() == [[6.5, -0.25]]


# --------------------------------------------------------------- whole layer
def _layer_inputs(cfg, T):
    experts = []
    for e in range(cfg.E + cfg.n_shared):
        experts.append([synth.gen_matrix(cfg, 0, e, m) for m in range(3)])
    return experts


def _dense_layer(cfg, x, experts, logits, residual):
    """Every expert on every token; one-hot routing weights pick the selected ones."""
    T = x.shape[0]
    E, k = cfg.E, cfg.k
    ids_ref = np.array([sorted(range(E), key=lambda e: (-float(logits[t, e]), e))[:k]
                        for t in range(T)])
    R = np.zeros((T, E))
    for t in range(T):
        sel = logits[t, ids_ref[t]].astype(np.float64)
        p = np.exp(sel - sel[0])
        p = (p / p.sum()).astype(np.float32)
        R[t, ids_ref[t]] = p
    xd = oracle.bf16_to_f64(x)
    acc = xd.copy() if residual else np.zeros_like(xd)
    for e in range(E + cfg.n_shared):
        Wg, Wu, Wd = (_dense_np(q, c, s) for q, (c, s) in zip(cfg.qtypes, experts[e]))
        h = _silu_np(xd @ Wg) * (xd @ Wu)
        hb = oracle.bf16_to_f64(oracle.f64_to_bf16(h))
        yb = oracle.bf16_to_f64(oracle.f64_to_bf16(hb @ Wd))
        wcol = R[:, e:e + 1] if e < E else np.ones((T, 1))
        acc = acc + wcol * yb
    return ids_ref, R, acc


@pytest.mark.parametrize("residual", [False, True])
def test_layer_vs_dense_one_hot_formulation(residual):
    cfg = synth.CONFIGS["c0"]
    cfg = synth.small_config(cfg, n_shared=1)
    experts = _layer_inputs(cfg, cfg.T)
    x = synth.gen_x(cfg)
    Wr = synth.gen_router(cfg)
    r = oracle.moe_layer((cfg.E, cfg.k, cfg.inter, cfg.n_shared, cfg.qtypes), x, experts, Wr=Wr,
                         residual=residual)
    ids_ref, R, acc = _dense_layer(cfg, x, experts, r["logits"], residual)
    assert np.array_equal(r["ids"], ids_ref)
    out = oracle.bf16_to_f64(r["out"])
    ref = oracle.bf16_to_f64(oracle.f64_to_bf16(acc))
    # same rounding points; sums in a different order may move a value across a bf16 boundary
    # only when it sits within ~1e-15 of it
    assert np.mean(out == ref) > 0.995
    assert np.allclose(out, acc, rtol=2 ** -8, atol=0)
    assert np.all(np.abs(r["w"].astype(np.float64).sum(1) - 1) <= 1e-6)
    assert r["counts"].sum() == cfg.T * cfg.k


def test_single_expert_is_dense_swiglu():
    cfg = synth.small_config(synth.CONFIGS["c0"], E=1, k=1)
    experts = _layer_inputs(cfg, cfg.T)
    x = synth.gen_x(cfg)
    r = oracle.moe_layer((1, 1, cfg.inter, 0, cfg.qtypes), x, experts,
                         logits=np.zeros((cfg.T, 1), np.float32))
    assert np.all(r["w"] == 1.0) and np.all(r["ids"] == 0)
    h, y = oracle.expert_rows(cfg.qtypes, experts[0], x)
    assert np.array_equal(r["out"], y)  # w = 1 and no other term: out is the FFN output itself
