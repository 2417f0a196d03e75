"""Pins for the oracle's routing: router logits, top-k + weights, permutation.

Each function is held against something other than itself: numpy's BLAS dot
in double, exact integer cases, Python's stable sort, closed-form softmax
special cases, and the invariants the definitions imply.
"""
import math

import numpy as np
import pytest

import oracle
import synth


def _bf16(vals):
    import torch
    t = torch.tensor(np.asarray(vals, np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


# ------------------------------------------------------------------ logits
def test_logits_vs_numpy_blas():
    rng = np.random.default_rng(0)
    T, d, E = 5, 256, 16
    x = _bf16(rng.standard_normal((T, d)))
    Wr = rng.standard_normal((E, d)).astype(np.float32) * 0.02
    b = rng.standard_normal(E).astype(np.float32)
    ours = oracle.router_logits(x, Wr, b).astype(np.float64)
    ref = oracle.bf16_to_f64(x) @ Wr.astype(np.float64).T + b.astype(np.float64)
    # both are double sums rounded once to fp32: at most one fp32 ulp apart
    assert np.all(np.abs(ours - ref) <= np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64))


def test_logits_exact_integer_case():
    # integer activations and power-of-two weights: every product and sum is exact
    T, d, E = 3, 64, 4
    xv = np.tile(np.arange(-2, 2, dtype=np.float32), (T, d // 4))
    xv[1] *= -1
    x = _bf16(xv)
    Wr = np.zeros((E, d), np.float32)
    Wr[0, :] = 0.25
    Wr[1, ::2] = 1.0
    Wr[2, 5] = -8.0
    Wr[3, :] = 2.0 ** -10
    L = oracle.router_logits(x, Wr, np.float32([0.5, 0, 0, 0]))
    expect = xv.astype(np.float64) @ Wr.astype(np.float64).T + np.array([0.5, 0, 0, 0])
    assert np.array_equal(L.astype(np.float64), expect)


# ------------------------------------------------------------------- top-k
def _brute_topk(L, k):
    T, E = L.shape
    ids = np.empty((T, k), np.int64)
    for t in range(T):
        order = sorted(range(E), key=lambda e: (-float(L[t, e]), e))
        ids[t] = order[:k]
    return ids


def test_topk_vs_python_sort_random_and_ties():
    rng = np.random.default_rng(1)
    T, E, k = 64, 32, 6
    L = rng.standard_normal((T, E)).astype(np.float32)
    L[::3] = np.round(L[::3] * 2) / 2  # many exact ties
    L[5] = 0.0
    L[6, :] = -0.0
    L[6, ::2] = 0.0  # +0 and -0 are equal
    L[7] = np.float32(1e-45) * rng.integers(0, 3, E)  # subnormals
    ids, w = oracle.topk_softmax(L, k)
    assert np.array_equal(ids, _brute_topk(L, k))


def test_topk_all_equal():
    L = np.full((3, 10), 0.7, np.float32)
    ids, w = oracle.topk_softmax(L, 4)
    assert np.array_equal(ids, np.tile(np.arange(4), (3, 1)))
    assert np.array_equal(w, np.full((3, 4), 0.25, np.float32))


def test_topk_k_equals_E_is_full_softmax():
    rng = np.random.default_rng(2)
    L = rng.standard_normal((4, 9)).astype(np.float32)
    ids, w = oracle.topk_softmax(L, 9)
    Ld = L.astype(np.float64)
    full = np.exp(Ld - Ld.max(1, keepdims=True))
    full /= full.sum(1, keepdims=True)
    for t in range(4):
        assert np.allclose(w[t], full[t, ids[t]].astype(np.float32), rtol=0, atol=1e-7)
        assert np.array_equal(np.sort(ids[t]), np.arange(9))


def test_two_experts_is_logistic():
    L = np.float32([[1.25, -0.5], [-3.0, 2.0], [0.0, 0.0]])
    ids, w = oracle.topk_softmax(L, 2)
    for t in range(3):
        a, b = float(L[t, ids[t, 0]]), float(L[t, ids[t, 1]])
        assert w[t, 0] == np.float32(1.0 / (1.0 + math.exp(b - a)))
    assert np.array_equal(ids, [[0, 1], [1, 0], [0, 1]])


def test_weights_sum_to_one_and_descend():
    rng = np.random.default_rng(3)
    L = (rng.standard_normal((200, 256)) * 3).astype(np.float32)
    ids, w = oracle.topk_softmax(L, 8)
    assert np.all(np.abs(w.astype(np.float64).sum(1) - 1.0) <= 1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)
    for t in range(200):
        assert len(set(ids[t])) == 8


def test_topk_rejects_nan_and_bad_k():
    L = np.zeros((1, 4), np.float32)
    L[0, 2] = np.nan
    with pytest.raises(oracle.OracleError):
        oracle.topk_softmax(L, 2)
    with pytest.raises(oracle.OracleError):
        oracle.topk_softmax(np.zeros((1, 4), np.float32), 5)


# ------------------------------------------------------------- permutation
def _check_perm(ids, E, counts, offsets, perm_tok, inv_row):
    T, k = ids.shape
    assert counts.sum() == T * k and offsets[0] == 0 and offsets[E] == T * k
    assert np.array_equal(np.diff(offsets), counts)
    assert np.array_equal(counts, np.bincount(ids.reshape(-1), minlength=E))
    # inv_row is a bijection onto rows, consistent with perm_tok and the expert ranges
    assert np.array_equal(np.sort(inv_row.reshape(-1)), np.arange(T * k))
    for t in range(T):
        for j in range(k):
            r = inv_row[t, j]
            assert perm_tok[r] == t
            e = ids[t, j]
            assert offsets[e] <= r < offsets[e + 1]
    # ascending tokens inside each expert's range
    for e in range(E):
        seg = perm_tok[offsets[e]:offsets[e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_permute_vs_stable_sort():
    rng = np.random.default_rng(4)
    T, E, k = 50, 12, 3
    L = rng.standard_normal((T, E)).astype(np.float32)
    ids, _ = oracle.topk_softmax(L, k)
    counts, offsets, perm_tok, inv_row = oracle.permute(ids, E)
    _check_perm(ids, E, counts, offsets, perm_tok, inv_row)
    flat = ids.reshape(-1)
    order = sorted(range(T * k), key=lambda r: int(flat[r]))  # Python's sort is stable
    assert np.array_equal(perm_tok, np.array(order) // k)


def test_permute_skewed_and_empty_experts():
    # Zipf-skewed routing as in the skewed prefill case: many empty experts, one very hot one
    cfg = synth.CONFIGS["c4"]
    L = synth.gen_logits(synth.small_config(cfg, E=64), T=300)
    ids, _ = oracle.topk_softmax(L, 8)
    counts, offsets, perm_tok, inv_row = oracle.permute(ids, 64)
    _check_perm(ids, 64, counts, offsets, perm_tok, inv_row)
    assert (counts == 0).any() and counts.max() > 150


def test_permute_single_expert():
    ids = np.zeros((7, 1), np.int32)
    counts, offsets, perm_tok, inv_row = oracle.permute(ids, 1)
    assert counts.tolist() == [7] and offsets.tolist() == [0, 7]
    assert perm_tok.tolist() == list(range(7))
    assert inv_row.reshape(-1).tolist() == list(range(7))
