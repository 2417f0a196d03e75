"""CPU check of the premise behind the bit-exact GPU tests: on the exact-input
construction every pre-rounding value the oracle forms is representable in
fp32, every gate output is 0 or at least 128 in magnitude, h is the exact
product, and the down projection's partial sums stay below 2^24 of their unit.
The same construction, shapes and routing as tests/test_gpu_exact.py (the
full-shape cases on a subset of tokens, to keep this fast)."""
import numpy as np
import pytest

import synth
from exact_inputs import PROJ, basis_tokens, check_premise, exact_mats

from test_gpu_exact import (DECODE_PATTERNS, FAMILIES, FULL, NARROW, ODD_KB, SMALL, WIDE_I,
                            _skewed_experts, odd_kb_positions)


@pytest.mark.parametrize("qt", FAMILIES)
def test_premise_small_prefill(qt):
    cfg = synth.small_config(SMALL, q_gate=qt[0], q_up=qt[1], q_down=qt[2])
    x, _ = basis_tokens(cfg.d, cfg.T, seed=7, positions=(np.arange(cfg.T) * 37) % cfg.d)
    check_premise(cfg, exact_mats(cfg), x, _skewed_experts(cfg.E, cfg.T, seed=8))


@pytest.mark.parametrize("qt", [(2, 2, 2), (1, 1, 1)])
def test_premise_narrow_prefill(qt):
    cfg = synth.small_config(NARROW, q_gate=qt[0], q_up=qt[1], q_down=qt[2])
    x, _ = basis_tokens(cfg.d, cfg.T, seed=11, positions=(np.arange(cfg.T) * 41) % cfg.d)
    check_premise(cfg, exact_mats(cfg), x, _skewed_experts(cfg.E, cfg.T, seed=12))


@pytest.mark.parametrize("qt", [(2, 2, 2), (3, 3, 2)])
def test_premise_full_shapes(qt):
    cfg = synth.small_config(FULL, q_gate=qt[0], q_up=qt[1], q_down=qt[2])
    mats = exact_mats(cfg)
    for i, pat in enumerate(DECODE_PATTERNS[:4]):
        x, _ = basis_tokens(cfg.d, len(pat), seed=1000 + i)
        check_premise(cfg, mats, x, np.array(pat))
    x, _ = basis_tokens(cfg.d, cfg.T, seed=9)
    experts = _skewed_experts(cfg.E, cfg.T, seed=10)
    keep = np.arange(0, cfg.T, 16)
    check_premise(cfg, mats, x[keep], experts[keep])


@pytest.mark.parametrize("odd", PROJ)
def test_premise_odd_scales(odd):
    small = synth.small_config(SMALL, q_gate=2, q_up=2, q_down=2)
    x, _ = basis_tokens(small.d, small.T, seed=7, positions=(np.arange(small.T) * 37) % small.d)
    check_premise(small, exact_mats(small, odd=odd), x, _skewed_experts(small.E, small.T, seed=8))
    full = synth.small_config(FULL, q_gate=2, q_up=2, q_down=2)
    mats = exact_mats(full, odd=odd)
    for i in (0, 3, 8):
        x, _ = basis_tokens(full.d, len(DECODE_PATTERNS[i]), seed=2000 + i)
        check_premise(full, mats, x, np.array(DECODE_PATTERNS[i]))
    x, _ = basis_tokens(full.d, full.T, seed=9)
    experts = _skewed_experts(full.E, full.T, seed=10)
    keep = np.arange(0, full.T, 16)
    check_premise(full, mats, x[keep], experts[keep])


@pytest.mark.parametrize("cfg0", ODD_KB, ids=lambda c: c.name)
@pytest.mark.parametrize("qt", [(2, 2, 2), (3, 3, 2), (1, 1, 1)])
def test_premise_single_token_odd_kblocks(cfg0, qt):
    cfg = synth.small_config(cfg0, q_gate=qt[0], q_up=qt[1], q_down=qt[2])
    mats = exact_mats(cfg)
    for i, pos in enumerate(odd_kb_positions(cfg.d)):
        x, _ = basis_tokens(cfg.d, 1, seed=3000 + i, positions=[pos])
        check_premise(cfg, mats, x, np.array([(3 * i + 1) % cfg.E]))


@pytest.mark.parametrize("qt", [(2, 2, 2), (3, 3, 2), (1, 1, 1)])
def test_premise_separate_down(qt):
    cfg = synth.small_config(WIDE_I, q_gate=qt[0], q_up=qt[1], q_down=qt[2])
    mats = exact_mats(cfg)
    for i in (0, 1, 3, 8, 9):
        x, _ = basis_tokens(cfg.d, len(DECODE_PATTERNS[i]), seed=4000 + i)
        check_premise(cfg, mats, x, np.array(DECODE_PATTERNS[i]))
