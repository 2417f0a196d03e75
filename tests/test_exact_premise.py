"""CPU check of the premise behind the bit-exact GPU tests: on the exact-input
construction every pre-rounding value the oracle forms is representable in
fp32, every gate output is 0 or at least 128 in magnitude, h is the exact
product, and the down projection's partial sums stay below 2^24 of their unit.
The same construction, shapes and routing as tests/test_gpu_exact.py (the
full-shape cases on a subset of tokens, to keep this fast)."""
import numpy as np
import pytest

import synth
from exact_inputs import basis_tokens, check_premise, exact_mats

from test_gpu_exact import DECODE_PATTERNS, FAMILIES, FULL, SMALL, _skewed_experts


@pytest.mark.parametrize("qt", FAMILIES)
def test_premise_small_prefill(qt):
    cfg = synth.small_config(SMALL, q_gate=qt[0], q_up=qt[1], q_down=qt[2])
    x, _ = basis_tokens(cfg.d, cfg.T, seed=7, positions=(np.arange(cfg.T) * 37) % cfg.d)
    check_premise(cfg, exact_mats(cfg), x, _skewed_experts(cfg.E, cfg.T, seed=8))


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
