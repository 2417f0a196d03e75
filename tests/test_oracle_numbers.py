"""Pins for the oracle's own number conversions (bf16, fp16).

The oracle converts with its own C routines; these tests hold them against
independent implementations (torch's bfloat16, numpy's float16) and against
hand-derived tie cases that a double->float->bf16 path would get wrong.
"""
import numpy as np
import pytest
import torch

import oracle


def _all_non_nan_bf16():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    f = (b.astype(np.uint32) << 16).view(np.float32)
    return b[~np.isnan(f)]


def test_bf16_to_f64_exhaustive_vs_torch():
    b = _all_non_nan_bf16()
    ours = oracle.bf16_to_f64(b)
    ref = torch.from_numpy(b.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)
    # the C routine itself, on a sample
    lib = oracle._load()
    for v in b[::257]:
        assert lib.oracle_bf16_to_f64(int(v)) == ours[np.searchsorted(b, v)]


def test_f16_to_f64_exhaustive_vs_numpy():
    b = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = b.view(np.float16).astype(np.float64)
    ours = oracle.f16_to_f64(b)
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.all(np.isnan(ours[~ok]))


def test_f64_to_bf16_matches_torch_on_float_values():
    # Values exactly representable in fp32: torch's fp32 -> bf16 (round to nearest even) is the
    # reference.  Cover normals, subnormals, near-overflow and exact ties.
    rng = np.random.default_rng(123)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ties = ((rng.integers(0, 2 ** 16, 5000, dtype=np.uint64).astype(np.uint32) << 16)
            | np.uint32(0x8000)).view(np.float32)
    ties = ties[np.isfinite(ties)]
    vals = np.concatenate([f, ties, np.float32([3.3895314e38, -3.3895314e38, 1e-40, -1e-45])])
    ref = torch.from_numpy(vals).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    ours = oracle.f64_to_bf16(vals.astype(np.float64))
    assert np.array_equal(ours, ref)


@pytest.mark.parametrize(
    "value,expected",
    [
        (1.0 + 2.0 ** -8, 0x3F80),               # exact tie -> even (1.0)
        (1.0 + 3 * 2.0 ** -8, 0x3F82),           # exact tie -> even (1 + 2^-6)
        (1.0 + 2.0 ** -8 + 2.0 ** -40, 0x3F81),  # just above the tie: up (an fp32 detour gives 0x3F80)
        (1.0 + 2.0 ** -8 - 2.0 ** -40, 0x3F80),  # just below the tie
        (-(1.0 + 2.0 ** -8 + 2.0 ** -40), 0xBF81),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (2.0 ** -133, 0x0001),                   # smallest bf16 subnormal
        (2.0 ** -134, 0x0000),                   # half of it: tie -> even (zero)
        (3 * 2.0 ** -134, 0x0002),               # 1.5 ulp: tie -> even (2 ulp)
        (2.0 ** 128, 0x7F80),                    # overflow
        (float("inf"), 0x7F80),
        (float("-inf"), 0xFF80),
        (1.6e15, 0x58B6),                        # magnitudes of a deep residual stack stay finite
    ],
)
def test_f64_to_bf16_hand_cases(value, expected):
    assert int(oracle.f64_to_bf16(np.float64(value))) == expected


def test_f64_to_bf16_nan():
    out = int(oracle.f64_to_bf16(np.float64("nan")))
    assert (out & 0x7F80) == 0x7F80 and (out & 0x7F) != 0
