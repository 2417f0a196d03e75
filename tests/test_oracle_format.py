"""Pins for the oracle's decoder of packed format v2.

The expected byte/bit positions below were worked out by hand from the format
definition (see the golden file's notes), not produced by any code here.
"""
import json
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden", "format_v2_positions.json")


@pytest.mark.parametrize(
    "q,K,N,nbytes",
    [
        (2, 4096, 2048, 2_621_440),   # 2.5 bits per weight incl. scales
        (1, 4096, 2048, 2_621_440),
        (3, 4096, 2048, 3_670_016),   # 3.5 bits per weight incl. scales
        (2, 2048, 4096, 2_621_440),
        (2, 256, 128, 10_240),
        (2, 128, 256, 10_240),
        (3, 128, 16, 1_024),          # 512 + 256 + 128, each region 256-aligned -> 1024
        (2, 100, 16, 0),              # K not a multiple of 128
        (2, 128, 8, 0),               # N not a multiple of 16
        (4, 128, 16, 0),              # unknown qtype
    ],
)
def test_packed_bytes(q, K, N, nbytes):
    assert oracle.packed_bytes(q, K, N) == nbytes


def _blob_with(q, K, N, sets):
    """Blob of zeros, with the listed (byte, bit, value_bits, width) fields written in."""
    blob = np.zeros(oracle.packed_bytes(q, K, N), np.uint8)
    for byte, bit, val, width in sets:
        for b in range(width):
            if (val >> b) & 1:
                pos = bit + b
                blob[byte + pos // 8] |= np.uint8(1 << (pos % 8))
    return blob


def test_single_code_positions_from_golden():
    gold = json.load(open(GOLD))
    for case in gold["int2_cases"]:
        K, N = case["K"], case["N"]
        n, k, u = case["n"], case["k"], case["u"]
        blob = _blob_with(2, K, N, [(case["byte"], case["bit"], u, 2)])
        codes, scales = oracle.unpack(2, K, N, blob)
        expect = np.zeros((N, K), np.uint8)
        expect[n, k] = u
        assert np.array_equal(codes, expect), case
        assert not scales.any()
    for case in gold["int3_hi_cases"]:
        K, N = case["K"], case["N"]
        n, k = case["n"], case["k"]
        blob = _blob_with(3, K, N, [(case["byte"], case["bit"], 1, 1)])
        codes, _ = oracle.unpack(3, K, N, blob)
        expect = np.zeros((N, K), np.uint8)
        expect[n, k] = 4
        assert np.array_equal(codes, expect), case
    for case in gold["scale_cases"]:
        K, N = case["K"], case["N"]
        blob = _blob_with(case["q"], K, N, [(case["byte"], 0, 0x3C00, 16)])
        _, scales = oracle.unpack(case["q"], K, N, blob)
        expect = np.zeros((N, K // 32), np.uint16)
        expect[case["n"], case["g"]] = 0x3C00
        assert np.array_equal(scales, expect), case


def test_ternary_rejects_level_3():
    blob = _blob_with(1, 128, 16, [(0, 0, 3, 2)])
    with pytest.raises(oracle.OracleError):
        oracle.unpack(1, 128, 16, blob)
    blob = _blob_with(1, 128, 16, [(0, 0, 2, 2)])
    codes, _ = oracle.unpack(1, 128, 16, blob)
    assert codes[0, 0] == 2


def test_unpack_rejects_short_blob():
    blob = np.zeros(oracle.packed_bytes(2, 128, 16) - 1, np.uint8)
    with pytest.raises(oracle.OracleError):
        oracle.unpack(2, 128, 16, blob)


def test_every_bit_of_plane0_is_one_code():
    # Each of the plane's bits belongs to exactly one code: setting all plane-0 bits to one gives
    # every int2 code level 3 and touches no scale.
    K, N = 256, 32
    nb = oracle.packed_bytes(2, K, N)
    blob = np.zeros(nb, np.uint8)
    blob[: (N // 16) * (K // 128) * 512] = 0xFF
    codes, scales = oracle.unpack(2, K, N, blob)
    assert (codes == 3).all() and not scales.any()


def test_every_bit_of_plane1_is_one_code():
    # The same for the 3-bit plane: with plane 0 all zeros and plane 1 all ones every code is 4,
    # so each plane-1 bit maps to exactly one (n, k) and all are used.
    K, N = 256, 32
    nb = oracle.packed_bytes(3, K, N)
    tiles = (N // 16) * (K // 128)
    blob = np.zeros(nb, np.uint8)
    blob[tiles * 512: tiles * 512 + tiles * 256] = 0xFF
    codes, scales = oracle.unpack(3, K, N, blob)
    assert (codes == 4).all() and not scales.any()
