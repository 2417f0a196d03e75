"""Host-side tests of the C ABI (no GPU needed).

* the library loads and exports every function include/moe.h declares, and
  the benchmark's ceilings library every function include/ceilings.h does;
* the host packer agrees with the oracle's independent decoder of the format
  (both written from the format definition) on every level and on special
  scales;
* every argument error is reported with its status code before any launch.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import bit_quantized_moe_router_amd as bq
import oracle
import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe.h")


def test_library_exports_every_declared_symbol():
    lib = bq.load()
    text = open(HEADER).read()
    declared = set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text))
    assert declared == set(bq.EXPORTED)
    for name in declared:
        assert hasattr(lib, name), name
    assert bq.moe_abi_version() == 3


def test_ceilings_library_exports_every_declared_symbol():
    from bit_quantized_moe_router_amd import build as B

    if not os.path.exists(B.CEIL_LIB):
        pytest.skip("libbqceil.so not built")
    lib = ctypes.CDLL(B.CEIL_LIB)
    text = open(os.path.join(ROOT, "include", "ceilings.h")).read()
    declared = set(re.findall(r"\b(bqc_[a-z0-9_]+)\s*\(", text))
    assert declared == {"bqc_read_stream", "bqc_mfma_bf16", "bqc_mfma_bf16_flops"}
    for name in declared:
        assert hasattr(lib, name), name
    # argument errors come back before any launch (no GPU needed)
    lib.bqc_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.bqc_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.bqc_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.bqc_mfma_bf16_flops.restype = ctypes.c_double
    assert lib.bqc_read_stream(None, 1024, 8, 4, 16, None) == 1
    assert lib.bqc_read_stream(16, 1000, 8, 4, 16, None) == 1   # not a multiple of 16
    assert lib.bqc_read_stream(16, 1024, 8, 3, 16, None) == 1   # unsupported unroll
    assert lib.bqc_mfma_bf16(0, 10, 16, None) == 1
    assert lib.bqc_mfma_bf16_flops(2, 3) == 2 * 4 * 3 * 4 * 32 * 32 * 16 * 2


def test_status_strings():
    for s in range(6):
        assert bq.status_string(s) and bq.status_string(s) != "unknown status"


@pytest.mark.parametrize("q,K,N", [(1, 128, 16), (2, 256, 128), (3, 128, 256), (2, 4096, 2048),
                                   (3, 2048, 4096), (2, 100, 16), (2, 128, 8), (0, 128, 16)])
def test_packed_bytes_matches_oracle(q, K, N):
    assert bq.moe_packed_bytes(q, K, N) == oracle.packed_bytes(q, K, N)


def test_expert_bytes():
    assert bq.moe_expert_bytes(2, 2, 2, 4096, 2048) == 7_864_320
    assert bq.moe_expert_bytes(3, 3, 2, 4096, 2048) == 9_961_472
    assert bq.moe_expert_bytes(1, 1, 1, 4096, 2048) == 7_864_320
    assert bq.moe_expert_bytes(2, 2, 2, 256, 128) == 30_720
    assert bq.moe_expert_bytes(2, 2, 2, 100, 128) == 0


@pytest.mark.parametrize("q", [1, 2, 3])
@pytest.mark.parametrize("K,N", [(128, 16), (256, 48), (384, 32)])
def test_pack_then_oracle_unpack_is_identity(q, K, N):
    levels = synth.LEVELS[q]
    codes = synth.codes(11, q, N * K, levels).reshape(N, K)
    codes[0, :] = np.arange(K) % levels  # every level at every position class
    scales = synth.absnormal_f16(11, 100 + q, N * K // 32, 0.05).reshape(N, K // 32)
    special = np.uint16([0x0000, 0x8000, 0x0001, 0x03FF, 0x0400, 0x7BFF, 0xFBFF, 0x3C00, 0xBC00])
    scales.reshape(-1)[:special.size] = special
    blob = bq.moe_pack_weights(q, codes, scales)
    assert blob.nbytes == oracle.packed_bytes(q, K, N)
    c2, s2 = oracle.unpack(q, K, N, blob)
    assert np.array_equal(c2, codes)
    assert np.array_equal(s2, scales)


def test_pack_exhaustive_single_positions():
    # each (level, k-slot) of one 16 x 128 tile placed alone decodes to itself
    K, N = 128, 16
    for q in (2, 3):
        for k in range(K):
            for u in range(1, synth.LEVELS[q]):
                codes = np.zeros((N, K), np.uint8)
                codes[(k * 7) % N, k] = u
                blob = bq.moe_pack_weights(q, codes, np.zeros((N, 4), np.uint16))
                c2, _ = oracle.unpack(q, K, N, blob)
                assert np.array_equal(c2, codes), (q, k, u)


def test_pack_rejects_bad_input():
    lib = bq.load()
    codes = np.zeros((16, 128), np.uint8)
    scales = np.zeros((16, 4), np.uint16)
    out = np.zeros(bq.moe_packed_bytes(1, 128, 16), np.uint8)
    codes[3, 5] = 3  # not a ternary level
    with pytest.raises(bq.MoeError) as ei:
        bq.moe_pack_weights(1, codes, scales, out)
    assert ei.value.status == bq.MOE_ERR_BAD_CODES
    codes[3, 5] = 8
    with pytest.raises(bq.MoeError) as ei:
        bq.moe_pack_weights(3, codes, scales)
    assert ei.value.status == bq.MOE_ERR_BAD_CODES
    codes[3, 5] = 0
    st = lib.moe_pack_weights(2, 128, 16, codes.ctypes.data, scales.ctypes.data,
                              out.ctypes.data, out.nbytes - 1)
    assert st == bq.MOE_ERR_INVALID_ARG
    st = lib.moe_pack_weights(2, 100, 16, codes.ctypes.data, scales.ctypes.data,
                              out.ctypes.data, out.nbytes)
    assert st == bq.MOE_ERR_UNSUPPORTED
    st = lib.moe_pack_weights(2, 128, 16, None, scales.ctypes.data, out.ctypes.data, out.nbytes)
    assert st == bq.MOE_ERR_INVALID_ARG


# ---------------------------------------------------------------- validation
FAKE = 1 << 40  # a 256-aligned address that is never dereferenced: every call below fails first


def _layer(**kw):
    p = dict(d=256, inter=128, n_experts=8, top_k=2, n_shared=0, qtypes=(2, 2, 2),
             experts=FAKE, expert_stride=30_720, shared=None, router_w=FAKE, router_bias=None)
    p.update(kw)
    return bq.make_layer(p["d"], p["inter"], p["n_experts"], p["top_k"], p["n_shared"],
                         p["qtypes"], p["experts"], p["expert_stride"], p["shared"],
                         p["router_w"], p["router_bias"], p.get("alt"))


def _routing():
    return bq.moe_routing(*([FAKE] * 7))


def _call(fn, L, T, flags=0, R=None, ws=FAKE, ws_bytes=None, x=FAKE, out=FAKE + (1 << 30)):
    lib = bq.load()
    R = _routing() if R is None else R
    if ws_bytes is None:
        ws_bytes = max(1, lib.moe_workspace_bytes(ctypes.byref(L.c), T))
    f = getattr(lib, fn)
    args = [ctypes.byref(L.c), x, T, flags, ctypes.byref(R), ws, ws_bytes]
    if fn != "moe_route_topk":
        args.append(out)
    args.append(None)
    return f(*args)


@pytest.mark.parametrize("fn", ["moe_forward_decode", "moe_forward_prefill", "moe_route_topk"])
def test_argument_errors_return_status(fn):
    L = _layer()
    assert _call(fn, L, -1) == bq.MOE_ERR_INVALID_ARG
    assert _call(fn, L, 2, flags=0x80) == bq.MOE_ERR_INVALID_ARG
    assert _call(fn, _layer(d=100), 2) == bq.MOE_ERR_UNSUPPORTED
    assert _call(fn, _layer(inter=200), 2) == bq.MOE_ERR_UNSUPPORTED
    assert _call(fn, _layer(qtypes=(2, 5, 2)), 2) == bq.MOE_ERR_UNSUPPORTED
    assert _call(fn, _layer(n_experts=2000, top_k=2), 2) == bq.MOE_ERR_UNSUPPORTED
    assert _call(fn, _layer(top_k=9), 2) == bq.MOE_ERR_INVALID_ARG
    assert _call(fn, _layer(n_shared=2), 2) == bq.MOE_ERR_INVALID_ARG
    assert _call(fn, _layer(router_w=None), 2) == bq.MOE_ERR_INVALID_ARG
    R = _routing()
    R.perm_tok = None
    assert _call(fn, L, 2, R=R) == bq.MOE_ERR_INVALID_ARG
    assert _call(fn, L, 2, ws_bytes=10) == bq.MOE_ERR_WORKSPACE
    assert _call(fn, L, 2, ws=None) == bq.MOE_ERR_WORKSPACE
    assert _call(fn, L, 2, ws=FAKE + 8) == bq.MOE_ERR_INVALID_ARG
    if fn != "moe_route_topk":
        assert _call(fn, _layer(expert_stride=30_720 - 256), 2) == bq.MOE_ERR_INVALID_ARG
        assert _call(fn, _layer(expert_stride=30_720 + 8), 2) == bq.MOE_ERR_INVALID_ARG
        assert _call(fn, _layer(experts=FAKE + 16), 2) == bq.MOE_ERR_INVALID_ARG
        assert _call(fn, _layer(n_shared=1, shared=None), 2) == bq.MOE_ERR_INVALID_ARG
        assert _call(fn, L, 2, out=FAKE + 256) == bq.MOE_ERR_INVALID_ARG  # overlaps x
        assert _call(fn, L, 2, out=None) == bq.MOE_ERR_INVALID_ARG
        assert _call(fn, L, 2, x=FAKE + 2) == bq.MOE_ERR_INVALID_ARG


ALT = (FAKE + (1 << 34), 30_720, (1, 1, 1), FAKE + (1 << 35))  # a valid second copy


@pytest.mark.parametrize("fn", ["moe_forward_decode", "moe_forward_prefill"])
def test_second_expert_copy_checks(fn):
    ae, st, q, sel = ALT
    assert _call(fn, _layer(alt=(ae, st, (1, 4, 1), sel)), 2) == bq.MOE_ERR_UNSUPPORTED
    assert _call(fn, _layer(alt=(ae, st, q, None)), 2) == bq.MOE_ERR_INVALID_ARG
    assert _call(fn, _layer(alt=(ae, 512, q, sel)), 2) == bq.MOE_ERR_INVALID_ARG
    assert _call(fn, _layer(alt=(ae, st + 8, q, sel)), 2) == bq.MOE_ERR_INVALID_ARG
    assert _call(fn, _layer(alt=(ae + 64, st, q, sel)), 2) == bq.MOE_ERR_INVALID_ARG
    # valid second copy: prefill refuses it, decode goes on to its other checks
    want = bq.MOE_ERR_UNSUPPORTED if fn == "moe_forward_prefill" else bq.MOE_ERR_INVALID_ARG
    assert _call(fn, _layer(alt=ALT), 2, out=None) == want
    # the router alone never reads expert weights
    assert _call("moe_route_topk", _layer(alt=(ae, st, q, None)), 2, ws_bytes=10) == \
        bq.MOE_ERR_WORKSPACE


def test_decode_token_range():
    L = _layer()
    assert _call("moe_forward_decode", L, 0) == bq.MOE_ERR_INVALID_ARG
    assert _call("moe_forward_decode", L, 9) == bq.MOE_ERR_INVALID_ARG
    # 8 tokens x top-9 = 72 routed rows exceeds the decode kernels' 64
    L9 = _layer(n_experts=16, top_k=9)
    assert _call("moe_forward_decode", L9, 8) == bq.MOE_ERR_UNSUPPORTED


def test_noalloc_decode_argument_checks():
    # the token range and a missing layer or routing are refused before the device is
    # looked up; on a host without a GPU the device lookup itself reports MOE_ERR_DEVICE
    lib = bq.load()
    L, R = _layer(), _routing()
    f = lib.moe_forward_decode_noalloc
    for T in (0, 9, -1):
        assert f(ctypes.byref(L.c), FAKE, T, 0, ctypes.byref(R), FAKE + (1 << 30), None) == \
            bq.MOE_ERR_INVALID_ARG
    assert f(None, FAKE, 2, 0, ctypes.byref(R), FAKE + (1 << 30), None) == bq.MOE_ERR_INVALID_ARG
    assert f(ctypes.byref(L.c), FAKE, 2, 0, None, FAKE + (1 << 30), None) == bq.MOE_ERR_INVALID_ARG
    import torch
    if not torch.cuda.is_available():
        assert f(ctypes.byref(L.c), FAKE, 2, 0, ctypes.byref(R), FAKE + (1 << 30), None) == \
            bq.MOE_ERR_DEVICE


def test_zero_tokens_is_a_noop():
    L = _layer()
    assert _call("moe_forward_prefill", L, 0) == bq.MOE_OK
    assert _call("moe_route_topk", L, 0) == bq.MOE_OK


def test_workspace_bytes():
    lib = bq.load()
    L = _layer()
    sizes = [lib.moe_workspace_bytes(ctypes.byref(L.c), T) for T in (1, 4, 8, 9, 100, 1000)]
    assert all(s > 0 for s in sizes) and sizes == sorted(sizes)
    assert lib.moe_workspace_bytes(ctypes.byref(_layer(d=100).c), 4) == 0
    assert lib.moe_workspace_bytes(ctypes.byref(L.c), -1) == 0


def test_stage_masks_are_checked():
    lib = bq.load()
    L = _layer()
    R = _routing()
    ws_bytes = lib.moe_workspace_bytes(ctypes.byref(L.c), 2)
    for fn, allm in (("moe_forward_decode_stages", 15), ("moe_forward_prefill_stages", 31)):
        f = getattr(lib, fn)
        for bad in (0, allm + 1, 1 << 8):
            assert f(ctypes.byref(L.c), FAKE, 2, 0, ctypes.byref(R), FAKE, ws_bytes,
                     FAKE + (1 << 30), bad, None) == bq.MOE_ERR_INVALID_ARG
        # a valid mask goes on to the ordinary argument checks
        assert f(ctypes.byref(L.c), FAKE, 2, 0x80, ctypes.byref(R), FAKE, ws_bytes,
                 FAKE + (1 << 30), 1, None) == bq.MOE_ERR_INVALID_ARG
