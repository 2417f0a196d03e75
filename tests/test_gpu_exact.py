"""Bit-exact GPU layer tests on inputs where every step is exact in fp32.

On these inputs (see exact_inputs.py) the oracle's result is the exact value
rounded once at each of the method's rounding points, and so is the GPU's:
the output must be identical bit for bit.  The tokens are basis vectors, so
the gate and up projections read single codes back through the kernels: a
code, a sign or a scale placed in the wrong lane, k-slot, plane or tile shows
up as a different output, which a tolerance could hide.  Covered: every code
family in every projection position, decode slots of 1..8 rows (single-token
launch, banded and per-group multi-row paths, fused and separate combine) at
the full 4096/2048 shapes, and prefill row tiles that are full, ragged and
multiple per expert at small and full shapes (2-bit/3-bit and ternary GEMMs).
The odd-scale variants put 11-bit scales in one projection of a 2-bit layer:
there the prefill's fp16 weight terms are off by the rounding residual of
0.75 s, and only an exact fp6 x fp4 correction gives the identical output.
"""
import numpy as np
import pytest
import torch

import bit_quantized_moe_router_amd as bq
import synth
import workloads
from exact_inputs import PROJ, basis_tokens, check_premise, exact_mats, top1_logits
from helpers import oracle_outputs, parity_stats

pytestmark = pytest.mark.gpu

DEV = "cuda"
FAMILIES = [(2, 2, 2), (3, 3, 2), (1, 1, 1), (3, 2, 3)]

SMALL = synth.small_config(synth.CONFIGS["c3"], name="exact_small", T=700, d=512, E=16, k=1,
                           inter=256, n_shared=1, router=False, zipf_s=0.0)
FULL = synth.small_config(synth.CONFIGS["c3"], name="exact_full", T=256, E=16, k=1,
                          n_shared=1, router=False, zipf_s=0.0)
# inter not a multiple of 256: all-ternary layers take the 4-wave fp16-term kernel and
# 2-bit layers the bf16-operand kernel (the wider shapes above take the 8-wave one)
NARROW = synth.small_config(synth.CONFIGS["c3"], name="exact_narrow", T=400, d=768, E=12, k=1,
                            inter=384, n_shared=1, router=False, zipf_s=0.0)

# single-token decode at hidden sizes of 17 and 31 k-blocks of 128: the gate/up launch
# splits them over two waves of up to 16 k-blocks, the second wave's range ragged (the
# clamped k-block path); decode only (prefill needs d % 256 == 0)
ODD_KB = [synth.small_config(synth.CONFIGS["c3"], name=f"exact_kb{d // 128}", T=8, d=d, E=16,
                             k=1, inter=256, n_shared=1, router=False, zipf_s=0.0)
          for d in (2176, 3968)]


# inter above 2048: decode takes the separate down launch and the few-token combine at
# every token count (the fused down + combine covers I <= 2048)
WIDE_I = synth.small_config(synth.CONFIGS["c3"], name="exact_widei", T=8, d=512, E=16, k=1,
                            inter=2560, n_shared=1, router=False, zipf_s=0.0)


def odd_kb_positions(d):
    """Basis positions in the first and last k-block of each wave's range and in the
    last, ragged k-block."""
    kb = d // 128
    half = (kb + 1) // 2
    return [0, half * 128 - 1, half * 128, half * 128 + 77, d - 128, d - 1]


# decode routing patterns (token -> expert): slot heights 1..8 and a 9-slot list
DECODE_PATTERNS = [[3], [5, 5], [1, 2, 1], [7, 7, 7, 7], [0, 0, 0, 0, 0], [2, 9, 9, 9, 9, 9],
                   [4] * 7, [6] * 8, [1, 2, 3, 4, 5, 6, 7, 8], [11, 11, 11, 12, 12, 13, 13, 13]]


def _skewed_experts(E, T, seed):
    rng = np.random.default_rng(seed)
    p = np.arange(1, E + 1, dtype=np.float64) ** -1.2
    p = p[rng.permutation(E)]
    return rng.choice(E, T, p=p / p.sum())


def _layer(cfg, qt, odd=""):
    c = synth.small_config(cfg, name=f"{cfg.name}_{qt}{odd}", q_gate=qt[0], q_up=qt[1],
                           q_down=qt[2])
    mats = exact_mats(c, odd=odd)
    print(f"building exact layer {c.name}", flush=True)
    return c, mats, workloads.DeviceLayer(c, 0, DEV, mats=mats)


def _run(dl, x_np, logits, mode):
    cfg = dl.cfg
    T = x_np.shape[0]
    x = torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).to(DEV)
    R = bq.alloc_routing(T, cfg.E, cfg.k, DEV, logits=torch.from_numpy(logits).to(DEV))
    ws = bq.alloc_workspace(dl.handle, T, DEV)
    out = torch.empty((T, cfg.d), dtype=torch.int16, device=DEV)
    fn = bq.moe_forward_decode if mode == "decode" else bq.moe_forward_prefill
    fn(dl.handle, x, T, bq.MOE_LOGITS_GIVEN, R, ws, out)
    torch.cuda.synchronize()
    return out.cpu().numpy().view(np.uint16), R.counts.cpu().numpy()


def _assert_identical(gpu, ref, what):
    st = parity_stats(gpu, ref)
    print(f"  {what}: {st}", flush=True)
    bad = np.argwhere(gpu != ref)
    assert bad.size == 0, (what, bad[:8].tolist(), st)


@pytest.mark.parametrize("qt", FAMILIES)
def test_exact_decode_full_shapes(qt):
    cfg, mats, dl = _layer(FULL, qt)
    for i, pat in enumerate(DECODE_PATTERNS):
        experts = np.array(pat)
        x, _ = basis_tokens(cfg.d, len(pat), seed=1000 + i)
        lg = top1_logits(experts, cfg.E)
        print(f"[exact decode {qt}] T={len(pat)} experts={pat}", flush=True)
        out, _ = _run(dl, x, lg, "decode")
        ref = oracle_outputs(cfg, 0, x, lg, np.arange(len(pat)), False, mats=mats)
        _assert_identical(out, ref, f"decode {qt} T={len(pat)}")


@pytest.mark.parametrize("cfg0", ODD_KB, ids=lambda c: c.name)
@pytest.mark.parametrize("qt", [(2, 2, 2), (3, 3, 2), (1, 1, 1)])
def test_exact_single_token_decode_odd_kblocks(cfg0, qt):
    cfg, mats, dl = _layer(cfg0, qt)
    for i, pos in enumerate(odd_kb_positions(cfg.d)):
        x, _ = basis_tokens(cfg.d, 1, seed=3000 + i, positions=[pos])
        lg = top1_logits(np.array([(3 * i + 1) % cfg.E]), cfg.E)
        print(f"[exact decode {qt} d={cfg.d}] position {pos}", flush=True)
        out, _ = _run(dl, x, lg, "decode")
        ref = oracle_outputs(cfg, 0, x, lg, np.arange(1), False, mats=mats)
        _assert_identical(out, ref, f"decode {qt} d={cfg.d} position {pos}")


@pytest.mark.parametrize("qt", [(2, 2, 2), (3, 3, 2), (1, 1, 1)])
def test_exact_decode_separate_down_and_combine(qt):
    cfg, mats, dl = _layer(WIDE_I, qt)
    for i in (0, 1, 3, 8, 9):
        pat = DECODE_PATTERNS[i]
        experts = np.array(pat)
        x, _ = basis_tokens(cfg.d, len(pat), seed=4000 + i)
        lg = top1_logits(experts, cfg.E)
        print(f"[exact decode {qt} inter={cfg.inter}] T={len(pat)} experts={pat}", flush=True)
        out, _ = _run(dl, x, lg, "decode")
        ref = oracle_outputs(cfg, 0, x, lg, np.arange(len(pat)), False, mats=mats)
        _assert_identical(out, ref, f"decode {qt} inter={cfg.inter} T={len(pat)}")


@pytest.mark.parametrize("qt", FAMILIES)
def test_exact_prefill_small_reads_whole_matrices(qt):
    # T = 700 basis tokens over d = 512 positions: every gate/up code of every expert a
    # token is routed to is read back; skewed routing gives experts of 1..4 row tiles
    cfg, mats, dl = _layer(SMALL, qt)
    x, _ = basis_tokens(cfg.d, cfg.T, seed=7, positions=(np.arange(cfg.T) * 37) % cfg.d)
    experts = _skewed_experts(cfg.E, cfg.T, seed=8)
    lg = top1_logits(experts, cfg.E)
    print(f"[exact prefill small {qt}] T={cfg.T}", flush=True)
    out, counts = _run(dl, x, lg, "prefill")
    print(f"  rows per expert {counts.tolist()}", flush=True)
    ref = oracle_outputs(cfg, 0, x, lg, np.arange(cfg.T), False, mats=mats)
    _assert_identical(out, ref, f"prefill small {qt}")


@pytest.mark.parametrize("qt", [(2, 2, 2), (1, 1, 1)])
def test_exact_prefill_narrow_shapes(qt):
    cfg, mats, dl = _layer(NARROW, qt)
    x, _ = basis_tokens(cfg.d, cfg.T, seed=11, positions=(np.arange(cfg.T) * 41) % cfg.d)
    experts = _skewed_experts(cfg.E, cfg.T, seed=12)
    lg = top1_logits(experts, cfg.E)
    print(f"[exact prefill narrow {qt}] T={cfg.T}", flush=True)
    out, counts = _run(dl, x, lg, "prefill")
    print(f"  rows per expert {counts.tolist()}", flush=True)
    ref = oracle_outputs(cfg, 0, x, lg, np.arange(cfg.T), False, mats=mats)
    _assert_identical(out, ref, f"prefill narrow {qt}")


@pytest.mark.parametrize("qt", [(2, 2, 2), (3, 3, 2), (1, 1, 1)])
def test_exact_prefill_full_shapes(qt):
    cfg, mats, dl = _layer(FULL, qt)
    x, _ = basis_tokens(cfg.d, cfg.T, seed=9)
    experts = _skewed_experts(cfg.E, cfg.T, seed=10)
    lg = top1_logits(experts, cfg.E)
    print(f"[exact prefill full {qt}] T={cfg.T}", flush=True)
    out, counts = _run(dl, x, lg, "prefill")
    print(f"  rows per expert {counts.tolist()}", flush=True)
    ref = oracle_outputs(cfg, 0, x, lg, np.arange(cfg.T), False, mats=mats)
    _assert_identical(out, ref, f"prefill full {qt}")


@pytest.mark.parametrize("odd", PROJ)
def test_exact_odd_scales_prefill(odd):
    for cfg, seeds in ((SMALL, (7, 8)), (FULL, (9, 10))):
        c, mats, dl = _layer(cfg, (2, 2, 2), odd)
        pos = (np.arange(c.T) * 37) % c.d if cfg is SMALL else None
        x, _ = basis_tokens(c.d, c.T, seed=seeds[0], positions=pos)
        experts = _skewed_experts(c.E, c.T, seed=seeds[1])
        lg = top1_logits(experts, c.E)
        print(f"[exact prefill odd {odd} scales] {c.name} T={c.T}", flush=True)
        out, counts = _run(dl, x, lg, "prefill")
        print(f"  rows per expert {counts.tolist()}", flush=True)
        ref = oracle_outputs(c, 0, x, lg, np.arange(c.T), False, mats=mats)
        _assert_identical(out, ref, f"prefill odd {odd} {c.name}")


@pytest.mark.parametrize("odd", PROJ)
def test_exact_odd_scales_decode(odd):
    cfg, mats, dl = _layer(FULL, (2, 2, 2), odd)
    for i in (0, 3, 8):
        pat = DECODE_PATTERNS[i]
        experts = np.array(pat)
        x, _ = basis_tokens(cfg.d, len(pat), seed=2000 + i)
        lg = top1_logits(experts, cfg.E)
        print(f"[exact decode odd {odd} scales] T={len(pat)} experts={pat}", flush=True)
        out, _ = _run(dl, x, lg, "decode")
        ref = oracle_outputs(cfg, 0, x, lg, np.arange(len(pat)), False, mats=mats)
        _assert_identical(out, ref, f"decode odd {odd} T={len(pat)}")
