"""GPU parity tests: the HIP path through the C ABI against the CPU oracle.

Integer results (top-k ids, counts, offsets, permutation, inverse map) must be
bit-exact; floating-point outputs must satisfy max|err| <= 2e-2 * max|ref| and
sum|err| / sum|ref| <= 1e-3.  Routing is checked by running the oracle on the
fp32 logits the GPU used, so that both sides take the integer decisions on
the same values; the GPU's own logits are checked against the oracle's
double-precision logits separately.
"""
import types

import numpy as np
import pytest
import torch

import bit_quantized_moe_router_amd as bq
import oracle
import synth
import workloads
from helpers import (assert_parity, check_routing_exact, oracle_outputs, parity_stats,
                     shadow_mats, stratified_tokens)

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _to_dev_u16(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def _host_u16(t):
    return t.cpu().numpy().view(np.uint16)


def _routing_host(R, T, k):
    return dict(ids=R.topk_ids.cpu().numpy(), w=R.topk_w.cpu().numpy(),
                counts=R.counts.cpu().numpy(), offsets=R.offsets.cpu().numpy(),
                perm_tok=R.perm_tok.cpu().numpy()[: T * k], inv_row=R.inv_row.cpu().numpy(),
                logits=R.logits.cpu().numpy())


def _run(dl, x_np, mode, flags=0, logits=None):
    cfg = dl.cfg
    T = x_np.shape[0]
    x = _to_dev_u16(x_np)
    lg = None if logits is None else torch.from_numpy(np.ascontiguousarray(logits)).to(DEV)
    R = bq.alloc_routing(T, cfg.E, cfg.k, DEV, logits=lg)
    if logits is not None:
        flags |= bq.MOE_LOGITS_GIVEN
    ws = bq.alloc_workspace(dl.handle, T, DEV)
    out = torch.empty((T, cfg.d), dtype=torch.int16, device=DEV)
    fn = bq.moe_forward_decode if mode == "decode" else bq.moe_forward_prefill
    fn(dl.handle, x, T, flags, R, ws, out)
    torch.cuda.synchronize()
    return _host_u16(out), _routing_host(R, T, cfg.k)


def _full_check(dl, x, mode, flags=0, logits=None, label="", mats=None, qtypes_of=None):
    cfg = dl.cfg
    print(f"[{label}] {mode} T={x.shape[0]} cfg={cfg.name}", flush=True)
    out, rt = _run(dl, x, mode, flags, logits)
    if logits is None:
        ref_logits = oracle.router_logits(x, synth.gen_router(cfg), synth.gen_bias(cfg))
        assert_parity_f32(rt["logits"], ref_logits)
        used = rt["logits"]
    else:
        used = logits
        assert np.array_equal(rt["logits"], logits)
    check_routing_exact(cfg, used, rt)
    tokens = np.arange(x.shape[0])
    ref = oracle_outputs(cfg, dl.layer, x, used, tokens, bool(flags & bq.MOE_ADD_RESIDUAL),
                         mats=mats, qtypes_of=qtypes_of)
    assert_parity(out, ref, f"{label} out")
    return out, rt


def assert_parity_f32(gpu, ref):
    err = np.abs(gpu.astype(np.float64) - ref.astype(np.float64))
    assert err.max() <= 2e-2 * np.abs(ref).max()
    assert err.sum() <= 1e-3 * np.abs(ref).sum()


@pytest.fixture(scope="module")
def layers():
    cache = {}

    def get(name, cfg=None):
        if name not in cache:
            if isinstance(cfg, workloads.DeviceLayer):
                cache[name] = cfg
            else:
                cfg = cfg or synth.CONFIGS[name]
                print(f"building layer {name} ({cfg.name})", flush=True)
                cache[name] = workloads.DeviceLayer(cfg, 0, DEV)
        return cache[name]

    yield get
    cache.clear()
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ tiny
def test_c0_decode(layers):
    dl = layers("c0")
    _full_check(dl, synth.gen_x(dl.cfg), "decode", label="c0")


def test_c0_prefill(layers):
    dl = layers("c0")
    out_p, _ = _full_check(dl, synth.gen_x(dl.cfg), "prefill", label="c0")
    out_d, _ = _run(dl, synth.gen_x(dl.cfg), "decode")
    # both paths compute the same layer; they may differ by bf16 rounding of near-ties only
    assert_parity(out_p, out_d, "c0 prefill vs decode")


def test_c0_route_topk_matches_oracle(layers):
    dl = layers("c0")
    cfg = dl.cfg
    x = synth.gen_x(cfg)
    R = bq.alloc_routing(cfg.T, cfg.E, cfg.k, DEV)
    ws = bq.alloc_workspace(dl.handle, cfg.T, DEV)
    bq.moe_route_topk(dl.handle, _to_dev_u16(x), cfg.T, 0, R, ws)
    torch.cuda.synchronize()
    rt = _routing_host(R, cfg.T, cfg.k)
    check_routing_exact(cfg, rt["logits"], rt)


# ------------------------------------------------------------ multi-tile
MULTI = synth.small_config(synth.CONFIGS["c3"], name="multitile", T=700, d=512, E=16, k=4,
                           inter=256, router=False, zipf_s=0.0)


def test_prefill_multitile_ragged(layers):
    dl = layers("multitile", MULTI)
    x = synth.gen_x(MULTI)
    logits = synth.gen_logits(MULTI)
    _full_check(dl, x, "prefill", logits=logits, label="multitile")


def test_prefill_multitile_residual_and_skew(layers):
    cfg = synth.small_config(MULTI, name="multitile_skew", zipf_s=1.2, residual=True,
                             q_gate=synth.QT_TERNARY, q_up=synth.QT_TERNARY,
                             q_down=synth.QT_TERNARY, T=513)
    dl = layers("multitile_skew", cfg)
    x = synth.gen_x(cfg)
    logits = synth.gen_logits(cfg)
    _full_check(dl, x, "prefill", flags=bq.MOE_ADD_RESIDUAL, logits=logits, label="skew")


def test_prefill_ternary_rows_beyond_fp16_range(layers):
    # all-ternary layers take fp16 operands: each row is staged with a power-of-two scale of
    # its own, so rows far above and far below fp16's range stay exact
    cfg = synth.small_config(MULTI, name="tern_range", q_gate=synth.QT_TERNARY,
                             q_up=synth.QT_TERNARY, q_down=synth.QT_TERNARY, T=200)
    dl = layers("tern_range", cfg)
    x = synth.gen_x(cfg).copy()
    xf = (x.astype(np.uint32) << 16).view(np.float32)
    big, tiny = slice(0, 40), slice(40, 80)
    xf[big] *= np.float32(2.0 ** 20)    # |x| up to ~2^22, beyond fp16's 65504
    xf[tiny] *= np.float32(2.0 ** -30)  # |x| ~2^-30, below fp16's smallest subnormal
    x = (xf.view(np.uint32) >> 16).astype(np.uint16)  # exact: power-of-two scaling of bf16
    logits = synth.gen_logits(cfg)
    print("[tern_range] prefill", flush=True)
    out, rt = _run(dl, x, "prefill", logits=logits)
    check_routing_exact(cfg, logits, rt)
    ref = oracle_outputs(cfg, dl.layer, x, logits, np.arange(cfg.T), False)
    for name, rows in (("big", big), ("tiny", tiny), ("plain", slice(80, cfg.T))):
        assert_parity(out[rows], ref[rows], f"tern_range {name} rows")


def test_shadow_of_3bit_experts(layers):
    # the fast-mode copy: 3-bit gate/up re-quantised to 2-bit on the host, selected through
    # its own layer handle; checked against the oracle's own re-quantisation
    src = synth.small_config(MULTI, name="shadow_src", q_gate=synth.QT_INT3,
                             q_up=synth.QT_INT3, q_down=synth.QT_INT2, T=300)
    dl = layers("shadow", workloads.DeviceLayer(src, 0, DEV, shadow_qtypes=(2, 2, 2)))
    assert dl.cfg.qtypes == (2, 2, 2) and dl.source_cfg.qtypes == (3, 3, 2)
    mats = shadow_mats(src, dl.cfg.qtypes, 0)
    _full_check(dl, synth.gen_x(src, T=8), "decode", logits=synth.gen_logits(src, T=8),
                label="shadow", mats=mats)
    _full_check(dl, synth.gen_x(src), "prefill", logits=synth.gen_logits(src), label="shadow",
                mats=mats)


@pytest.mark.parametrize("alt_q", [(2, 2, 2), (1, 1, 1), (2, 1, 1)])
def test_per_expert_mixed_precision_decode(layers, alt_q):
    # a second, lower-bit copy of the routed experts chosen per expert by a device mask.
    # Gate/up: one launch over both copies when gate and up share a family within each
    # copy, else one filtered launch per copy ((2,1,1)).  Down: the fused down + combine
    # reads both copies when the down families agree ((2,2,2) at a single token), else one
    # launch over both copies, then the combine
    src = synth.small_config(MULTI, name="shadow_src", q_gate=synth.QT_INT3,
                             q_up=synth.QT_INT3, q_down=synth.QT_INT2, T=300)
    main = layers("mix_main", src)
    alt = layers(f"mix_alt{alt_q}", workloads.DeviceLayer(src, 0, DEV, shadow_qtypes=alt_q))
    sel_np = (np.arange(src.E) % 3 == 1).astype(np.uint8)
    ids1 = oracle.topk_softmax(synth.gen_logits(src, T=1), src.k)[0][0]
    sel_np[ids1[0]], sel_np[ids1[1:]] = 1, 0  # the single token reads both copies
    sel = torch.from_numpy(sel_np).to(DEV)
    h = bq.make_layer(src.d, src.inter, src.E, src.k, src.n_shared, src.qtypes, main.experts,
                      main.stride, main.shared, main.router_w, main.router_bias,
                      alt=(alt.experts, alt.stride, alt_q, sel))
    dl = types.SimpleNamespace(cfg=src, layer=0, handle=h)
    shadow = shadow_mats(src, alt_q, 0)

    def mats(e):
        if e < src.E and sel_np[e]:
            return shadow(e)
        return [synth.gen_matrix(src, 0, e, m) for m in range(3)]

    def qtypes_of(e):
        return alt_q if e < src.E and sel_np[e] else src.qtypes

    for T in (1, 4, 8):
        x_np, lg_np = synth.gen_x(src, T=T), synth.gen_logits(src, T=T)
        full, rt = _full_check(dl, x_np, "decode", logits=lg_np, label=f"mixed{alt_q}",
                               mats=mats, qtypes_of=qtypes_of)
        used = np.unique(rt["ids"][:T])
        assert sel_np[used].any() and not sel_np[used].all()  # both copies were read
        # the stages one call at a time give the full call's output bit for bit
        x = _to_dev_u16(x_np)
        R = bq.alloc_routing(T, src.E, src.k, DEV,
                             logits=torch.from_numpy(np.ascontiguousarray(lg_np)).to(DEV))
        ws = bq.alloc_workspace(h, T, DEV)
        out = torch.zeros((T, src.d), dtype=torch.int16, device=DEV)
        for st in (bq.MOE_DECODE_STAGE_ROUTE, bq.MOE_DECODE_STAGE_SELECT,
                   bq.MOE_DECODE_STAGE_GATEUP, bq.MOE_DECODE_STAGE_DOWN):
            bq.moe_forward_decode_stages(h, x, T, bq.MOE_LOGITS_GIVEN, R, ws, out, st)
        torch.cuda.synchronize()
        assert np.array_equal(_host_u16(out), full), T
    with pytest.raises(bq.MoeError) as ei:
        _run(dl, synth.gen_x(src, T=8), "prefill", logits=synth.gen_logits(src, T=8))
    assert ei.value.status == bq.MOE_ERR_UNSUPPORTED


@pytest.mark.parametrize("alt_q", [(2, 2, 2), (2, 1, 1)])
def test_mixed_precision_decode_wide(layers, alt_q):
    """The per-expert second copy at d = 4096: the single-token gate/up launch over both
    copies (or one per copy) on two waves of 16 k-blocks, and T = 3."""
    src = synth.small_config(MULTI, name="mixwide_src", d=4096, inter=256, q_gate=synth.QT_INT3,
                             q_up=synth.QT_INT3, q_down=synth.QT_INT2, T=3)
    main = layers("mixwide_main", src)
    alt = layers(f"mixwide_alt{alt_q}",
                 workloads.DeviceLayer(src, 0, DEV, shadow_qtypes=alt_q))
    ids1 = oracle.topk_softmax(synth.gen_logits(src, T=1), src.k)[0][0]
    sel_np = np.zeros(src.E, np.uint8)
    sel_np[ids1[0]] = sel_np[ids1[2]] = 1  # the single token reads both copies
    h = bq.make_layer(src.d, src.inter, src.E, src.k, src.n_shared, src.qtypes, main.experts,
                      main.stride, main.shared, main.router_w, main.router_bias,
                      alt=(alt.experts, alt.stride, alt_q, torch.from_numpy(sel_np).to(DEV)))
    dl = types.SimpleNamespace(cfg=src, layer=0, handle=h)
    shadow = shadow_mats(src, alt_q, 0)

    def mats(e):
        if e < src.E and sel_np[e]:
            return shadow(e)
        return [synth.gen_matrix(src, 0, e, m) for m in range(3)]

    def qtypes_of(e):
        return alt_q if e < src.E and sel_np[e] else src.qtypes

    for T in (1, 3):
        _full_check(dl, synth.gen_x(src, T=T), "decode", logits=synth.gen_logits(src, T=T),
                    label=f"mixed wide {alt_q}", mats=mats, qtypes_of=qtypes_of)


def test_prefill_int3_mixed(layers):
    cfg = synth.small_config(MULTI, name="int3mix", q_gate=synth.QT_INT3, q_up=synth.QT_INT2,
                             q_down=synth.QT_INT3, T=300)
    dl = layers("int3mix", cfg)
    _full_check(dl, synth.gen_x(cfg), "prefill", logits=synth.gen_logits(cfg), label="int3mix")
    _full_check(dl, synth.gen_x(cfg, T=8), "decode", logits=synth.gen_logits(cfg, T=8),
                label="int3mix")


# ------------------------------------------------------------- full size
def test_c1_decode_full(layers):
    dl = layers("c1")
    _full_check(dl, synth.gen_x(dl.cfg), "decode", label="c1")


def test_c2_decode_full(layers):
    dl = layers("c2")
    out, rt = _full_check(dl, synth.gen_x(dl.cfg), "decode", label="c2")
    U = int((rt["counts"] > 0).sum())
    print(f"  c2 unique routed experts U={U}", flush=True)


def test_decode_is_deterministic(layers):
    dl = layers("c2")
    x = synth.gen_x(dl.cfg)
    a, _ = _run(dl, x, "decode")
    b, _ = _run(dl, x, "decode")
    assert np.array_equal(a, b)


@pytest.mark.parametrize("name", ["c0", "c1", "c2"])
def test_decode_stages_one_by_one_and_rerun(layers, name):
    """The decode stages run one call at a time match the oracle, and
    re-running the two projection stages on the same workspace reproduces the
    full call's output bit for bit (no state carried between launches)."""
    dl = layers(name)
    cfg = dl.cfg
    x_np = synth.gen_x(cfg)
    T = x_np.shape[0]
    x = _to_dev_u16(x_np)
    R = bq.alloc_routing(T, cfg.E, cfg.k, DEV)
    ws = bq.alloc_workspace(dl.handle, T, DEV)
    out = torch.empty((T, cfg.d), dtype=torch.int16, device=DEV)
    print(f"[{name}] decode stages one by one", flush=True)
    for st in (bq.MOE_DECODE_STAGE_ROUTE, bq.MOE_DECODE_STAGE_SELECT,
               bq.MOE_DECODE_STAGE_GATEUP, bq.MOE_DECODE_STAGE_DOWN):
        bq.moe_forward_decode_stages(dl.handle, x, T, 0, R, ws, out, st)
    torch.cuda.synchronize()
    staged = _host_u16(out).copy()
    rt = _routing_host(R, T, cfg.k)
    check_routing_exact(cfg, rt["logits"], rt)
    ref = oracle_outputs(cfg, dl.layer, x_np, rt["logits"], np.arange(T), False)
    assert_parity(staged, ref, f"{name} staged")
    print(f"[{name}] full call, then the projection stages twice", flush=True)
    bq.moe_forward_decode(dl.handle, x, T, 0, R, ws, out)
    torch.cuda.synchronize()
    full = _host_u16(out).copy()
    assert np.array_equal(full, staged)
    both = bq.MOE_DECODE_STAGE_GATEUP | bq.MOE_DECODE_STAGE_DOWN
    for rep in range(2):
        out.zero_()
        bq.moe_forward_decode_stages(dl.handle, x, T, 0, R, ws, out, both)
        torch.cuda.synchronize()
        assert np.array_equal(_host_u16(out), full), rep


@pytest.mark.parametrize("q", [synth.QT_INT2, synth.QT_TERNARY])
def test_prefill_stages_one_by_one_and_rerun(layers, q):
    """The prefill stages run one call at a time give the full call's output bit for bit
    (2-bit: bf16-operand kernels; ternary: fp16-operand kernels), and any stage re-run on
    the same workspace reproduces it (no stage consumes what it reads)."""
    cfg = synth.small_config(MULTI, name=f"pstages{q}", q_gate=q, q_up=q, q_down=q, T=260)
    dl = layers(cfg.name, cfg)
    x_np = synth.gen_x(cfg)
    logits = synth.gen_logits(cfg)
    T = cfg.T
    x = _to_dev_u16(x_np)
    R = bq.alloc_routing(T, cfg.E, cfg.k, DEV, logits=torch.from_numpy(logits).to(DEV))
    ws = bq.alloc_workspace(dl.handle, T, DEV)
    out = torch.empty((T, cfg.d), dtype=torch.int16, device=DEV)
    fl = bq.MOE_LOGITS_GIVEN
    print(f"[pstages q={q}] full call, then stage by stage", flush=True)
    bq.moe_forward_prefill(dl.handle, x, T, fl, R, ws, out)
    torch.cuda.synchronize()
    full = _host_u16(out).copy()
    ref = oracle_outputs(cfg, dl.layer, x_np, logits, np.arange(T), False)
    assert_parity(full, ref, f"pstages q={q}")
    stages = (bq.MOE_PREFILL_STAGE_ROUTE, bq.MOE_PREFILL_STAGE_STAGE_X,
              bq.MOE_PREFILL_STAGE_GATEUP, bq.MOE_PREFILL_STAGE_DOWN,
              bq.MOE_PREFILL_STAGE_COMBINE)
    out.zero_()
    for st in stages:
        bq.moe_forward_prefill_stages(dl.handle, x, T, fl, R, ws, out, st)
    torch.cuda.synchronize()
    assert np.array_equal(_host_u16(out), full)
    for st in stages:  # each stage twice in a row
        out.zero_()
        for s_ in stages:
            bq.moe_forward_prefill_stages(dl.handle, x, T, fl, R, ws, out, s_)
            if s_ == st:
                bq.moe_forward_prefill_stages(dl.handle, x, T, fl, R, ws, out, s_)
        torch.cuda.synchronize()
        assert np.array_equal(_host_u16(out), full), st


# Row blocks the stratified samples reach: every 64-row block of the 2-bit layer (its grouped
# GEMMs run 128-row tiles, so both halves of every tile; mixed 2-/3-bit layers run 64-row
# tiles), and every 128-row tile of the all-ternary layers.
TILE_ROWS_INT = 64
TILE_ROWS_TERNARY = 128


def _assert_cover(cov, n_shared):
    print(f"  sample coverage: {cov}", flush=True)
    assert cov["tokens"] >= 256
    assert cov["tiles_reached"] == cov["tiles"]
    assert cov["active_reached"] == cov["active"]
    if n_shared:
        assert cov["shared_reached"] == cov["shared_blocks"]


@pytest.mark.timeout(600)
def test_c3_prefill_stratified(layers):
    """C3 at full size: routing bit-exact over all 8192 tokens, and the output of a
    stratified sample of >= 256 tokens whose rows reach every 64-row block of every active
    expert (and every 64-token block of the shared expert) against the oracle."""
    dl = layers("c3")
    cfg = dl.cfg
    x = synth.gen_x(cfg)
    logits = synth.gen_logits(cfg)
    print("[c3] prefill T=8192", flush=True)
    out, rt = _run(dl, x, "prefill", logits=logits)
    check_routing_exact(cfg, logits, rt)
    toks, cov = stratified_tokens(rt["counts"], rt["offsets"], rt["perm_tok"], rt["inv_row"],
                                  cfg.T, TILE_ROWS_INT, cfg.n_shared, seed=3)
    _assert_cover(cov, cfg.n_shared)
    ref = oracle_outputs(cfg, 0, x, logits, toks, False)
    assert_parity(out[toks], ref, "c3 stratified out")


# end-to-end relL1 bounds after each C4 layer: about twice the oracle's own spread
C4_E2E_REL_L1 = (1e-3, 4e-3, 1e-2, 2e-2)


@pytest.mark.timeout(900)
def test_c4_stack_stratified_and_end_to_end(layers):
    """C4, four ternary layers with the residual, at full size.

    Per layer: routing bit-exact over all 16384 tokens, and a stratified sample reaching
    every 128-row tile of every active expert checked against the oracle fed this layer's
    GPU input (the parity criterion).  End to end: 128 tokens (the first, the last and
    random ones) carried through all four layers by the oracle on its own outputs,
    compared with the GPU after each layer.  The stack has no normalisation and amplifies
    a one-ulp difference in a fraction of a layer's outputs about a hundredfold per layer:
    the oracle against itself with 0.55 % of its layer-0 outputs moved by one ulp differs
    by relL1 1.9e-3, 5.1e-3 and 8.5e-3 after layers 1-3 (tests/c4_sensitivity.py).  The
    end-to-end figures are held to about twice that."""
    cfg = synth.CONFIGS["c4"]
    x = synth.gen_x(cfg)
    rng = np.random.default_rng(4)
    e2e_toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 126, replace=False)]))
    x_e2e = x[e2e_toks].copy()
    for layer in range(cfg.layers):
        print(f"[c4] building layer {layer}", flush=True)
        dl = workloads.DeviceLayer(cfg, layer, DEV)
        logits = synth.gen_logits(cfg, layer)
        out, rt = _run(dl, x, "prefill", flags=bq.MOE_ADD_RESIDUAL, logits=logits)
        check_routing_exact(cfg, logits, rt)
        counts = rt["counts"]
        print(f"  layer {layer}: max rows/expert {counts.max()}, empty experts "
              f"{int((counts == 0).sum())}", flush=True)
        toks, cov = stratified_tokens(counts, rt["offsets"], rt["perm_tok"], rt["inv_row"],
                                      cfg.T, TILE_ROWS_TERNARY, cfg.n_shared, seed=40 + layer)
        _assert_cover(cov, cfg.n_shared)
        # one pass of the oracle over this layer's experts serves both checks
        x_cat = np.concatenate([x[toks], x_e2e])
        lg_cat = np.concatenate([logits[toks], logits[e2e_toks]])
        ref = oracle_outputs(cfg, layer, x_cat, lg_cat, np.arange(len(x_cat)), True)
        assert_parity(out[toks], ref[: len(toks)], f"c4 layer {layer} per-layer")
        x_e2e = ref[len(toks):]
        st = parity_stats(out[e2e_toks], x_e2e)
        print(f"  end-to-end after layer {layer}: {st}", flush=True)
        assert st["rel_l1"] <= C4_E2E_REL_L1[layer], (layer, st)
        assert st["max_err_frac"] <= 2e-2, (layer, st)
        x = out  # next layer's input
        del dl
        torch.cuda.empty_cache()
    print(f"  c4 end-to-end over {cfg.layers} layers: {st}", flush=True)


@pytest.mark.parametrize("T", range(1, 9))
def test_c1_decode_router_every_T(layers, T):
    """Decode at C1 shapes through the router (no given logits) for every token count
    1..8, without and with the residual: the single-token launch with its own selection,
    the fused down + combine (<= 16 slots) and the separate combine (more slots)."""
    dl = layers("c1")
    cfg = dl.cfg
    x = synth.gen_x(cfg, seed=100 + T, T=T)
    outs = {}
    for flags in (0, bq.MOE_ADD_RESIDUAL):
        print(f"[c1-router] decode T={T} flags={flags}", flush=True)
        outs[flags], rt = _run(dl, x, "decode", flags)
        ref_logits = oracle.router_logits(x, synth.gen_router(cfg), synth.gen_bias(cfg))
        assert_parity_f32(rt["logits"], ref_logits)
        check_routing_exact(cfg, rt["logits"], rt)
    slots = int((rt["counts"] > 0).sum()) + cfg.n_shared
    print(f"  T={T}: {slots} slots ({'fused' if slots <= 16 else 'separate'} combine)", flush=True)
    ref0, ref1 = oracle_outputs(cfg, 0, x, rt["logits"], np.arange(T), "both")
    assert_parity(outs[0], ref0, f"c1 router T={T}")
    assert_parity(outs[bq.MOE_ADD_RESIDUAL], ref1, f"c1 router T={T} residual")


SMALL_ROUTER = synth.small_config(synth.CONFIGS["c0"], name="small_router", n_shared=1)


def test_small_decode_router_every_T(layers):
    """Decode at C0 shapes with a shared expert, through the router, T = 1..8, without
    and with the residual (every slot list fits the fused down + combine)."""
    dl = layers("small_router", SMALL_ROUTER)
    cfg = dl.cfg
    for T in range(1, 9):
        x = synth.gen_x(cfg, seed=200 + T, T=T)
        outs = {}
        for flags in (0, bq.MOE_ADD_RESIDUAL):
            print(f"[small-router] decode T={T} flags={flags}", flush=True)
            outs[flags], rt = _run(dl, x, "decode", flags)
            ref_logits = oracle.router_logits(x, synth.gen_router(cfg), synth.gen_bias(cfg))
            assert_parity_f32(rt["logits"], ref_logits)
            check_routing_exact(cfg, rt["logits"], rt)
        ref0, ref1 = oracle_outputs(cfg, 0, x, rt["logits"], np.arange(T), "both")
        assert_parity(outs[0], ref0, f"small router T={T}")
        assert_parity(outs[bq.MOE_ADD_RESIDUAL], ref1, f"small router T={T} residual")


@pytest.mark.parametrize("q", [synth.QT_INT2, synth.QT_TERNARY, synth.QT_INT3])
def test_prefill_few_tokens(layers, q):
    """Prefill at T = 1, 2 and 5 (a partial 32-row sub-tile per expert, the few-token
    combine) through the router, with and without the residual, for each code family:
    the 8-wave 2-bit and ternary GEMMs (d = 512, inter = 256) and the bf16-operand one."""
    cfg = synth.small_config(SMALL_ROUTER, name=f"few_{q}", d=512, inter=256, E=16, k=4,
                             q_gate=q, q_up=q, q_down=q)
    dl = layers(cfg.name, cfg)
    for T in (1, 2, 5):
        x = synth.gen_x(cfg, seed=600 + T, T=T)
        for flags in (0, bq.MOE_ADD_RESIDUAL):
            _full_check(dl, x, "prefill", flags=flags, label=f"few tokens q={q} T={T}")


WIDE_E = [synth.small_config(synth.CONFIGS["c0"], name="wide_e1000", E=1000, k=6, n_shared=1,
                             T=8),
          synth.small_config(synth.CONFIGS["c0"], name="wide_e1024", E=1024, k=32, n_shared=1,
                             T=2)]


@pytest.mark.parametrize("cfg", WIDE_E, ids=lambda c: c.name)
def test_many_experts_router(layers, cfg):
    """More than 256 experts (E = 1000, not a multiple of the wave; E = 1024 with the
    largest top-k, 32) through the router: the top-k with 16 entries per lane, the
    single-token decode with its selection in the select kernel, several tokens up to
    T*k = 64, and prefill."""
    dl = layers(cfg.name, cfg)
    for T in sorted({1, cfg.T}):
        _full_check(dl, synth.gen_x(cfg, seed=300 + T, T=T), "decode", label=f"{cfg.name} T={T}")
    _full_check(dl, synth.gen_x(cfg, seed=399, T=100), "prefill", label=f"{cfg.name} prefill")


MAX_DIMS = synth.small_config(synth.CONFIGS["c0"], name="max_dims", d=8192, inter=8192, E=4,
                              k=2, n_shared=1, T=3)


@pytest.mark.timeout(600)
def test_largest_decode_dims(layers):
    """d = I = 8192, the largest the decode path takes: single-token gate/up on eight
    waves of 8 k-blocks, the down projection on sixteen waves of 4 (I > 2048: separate
    down launch and the few-token combine), several rows on eight waves of 8; and
    prefill at the same dimensions."""
    dl = layers("max_dims", MAX_DIMS)
    for T in (1, 3):
        _full_check(dl, synth.gen_x(MAX_DIMS, seed=500 + T, T=T), "decode",
                    flags=bq.MOE_ADD_RESIDUAL, label=f"max dims T={T}")
    _full_check(dl, synth.gen_x(MAX_DIMS, seed=510, T=40), "prefill", label="max dims prefill")


@pytest.mark.parametrize("q", [synth.QT_INT2, synth.QT_TERNARY])
@pytest.mark.parametrize("T", [37, 300])
def test_prefill_router_ragged(layers, q, T):
    """Prefill through the router (logits computed from x, several row blocks of the
    logits kernel with a clamped last one) at token counts that are not multiples of 8,
    with the residual; and moe_route_topk alone at the same T."""
    cfg = synth.small_config(MULTI, name=f"prouter{q}", router=True, T=T, q_gate=q, q_up=q,
                             q_down=q)
    dl = layers(cfg.name, cfg)
    x = synth.gen_x(cfg, seed=300 + T)
    _full_check(dl, x, "prefill", flags=bq.MOE_ADD_RESIDUAL, label=f"prouter q={q} T={T}")
    R = bq.alloc_routing(T, cfg.E, cfg.k, DEV)
    ws = bq.alloc_workspace(dl.handle, T, DEV)
    bq.moe_route_topk(dl.handle, _to_dev_u16(x), T, 0, R, ws)
    torch.cuda.synchronize()
    rt = _routing_host(R, T, cfg.k)
    assert_parity_f32(rt["logits"], oracle.router_logits(x, synth.gen_router(cfg),
                                                         synth.gen_bias(cfg)))
    check_routing_exact(cfg, rt["logits"], rt)


# ------------------------------------------------------------ edge cases
def test_ties_and_k_equals_E(layers):
    cfg = synth.small_config(synth.CONFIGS["c0"], name="ties", E=8, k=8, T=6, router=False)
    dl = layers("ties", cfg)
    x = synth.gen_x(cfg)
    logits = np.zeros((cfg.T, cfg.E), np.float32)
    logits[1] = [1, 1, 0.5, 1, -0.0, 0.0, 1, 2]
    logits[2] = np.float32(1e-45) * np.arange(8)
    logits[3] = -np.arange(8, dtype=np.float32)
    logits[4] = [3, 3, 3, 3, 3, 3, 3, 3]
    logits[5] = [0.0, -0.0, 0.0, -0.0, 1, 1, 1, 1]
    for mode in ("decode", "prefill"):
        _full_check(dl, x, mode, logits=logits, label=f"ties-{mode}")


def test_single_expert_top1(layers):
    cfg = synth.small_config(synth.CONFIGS["c0"], name="e1", E=1, k=1, T=5, router=False,
                             n_shared=1)
    dl = layers("e1", cfg)
    logits = np.zeros((cfg.T, 1), np.float32)
    _full_check(dl, synth.gen_x(cfg), "decode", logits=logits, label="e1")
    _full_check(dl, synth.gen_x(cfg), "prefill", logits=logits, label="e1")


def test_all_tokens_one_expert_decode(layers):
    dl = layers("c1")
    cfg = dl.cfg
    T = 8
    x = synth.gen_x(cfg, T=T)
    logits = np.tile(np.linspace(1, -1, cfg.E, dtype=np.float32), (T, 1))
    _full_check(dl, x, "decode", logits=logits, label="one-hot-experts")


def test_zero_weights_give_shared_only(layers):
    cfg = synth.small_config(synth.CONFIGS["c0"], name="zero", n_shared=1,
                             q_gate=synth.QT_TERNARY, q_up=synth.QT_TERNARY,
                             q_down=synth.QT_TERNARY, router=False)

    def zero_routed(host, stride):
        # every routed expert's codes at level 1 (weight 0); scales untouched
        for e in range(cfg.E):
            blob = workloads.pack_expert(cfg, 0, e)
            off = 0
            for m in range(3):
                K, N = synth.matrix_shape(cfg, m)
                c, s = synth.gen_matrix(cfg, 0, e, m)
                nb = bq.moe_packed_bytes(cfg.qtypes[m], K, N)
                bq.moe_pack_weights(cfg.qtypes[m], np.ones_like(c), s, blob[off:off + nb])
                off += nb
            host[e * stride:(e + 1) * stride] = blob

    dl = workloads.DeviceLayer(cfg, 0, DEV, experts_override=zero_routed)
    x = synth.gen_x(cfg)
    logits = synth.gen_logits(cfg)
    for mode in ("decode", "prefill"):
        out, _ = _run(dl, x, mode, logits=logits)
        mats = [synth.gen_matrix(cfg, 0, cfg.E, m) for m in range(3)]
        _, ysh = oracle.expert_rows(cfg.qtypes, mats, x)
        assert_parity(out, ysh, f"zero-{mode}")


@pytest.mark.parametrize("q", [synth.QT_INT2, synth.QT_TERNARY])
def test_prefill_refuses_d_not_multiple_of_256_decode_serves_it(q):
    # d = 384: a valid layer (multiples of 128), which decode handles; the prefill
    # GEMMs cover 256 output columns per block and refuse it
    cfg = synth.small_config(synth.CONFIGS["c0"], name=f"d384_{q}", d=384, inter=256,
                             q_gate=q, q_up=q, q_down=q)
    dl = workloads.DeviceLayer(cfg, 0, DEV)
    x = synth.gen_x(cfg)
    with pytest.raises(bq.MoeError) as ei:
        _run(dl, x, "prefill")
    assert ei.value.status == bq.MOE_ERR_UNSUPPORTED
    _full_check(dl, x, "decode", label="d384")
