#!/usr/bin/env python3
"""Benchmark of the quantized MoE expert layer on one MI355X.

Default run (prints one JSON line):
  * decode, 1 token (256 experts top-8 + shared, d=4096, I=2048, 2-bit group-32
    weights): one step = one full layer call (router, top-k, permutation,
    gate/up + SiLU, down + weighted combine).  Each step uses a fresh token and
    the next of 8 device copies of the layer (16 GB), so no step finds its
    expert bytes in the 256 MB Infinity Cache.  The K timed steps are one HIP
    graph; `value` is packed expert bytes per step / step time (GB/s).
  * roofline: the gate/up kernel (two thirds of the streamed bytes) timed
    launch by launch with HIP events on its stream.
  * prefill, 8192 tokens (logits given): tokens/s of the full layer call and
    the grouped GEMMs' matrix-core utilisation (useful flops / GEMM time /
    2.5 PFLOP/s).
  * decode_kernels: packed expert bytes / (gate/up + down kernel time), the
    kernels' HBM figure; us_per_layer_warm: the same layer and token every
    step (experts cached), for reference only.
  * ceilings: measured on the box (libbqceil.so) -- the best single-launch HBM
    read rate at the kernels' byte counts and dense bf16 matrix-core TFLOP/s;
    each kernel figure is also given as a fraction of these.
  * cpu_baseline: the CPU oracle on a bounded sample of decode tokens.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "quantized MoE layer: decode µs/layer + HBM GB/s; prefill tokens/s + MFMA %"
HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = ["bit_quantized_moe_router_amd/csrc/decode.hip",
                  "bit_quantized_moe_router_amd/csrc/device_common.h",
                  "bit_quantized_moe_router_amd/csrc/topk_common.h"]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per launch from the rocprofv3 counter runs, if taken on this kernel source."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    ent = t.get(kernel)
    if not ent or ent.get("source_hash") != kernel_source_hash():
        return None
    return ent.get("bytes_per_launch")


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="c1", choices=["c1", "c2"], help="decode workload")
    ap.add_argument("--copies", type=int, default=8, help="device copies of the layer to rotate")
    ap.add_argument("--prefill-config", default="c3", choices=["c3", "c4", "none"])
    ap.add_argument("--prefill-steps", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="budget of the CPU-oracle sample (0 disables it)")
    ap.add_argument("--kernel-loop", type=int, default=0,
                    help="profiling aid: only launch one decode stage (--loop-stage) this many "
                         "times")
    ap.add_argument("--loop-stage", default="gateup", choices=["gateup", "down"],
                    help="the stage --kernel-loop launches")
    ap.add_argument("--extra", default="c2,c2s,c4,c1t",
                    help="further workloads measured after the headline ones and reported in "
                         "the same line: c2 (decode, 8 tokens), c2s (c2 through a 2-bit shadow "
                         "of its 3-bit experts), c4 (4-layer prefill stack), c1t (c1 decode with "
                         "ternary experts), c2m (c2 with its 64 most favoured experts read from "
                         "a 2-bit copy; not run by default); 'none' skips them")
    ap.add_argument("--no-ceilings", action="store_true",
                    help="skip the measured roofline ceilings (read stream, matrix-core peak)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="profiling aid: run only the prefill leg and print its result")
    ap.add_argument("--traffic-probe", action="store_true",
                    help="profiling aid: only run 10 device copies of 256 MiB (a plain copy of "
                         "known size, to calibrate the HBM byte counters)")
    return ap.parse_args()


def decode_leg(args, dev):
    import numpy as np
    import torch

    import bit_quantized_moe_router_amd as bq
    import synth
    import workloads

    cfg = synth.CONFIGS[args.config]
    qts = getattr(args, "qtypes", None)
    if qts is not None:  # the same shapes with other code families
        cfg = synth.small_config(cfg, name=f"{cfg.name}_{'_'.join(synth_qname(q) for q in qts)}",
                                 q_gate=qts[0], q_up=qts[1], q_down=qts[2])
    T, K, W, C = cfg.T, args.steps, args.warmup, max(1, args.copies)
    log(f"[decode] building {cfg.name} + {C - 1} device copies")
    shadow = getattr(args, "shadow", None)
    base = workloads.DeviceLayer(cfg, 0, dev, shadow_qtypes=shadow)
    cfg = base.cfg  # the shadow's code families when one is built
    experts = [base.experts] + [base.experts.clone() for _ in range(C - 1)]
    shared = [base.shared] + [None if base.shared is None else base.shared.clone()
                              for _ in range(C - 1)]
    handles = [base.make_handle(e, s) for e, s in zip(experts, shared)]
    # per-expert mixed precision: a second copy of the routed experts in the families
    # alt_q, read for the n_alt experts the router bias favours most
    alt = getattr(args, "alt", None)
    sel_np = np.zeros(cfg.E, bool)
    fam = {False: cfg.qtypes}
    if alt is not None:
        alt_q, n_alt = alt
        adl = workloads.DeviceLayer(cfg, 0, dev, shadow_qtypes=alt_q)
        bias = synth.gen_bias(cfg, 0) if cfg.router else None
        order = np.argsort(-bias, kind="stable") if bias is not None else np.arange(cfg.E)
        sel_np[order[:n_alt]] = True
        sel = torch.from_numpy(sel_np.astype(np.uint8)).to(dev)
        alt_ex = [adl.experts] + [adl.experts.clone() for _ in range(C - 1)]
        handles = [bq.make_layer(cfg.d, cfg.inter, cfg.E, cfg.k, cfg.n_shared, cfg.qtypes, e,
                                 base.stride, s_, base.router_w, base.router_bias,
                                 alt=(a_, adl.stride, alt_q, sel))
                   for e, s_, a_ in zip(experts, shared, alt_ex)]
        fam[True] = tuple(alt_q)

    def copy_bytes(counts, gateup_only=False):
        # packed bytes one step reads: each active routed expert from its copy, plus shared
        act = counts.cpu().numpy() > 0
        def per(q):
            if gateup_only:
                return (bq.moe_packed_bytes(q[0], cfg.d, cfg.inter) +
                        bq.moe_packed_bytes(q[1], cfg.d, cfg.inter))
            return bq.moe_expert_bytes(*q, cfg.d, cfg.inter)
        n_alt_act = int((act & sel_np).sum())
        return ((int(act.sum()) - n_alt_act + cfg.n_shared) * per(fam[False]) +
                n_alt_act * (per(fam[True]) if n_alt_act else 0))
    n = W + K
    n_tok = max(n, C)  # the per-copy kernel timings below take token j for copy j
    X = synth.gen_x(cfg, T=T * n_tok).reshape(n_tok, T, cfg.d)
    xd = torch.from_numpy(X.view(np.int16)).to(dev)
    R = bq.alloc_routing(T, cfg.E, cfg.k, dev)
    ws = bq.alloc_workspace(handles[0], T, dev)
    out = torch.empty((T, cfg.d), dtype=torch.int16, device=dev)
    router_bytes = cfg.E * cfg.d * 4 if cfg.router else 0

    def step(i):
        bq.moe_forward_decode(handles[i % C], xd[i], T, 0, R, ws, out)

    # bytes streamed per step: each active expert (and the shared one) once
    active, step_bytes = [], []
    for i in range(W, n):
        step(i)
        active.append(int((R.counts > 0).sum().item()) + cfg.n_shared)
        step_bytes.append(copy_bytes(R.counts))
    torch.cuda.synchronize()
    bytes_per_step = float(np.mean(step_bytes))
    for i in range(W):
        step(i)
    torch.cuda.synchronize()

    # eager timing (includes host launch overhead)
    t0 = time.perf_counter()
    for i in range(W, n):
        step(i)
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / K

    # the K timed steps as one HIP graph
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(W, n):
            step(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / K

    # dominant kernel: gate/up, one launch per prepared workspace (layer copy j, token j)
    wss = [bq.alloc_workspace(handles[0], T, dev) for _ in range(C)]
    Rs = [bq.alloc_routing(T, cfg.E, cfg.k, dev) for _ in range(C)]
    outs = [torch.empty((T, cfg.d), dtype=torch.int16, device=dev) for _ in range(C)]
    gu_bytes = []
    for j in range(C):
        bq.moe_forward_decode(handles[j], xd[j], T, 0, Rs[j], wss[j], outs[j])
        gu_bytes.append(copy_bytes(Rs[j].counts, gateup_only=True))
    torch.cuda.synchronize()
    GU = bq.MOE_DECODE_STAGE_GATEUP
    if args.kernel_loop:
        st = GU if args.loop_stage == "gateup" else bq.MOE_DECODE_STAGE_DOWN
        for r in range(args.kernel_loop):
            j = r % C
            bq.moe_forward_decode_stages(handles[j], xd[j], T, 0, Rs[j], wss[j], outs[j], st)
        torch.cuda.synchronize()
        return None
    # back-to-back launches between one pair of events on the launch stream:
    # the average includes the short gap between consecutive kernels
    reps = max(K, 8 * C)

    def stage_us(stage):
        for r in range(C):
            bq.moe_forward_decode_stages(handles[r], xd[r], T, 0, Rs[r], wss[r], outs[r], stage)
        a_ev, b_ev = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a_ev.record()
        for r in range(reps):
            j = r % C
            bq.moe_forward_decode_stages(handles[j], xd[j], T, 0, Rs[j], wss[j], outs[j], stage)
        b_ev.record()
        torch.cuda.synchronize()
        return a_ev.elapsed_time(b_ev) * 1e3 / reps

    gu_us = stage_us(GU)
    # the down projection (+ combine) re-runs on each copy's h from the gate/up runs above
    dn_us = stage_us(bq.MOE_DECODE_STAGE_DOWN)
    gu_b = float(np.mean([gu_bytes[r % C] for r in range(reps)]))
    exp_b = float(np.mean([copy_bytes(Rs[r % C].counts) for r in range(C)]))

    # warm: the same layer copy and token every step (its experts stay in the
    # last-level cache), K steps as one graph
    gw = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gw):
        for i in range(K):
            step(W)
    gw.replay()
    torch.cuda.synchronize()
    e0.record()
    gw.replay()
    e1.record()
    torch.cuda.synchronize()
    warm_ms = e0.elapsed_time(e1) / K
    traffic = measured_traffic("k_dec_gateup")
    roof = {"kernel": "k_dec_gateup (decode gate/up + SiLU)", "bound": "hbm",
            "achieved": gu_b / (gu_us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": gu_b / (gu_us * 1e-6) / 1e9 / HBM_PEAK_GBS, "traffic": traffic,
            "avg_launch_us": gu_us, "algorithmic_bytes_per_launch": gu_b,
            "timing": "HIP events around back-to-back launches on the launch stream (includes "
                      "the gaps between launches); the rocprofv3 kernel-trace average of the same "
                      "command is kept under profiles/"}
    kernels = {"gateup_us": gu_us, "down_us": dn_us, "packed_expert_bytes": exp_b,
               "gbs": exp_b / ((gu_us + dn_us) * 1e-6) / 1e9,
               "frac": exp_b / ((gu_us + dn_us) * 1e-6) / 1e9 / HBM_PEAK_GBS}
    res = dict(cfg=cfg, ms=ms, eager_ms=eager_ms, warm_ms=warm_ms, bytes_per_step=bytes_per_step,
               router_bytes=router_bytes, roof=roof, kernels=kernels,
               active=float(np.mean(active)))
    del g, gw, experts, shared, handles
    torch.cuda.empty_cache()
    return res


def ceilings_leg(dev, sizes):
    """Measured roofline ceilings (libbqceil.so): the best single-launch HBM read
    rate for each size over a few launch shapes (rotating over 2 GiB so the
    last-level cache holds none of it), and dense bf16 matrix-core TFLOP/s."""
    import ctypes

    import torch

    from bit_quantized_moe_router_amd import build as B

    lib = ctypes.CDLL(B.CEIL_LIB)
    lib.bqc_read_stream.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int,
                                    ctypes.c_void_p, ctypes.c_void_p]
    lib.bqc_mfma_bf16.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.bqc_mfma_bf16_flops.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.bqc_mfma_bf16_flops.restype = ctypes.c_double
    stream = torch.cuda.current_stream().cuda_stream
    span = 256 << 20
    buf = torch.ones(8 * span, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1 << 16, dtype=torch.int32, device=dev)
    base = buf.data_ptr()
    reps = 24

    def timed(launch):
        launch(0)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for r in range(reps):
            launch(r)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps  # ms

    read = {}
    for n in sizes:
        best = None
        for blocks, unroll in ((512, 4), (1024, 2), (1024, 4), (2048, 1)):
            def launch(r, n=n, blocks=blocks, unroll=unroll):
                assert lib.bqc_read_stream(base + (r % 8) * span, n, blocks, unroll,
                                           sink.data_ptr(), stream) == 0
            ms = timed(launch)
            best = ms if best is None or ms < best else best
        read[str(n)] = {"us": best * 1e3, "gbs": n / (best * 1e-3) / 1e9}
    blocks, iters = 1024, 2000

    def mlaunch(r):
        assert lib.bqc_mfma_bf16(blocks, iters, sink.data_ptr(), stream) == 0
    ms = timed(mlaunch)
    tflops = lib.bqc_mfma_bf16_flops(blocks, iters) / (ms * 1e-3) / 1e12
    del buf
    torch.cuda.empty_cache()
    return {"hbm_read": read, "mfma_bf16_tflops": tflops,
            "note": "single launches, best of 4 launch shapes; spec peaks 8000 GB/s, 2500 TFLOP/s"}


def prefill_leg(args, dev):
    import numpy as np
    import torch

    import bit_quantized_moe_router_amd as bq
    import synth
    import workloads

    cfg = synth.CONFIGS[args.prefill_config]
    T = cfg.T
    log(f"[prefill] building {cfg.name}")
    layers = [workloads.DeviceLayer(cfg, l, dev) for l in range(cfg.layers)]
    x = torch.from_numpy(synth.gen_x(cfg).view(np.int16)).to(dev)
    bufs = [x, torch.empty_like(x)]
    Rs = [bq.alloc_routing(T, cfg.E, cfg.k, dev,
                           logits=torch.from_numpy(synth.gen_logits(cfg, l)).to(dev))
          for l in range(cfg.layers)]
    ws = bq.alloc_workspace(layers[0].handle, T, dev)
    flags = bq.MOE_LOGITS_GIVEN | (bq.MOE_ADD_RESIDUAL if cfg.residual else 0)

    def stack(mask=bq.MOE_PREFILL_STAGES_ALL, events=None):
        for l, dl in enumerate(layers):
            src, dst = bufs[l % 2], bufs[(l + 1) % 2]
            if events is not None:
                events[l][0].record()
            bq.moe_forward_prefill_stages(dl.handle, src, T, flags, Rs[l], ws, dst, mask)
            if events is not None:
                events[l][1].record()

    stack()
    torch.cuda.synchronize()
    K = max(1, args.prefill_steps)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(K):
        stack()
    e1.record()
    torch.cuda.synchronize()
    ms_stack = e0.elapsed_time(e1) / K
    # grouped-GEMM time per layer: run each layer's preparation, then time its GEMM stages
    gemm_ms = []
    rows = []
    for l, dl in enumerate(layers):
        src, dst = bufs[l % 2], bufs[(l + 1) % 2]
        prep = bq.MOE_PREFILL_STAGE_ROUTE | bq.MOE_PREFILL_STAGE_STAGE_X
        bq.moe_forward_prefill_stages(dl.handle, src, T, flags, Rs[l], ws, dst, prep)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(K)]
        for r in range(K):
            ev[r][0].record()
            bq.moe_forward_prefill_stages(dl.handle, src, T, flags, Rs[l], ws, dst,
                                          bq.MOE_PREFILL_STAGE_GATEUP | bq.MOE_PREFILL_STAGE_DOWN)
            ev[r][1].record()
        torch.cuda.synchronize()
        gemm_ms.append(float(np.mean([a.elapsed_time(b) for a, b in ev])))
        rows.append(int(Rs[l].counts.sum().item()) + T * cfg.n_shared)
    flops = sum(2.0 * r * 3 * cfg.d * cfg.inter for r in rows)
    gemm_total_ms = float(sum(gemm_ms))
    res = {"workload": cfg.name, "T": T, "layers": cfg.layers,
           "ms_per_stack": ms_stack, "ms_per_layer": ms_stack / cfg.layers,
           "tokens_per_s": T / (ms_stack * 1e-3),
           "tokens_per_s_per_layer": T * cfg.layers / (ms_stack * 1e-3),
           "gemm_ms_per_layer": gemm_ms, "useful_tflop_per_stack": flops / 1e12,
           "mfma_frac": flops / (gemm_total_ms * 1e-3) / (BF16_PEAK_TFLOPS * 1e12),
           "mfma_frac_whole_layer": flops / (ms_stack * 1e-3) / (BF16_PEAK_TFLOPS * 1e12)}
    del layers
    torch.cuda.empty_cache()
    return res


def cpu_baseline(args, cfg, bytes_per_step, threads=1):
    """The CPU oracle (C, double precision) on a bounded token sample.  threads > 1 runs the
    active experts of a step on a pool of host threads (the oracle code unchanged)."""
    from concurrent.futures import ThreadPoolExecutor

    import numpy as np

    import oracle
    import synth

    pool = ThreadPoolExecutor(threads) if threads > 1 else None
    used = 1
    budget = args.cpu_seconds
    Wr = synth.gen_router(cfg) if cfg.router else None
    bias = synth.gen_bias(cfg)
    X = synth.gen_x(cfg, T=64 * cfg.T, seed=cfg.seed + 1000).reshape(64, cfg.T, cfg.d)
    spent, done = 0.0, 0
    while done < 64 and (spent < budget or done < 2):
        x = X[done]
        mats = {}
        L = oracle.router_logits(x, Wr, bias)
        ids, w = oracle.topk_softmax(L, cfg.k)
        need = sorted(set(ids.reshape(-1).tolist())) + ([cfg.E] if cfg.n_shared else [])
        for e in need:  # regenerating the weights is not part of the timed work
            mats[e] = [synth.gen_matrix(cfg, 0, e, m) for m in range(3)]
        t0 = time.perf_counter()
        L = oracle.router_logits(x, Wr, bias)
        ids, w = oracle.topk_softmax(L, cfg.k)
        counts, offsets, perm, inv = oracle.permute(ids, cfg.E)
        y = np.zeros((cfg.T * cfg.k, cfg.d), np.uint16)
        active = [e for e in range(cfg.E) if counts[e]]

        def rows_of(e):
            rows = perm[offsets[e]:offsets[e + 1]]
            return e, oracle.expert_rows(cfg.qtypes, mats[e], x[rows])[1]

        jobs = [lambda e=e: rows_of(e) for e in active]
        if cfg.n_shared:
            jobs.append(lambda: (cfg.E, oracle.expert_rows(cfg.qtypes, mats[cfg.E], x)[1]))
        res = [j() for j in jobs] if pool is None else list(pool.map(lambda j: j(), jobs))
        used = max(used, min(threads, len(jobs)))
        ysh = None
        for e, yy in res:
            if e == cfg.E:
                ysh = yy
            else:
                y[offsets[e]:offsets[e + 1]] = yy
        oracle.combine(w, inv, y, ysh, x, False)
        spent += time.perf_counter() - t0
        done += 1
    per_step = spent / done
    if pool is not None:
        pool.shutdown()
    how = ("single-threaded C" if used == 1 else
           f"C with the step's {used} expert evaluations on {used} host threads")
    return {"value": bytes_per_step / per_step / 1e9, "unit": "GB/s", "cores": used,
            "kind": "oracle",
            "sample": f"{done} decode steps of {cfg.name} (T={cfg.T}) through the full CPU oracle "
                      f"(logits, top-k, permutation, every active expert + shared, combine), "
                      f"{how} in double precision; {per_step * 1e3:.0f} ms per step; "
                      f"weight regeneration excluded",
            "ms_per_step": per_step * 1e3, "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def cpu_model() -> str:
    """The host CPU's model name (what lscpu reports as 'Model name')."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the whole layer (all experts) fits in one MI355X's HBM "
              "and the library has no multi-GPU path; run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = "cuda:0"
    if args.traffic_probe:
        n = 256 << 20
        src = torch.ones(n, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(10):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"traffic_probe_bytes_per_copy": n, "copies": 10}), flush=True)
        return
    import bit_quantized_moe_router_amd as bq

    bq.load()
    if args.prefill_only:
        print(json.dumps({"prefill": prefill_leg(args, dev)}), flush=True)
        return
    d = decode_leg(args, dev)
    if d is None:  # profiling loop only
        return
    pre = None if args.prefill_config == "none" else prefill_leg(args, dev)
    extra = extra_legs(args, dev)
    cfg = d["cfg"]
    kern = d["kernels"]
    ceil = None
    if not args.no_ceilings:
        ceil = ceilings_leg(dev, [int(d["roof"]["algorithmic_bytes_per_launch"]),
                                  int(kern["packed_expert_bytes"]), 256 << 20])
        c_gu = ceil["hbm_read"][str(int(d["roof"]["algorithmic_bytes_per_launch"]))]["gbs"]
        c_all = ceil["hbm_read"][str(int(kern["packed_expert_bytes"]))]["gbs"]
        d["roof"]["ceiling_gbs"] = c_gu
        d["roof"]["frac_of_ceiling"] = d["roof"]["achieved"] / c_gu
        kern["ceiling_gbs"] = c_all
        kern["frac_of_ceiling"] = kern["gbs"] / c_all
        for leg in (pre, extra.get("prefill_c4")):
            if leg:
                leg["mfma_frac_of_ceiling"] = leg["mfma_frac"] * BF16_PEAK_TFLOPS / ceil["mfma_bf16_tflops"]
    cpu = cpu_baseline(args, cfg, d["bytes_per_step"]) if args.cpu_seconds > 0 else None
    cpu_par = None
    if args.cpu_seconds > 0:
        a = argparse.Namespace(**vars(args))
        a.cpu_seconds = max(2.0, args.cpu_seconds / 3)
        cpu_par = cpu_baseline(a, cfg, d["bytes_per_step"], threads=min(16, os.cpu_count() or 1))
    gbs = d["bytes_per_step"] / (d["ms"] * 1e-3) / 1e9
    line = {
        "metric": METRIC,
        "value": gbs,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": d["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": cfg.name, "T": cfg.T, "d": cfg.d, "experts": cfg.E, "top_k": cfg.k,
                   "shared": cfg.n_shared, "inter": cfg.inter,
                   "quant": [synth_qname(q) for q in cfg.qtypes], "layer_copies": args.copies,
                   "step": "one full decode layer call (fresh token, next layer copy)"},
        "us_per_layer": d["ms"] * 1e3,
        "us_per_layer_eager": d["eager_ms"] * 1e3,
        "us_per_layer_warm": d["warm_ms"] * 1e3,
        "decode_kernels": kern,
        "packed_expert_bytes_per_step": d["bytes_per_step"],
        "active_experts_per_step": d["active"],
        "gbs_incl_router": (d["bytes_per_step"] + d["router_bytes"]) / (d["ms"] * 1e-3) / 1e9,
        "hbm_frac": gbs / HBM_PEAK_GBS,
        "roofline": d["roof"],
        "cpu_baseline": cpu,
        "cpu_baseline_parallel": cpu_par,
        "ceilings": ceil,
        "prefill": pre,
        **extra,
    }
    print(json.dumps(line), flush=True)


def extra_legs(args, dev):
    """C2 decode (8 tokens, 3/3/2-bit, Zipf-biased router) and the C4 prefill stack (4 layers,
    16384 tokens, ternary, residual), each with a short run of its own."""
    want = set(args.extra.split(",")) - {"none", ""}
    out = {}
    if "c2" in want:
        a = argparse.Namespace(**vars(args))
        a.config, a.steps, a.warmup, a.copies, a.kernel_loop = "c2", 50, 5, 4, 0
        d = decode_leg(a, dev)
        gbs = d["bytes_per_step"] / (d["ms"] * 1e-3) / 1e9
        out["decode_c2"] = {
            "workload": d["cfg"].name, "T": d["cfg"].T, "steps": a.steps, "layer_copies": a.copies,
            "us_per_layer": d["ms"] * 1e3, "packed_expert_bytes_per_step": d["bytes_per_step"],
            "unique_routed_experts_per_step": d["active"] - d["cfg"].n_shared,
            "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "gateup_kernel_us": d["roof"]["avg_launch_us"],
            "gateup_kernel_gbs": d["roof"]["achieved"],
            "decode_kernels": d["kernels"]}
    if "c2s" in want:
        # C2 read through its fast-mode copy: the 3-bit gate/up experts re-quantised to 2-bit
        a = argparse.Namespace(**vars(args))
        a.config, a.steps, a.warmup, a.copies, a.kernel_loop = "c2", 50, 5, 4, 0
        a.shadow = (2, 2, 2)
        d = decode_leg(a, dev)
        gbs = d["bytes_per_step"] / (d["ms"] * 1e-3) / 1e9
        out["decode_c2_shadow"] = {
            "workload": "c2_decode_t8_zipf, gate/up read from a 2-bit shadow of the 3-bit experts",
            "T": d["cfg"].T, "steps": a.steps, "layer_copies": a.copies,
            "us_per_layer": d["ms"] * 1e3, "packed_expert_bytes_per_step": d["bytes_per_step"],
            "unique_routed_experts_per_step": d["active"] - d["cfg"].n_shared,
            "gbs": gbs, "decode_kernels": d["kernels"]}
    if "c2m" in want:
        # C2 with per-expert mixed precision: the 64 experts the router bias favours most
        # read from a 2-bit copy, the rest from the 3-bit experts (one layer handle)
        a = argparse.Namespace(**vars(args))
        a.config, a.steps, a.warmup, a.copies, a.kernel_loop = "c2", 50, 5, 4, 0
        a.alt = ((2, 2, 2), 64)
        d = decode_leg(a, dev)
        gbs = d["bytes_per_step"] / (d["ms"] * 1e-3) / 1e9
        out["decode_c2_mixed"] = {
            "workload": "c2_decode_t8_zipf, the 64 most favoured experts read from a 2-bit copy",
            "T": d["cfg"].T, "steps": a.steps, "layer_copies": a.copies,
            "us_per_layer": d["ms"] * 1e3, "packed_expert_bytes_per_step": d["bytes_per_step"],
            "unique_routed_experts_per_step": d["active"] - d["cfg"].n_shared,
            "gbs": gbs, "decode_kernels": d["kernels"]}
    if "c4" in want:
        a = argparse.Namespace(**vars(args))
        a.prefill_config, a.prefill_steps = "c4", 2
        out["prefill_c4"] = prefill_leg(a, dev)
    if "c1t" in want:
        # single-token decode at c1's shapes with ternary experts (2 bits per code, as int2)
        a = argparse.Namespace(**vars(args))
        a.config, a.steps, a.warmup, a.copies, a.kernel_loop = "c1", 100, 10, 8, 0
        a.qtypes = (1, 1, 1)
        d = decode_leg(a, dev)
        gbs = d["bytes_per_step"] / (d["ms"] * 1e-3) / 1e9
        out["decode_c1_ternary"] = {
            "workload": d["cfg"].name, "T": d["cfg"].T, "steps": a.steps, "layer_copies": a.copies,
            "us_per_layer": d["ms"] * 1e3, "packed_expert_bytes_per_step": d["bytes_per_step"],
            "gbs": gbs, "hbm_frac": gbs / HBM_PEAK_GBS,
            "gateup_kernel_us": d["roof"]["avg_launch_us"],
            "gateup_kernel_gbs": d["roof"]["achieved"], "decode_kernels": d["kernels"]}
    return out


def synth_qname(q):
    return {1: "ternary", 2: "int2", 3: "int3"}[q]


if __name__ == "__main__":
    main()
