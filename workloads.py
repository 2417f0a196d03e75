"""Device-resident synthetic layers for the tests, the smoke check and the benchmark.

Glue only: draws the canonical inputs from ``synth`` (seeded, counter-based),
packs each projection with the library's own host packer
(``moe_pack_weights``) and uploads the blobs with torch.  Holds none of the
layer's arithmetic.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import torch

import bit_quantized_moe_router_amd as bq
import synth


def host_threads() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def pack_expert(cfg: synth.Config, layer: int, e: int, out: np.ndarray | None = None,
                seed: int | None = None, qtypes=None, mats=None) -> np.ndarray:
    """Packed gate|up|down blob of expert e (e == E is the shared expert).  With `qtypes`,
    a projection whose code family differs from cfg's is packed in cfg's family and then
    re-quantised to the one given (moe_requantize): a lower-bit shadow copy.  With `mats`,
    mats(e) supplies the three (codes [N][K], scales [N][K/32]) instead of the generator."""
    qt = tuple(qtypes or cfg.qtypes)
    nbytes = bq.moe_expert_bytes(*qt, cfg.d, cfg.inter)
    if out is None:
        out = np.empty(nbytes, np.uint8)
    off = 0
    given = mats(e) if mats is not None else None
    for m in range(3):
        K, N = synth.matrix_shape(cfg, m)
        c, s = given[m] if given is not None else synth.gen_matrix(cfg, layer, e, m, seed)
        nb = bq.moe_packed_bytes(qt[m], K, N)
        if qt[m] == cfg.qtypes[m]:
            bq.moe_pack_weights(qt[m], c, s, out[off:off + nb])
        else:
            src = bq.moe_pack_weights(cfg.qtypes[m], c, s)
            out[off:off + nb] = bq.moe_requantize(cfg.qtypes[m], qt[m], K, N, src)
        off += nb
    return out


class DeviceLayer:
    """One layer's packed experts (+ shared expert, router, bias) in device memory."""

    def __init__(self, cfg: synth.Config, layer: int = 0, device="cuda", seed=None,
                 experts_override=None, shadow_qtypes=None, mats=None):
        # with shadow_qtypes, the experts of `cfg` re-quantised to those code families (a
        # lower-bit copy selected per call through its own layer handle); self.cfg then
        # carries the shadow's families and self.source_cfg the original ones.  `mats(e)`,
        # if given, supplies every expert's (codes, scales) instead of the generator
        self.source_cfg = cfg
        if shadow_qtypes is not None:
            q = tuple(shadow_qtypes)
            cfg = dataclasses.replace(cfg, q_gate=q[0], q_up=q[1], q_down=q[2])
        self.cfg = cfg
        self.layer = layer
        E = cfg.E
        self.stride = bq.moe_expert_bytes(*cfg.qtypes, cfg.d, cfg.inter)
        host = np.empty(E * self.stride, np.uint8)
        src, qt = self.source_cfg, cfg.qtypes

        def work(e):
            pack_expert(src, layer, e, host[e * self.stride:(e + 1) * self.stride], seed, qt,
                        mats)

        with ThreadPoolExecutor(host_threads()) as ex:
            list(ex.map(work, range(E)))
        if experts_override is not None:
            experts_override(host, self.stride)
        self.experts = torch.from_numpy(host).to(device)
        self.shared = None
        if cfg.n_shared:
            sh = pack_expert(src, layer, E, None, seed, qt, mats)
            self.shared = torch.from_numpy(sh).to(device)
        self.router_w = None
        if cfg.router:
            self.router_w = torch.from_numpy(synth.gen_router(cfg, layer, seed)).to(device)
        b = synth.gen_bias(cfg, layer, seed) if cfg.router else None
        self.router_bias = None if b is None else torch.from_numpy(b).to(device)
        self.handle = self.make_handle(self.experts, self.shared)

    def make_handle(self, experts: torch.Tensor, shared: torch.Tensor | None) -> bq.Layer:
        c = self.cfg
        return bq.make_layer(c.d, c.inter, c.E, c.k, c.n_shared, c.qtypes, experts, self.stride,
                             shared, self.router_w, self.router_bias)
