"""moe_forward_decode_noalloc (workspace in the library's static device array)
against moe_forward_decode (caller's workspace): the same kernels, so every
output -- the layer's and the routing's -- must be identical bit for bit.
Calls in a row on the array with fewer tokens after the first (the array keeps
the previous call's contents; the single-token call takes its selection inside
gate/up), then a call at other shapes; one call is also checked against the
oracle."""
import numpy as np
import pytest
import torch

import bit_quantized_moe_router_amd as bq
import synth
import workloads
from helpers import assert_parity, check_routing_exact, oracle_outputs

pytestmark = pytest.mark.gpu

DEV = "cuda"
CFG = synth.small_config(synth.CONFIGS["c2"], name="noalloc_c2shape", E=32)
SMALL = synth.small_config(synth.CONFIGS["c0"], name="noalloc_small", n_shared=1)


def _both(dl, x_np, flags):
    cfg = dl.cfg
    T = x_np.shape[0]
    x = torch.from_numpy(np.ascontiguousarray(x_np).view(np.int16)).to(DEV)
    res = []
    for noalloc in (False, True):
        R = bq.alloc_routing(T, cfg.E, cfg.k, DEV)
        out = torch.full((T, cfg.d), -1, dtype=torch.int16, device=DEV)
        if noalloc:
            bq.moe_forward_decode_noalloc(dl.handle, x, T, flags, R, out)
        else:
            ws = bq.alloc_workspace(dl.handle, T, DEV)
            bq.moe_forward_decode(dl.handle, x, T, flags, R, ws, out)
        torch.cuda.synchronize()
        res.append((out.cpu().numpy().view(np.uint16),
                    {n: getattr(R, n).cpu().numpy() for n in
                     ("logits", "topk_ids", "topk_w", "counts", "offsets", "perm_tok",
                      "inv_row")}))
    (o0, r0), (o1, r1) = res
    assert np.array_equal(o0, o1)
    for n in r0:
        assert np.array_equal(r0[n].view(np.uint8), r1[n].view(np.uint8)), n
    return o1, r1


def test_noalloc_decode_matches_decode():
    dl = workloads.DeviceLayer(CFG, 0, DEV)
    for T, flags in ((8, 0), (1, 0), (3, bq.MOE_ADD_RESIDUAL)):
        print(f"[noalloc] c2 shapes E=32 T={T} flags={flags}", flush=True)
        x = synth.gen_x(CFG, seed=500 + T, T=T)
        out, r = _both(dl, x, flags)
    rt = dict(ids=r["topk_ids"], w=r["topk_w"], counts=r["counts"], offsets=r["offsets"],
              perm_tok=r["perm_tok"][: 3 * CFG.k], inv_row=r["inv_row"], logits=r["logits"])
    check_routing_exact(CFG, rt["logits"], rt)
    ref = oracle_outputs(CFG, 0, x, rt["logits"], np.arange(3), True)
    assert_parity(out, ref, "noalloc T=3 residual")
    dls = workloads.DeviceLayer(SMALL, 0, DEV)
    print("[noalloc] small shapes T=1", flush=True)
    _both(dls, synth.gen_x(SMALL, seed=7, T=1), 0)


def test_noalloc_decode_refuses_bad_token_counts():
    dl = workloads.DeviceLayer(SMALL, 0, DEV)
    x = torch.zeros((9, SMALL.d), dtype=torch.int16, device=DEV)
    R = bq.alloc_routing(9, SMALL.E, SMALL.k, DEV)
    out = torch.empty((9, SMALL.d), dtype=torch.int16, device=DEV)
    for T in (0, 9):
        with pytest.raises(bq.MoeError) as ei:
            bq.moe_forward_decode_noalloc(dl.handle, x, T, 0, R, out)
        assert ei.value.status == bq.MOE_ERR_INVALID_ARG
