"""How far the 4-layer ternary stack (C4 shapes) carries a tiny input difference,
measured on the oracle alone: the basis of the end-to-end bounds in
test_gpu_parity.py::test_c4_stack_stratified_and_end_to_end.

The layer has no normalisation (x <- x + MoE(x)), and its output grows about a
hundredfold per layer, so a one-ulp bf16 difference in a fraction of one
layer's outputs is amplified by the next.  This script runs 48 tokens through
the four layers twice on the oracle: once on its own outputs, once with one
bf16 ulp added to or taken from a random 0.55 % of the layer-0 outputs (the
rate at which the GPU's and the oracle's layer-0 outputs differ), and prints
the relL1 between the two after each layer.  Run: python tests/c4_sensitivity.py
(about a minute on 8 cores).  Measured: relL1 3.1e-5 after layer 0 (the
perturbation itself), 1.9e-3, 5.1e-3 and 8.5e-3 after layers 1, 2 and 3;
max|err|/max|ref| 0.52 %, 0.58 %, 0.75 % and 1.05 %.
"""
import os
import sys

import numpy as np

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))

import synth  # noqa: E402
from helpers import oracle_outputs, parity_stats  # noqa: E402


def main():
    cfg = synth.CONFIGS["c4"]
    rng = np.random.default_rng(1)
    toks = np.unique(np.concatenate([[0, cfg.T - 1], rng.choice(cfg.T, 46, replace=False)]))
    a = synth.gen_x(cfg)[toks]
    b = None
    for layer in range(cfg.layers):
        lg = synth.gen_logits(cfg, layer)[toks]
        xin = a if b is None else np.concatenate([a, b])
        lgin = lg if b is None else np.concatenate([lg, lg])
        out = oracle_outputs(cfg, layer, xin, lgin, np.arange(len(xin)), True)
        a = out[: len(toks)]
        if b is None:
            b = a.copy()
            m = rng.random(b.shape) < 0.0055
            b[m] = (b[m].astype(np.int32) + rng.choice([-1, 1], m.sum())).astype(np.uint16)
            print(f"layer {layer}: perturbed copy {parity_stats(b, a)}", flush=True)
        else:
            b = out[len(toks):]
            print(f"layer {layer}: oracle vs perturbed oracle {parity_stats(b, a)}", flush=True)


if __name__ == "__main__":
    main()
