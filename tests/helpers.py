"""Helpers for the GPU parity tests: run the oracle on the experts a set of
tokens actually uses (regenerating only those experts), and the parity metrics.
"""
from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
import synth

# Tolerance on floating-point outputs: both must hold for every output tensor.
MAX_ERR_FRAC = 2e-2   # max |gpu - ref| <= 2e-2 * max |ref|
REL_L1 = 1e-3         # sum |gpu - ref| / sum |ref| <= 1e-3


def parity_stats(gpu_bf16: np.ndarray, ref_bf16: np.ndarray):
    g = oracle.bf16_to_f64(gpu_bf16)
    r = oracle.bf16_to_f64(ref_bf16)
    assert np.all(np.isfinite(g)), "non-finite GPU output"
    err = np.abs(g - r)
    ref_max = float(np.abs(r).max()) or 1.0
    return dict(max_err_frac=float(err.max()) / ref_max,
                rel_l1=float(err.sum()) / max(float(np.abs(r).sum()), 1e-300),
                frac_equal=float(np.mean(gpu_bf16 == ref_bf16)))


def assert_parity(gpu_bf16, ref_bf16, what=""):
    st = parity_stats(gpu_bf16, ref_bf16)
    print(f"  parity {what}: {st}", flush=True)
    assert st["max_err_frac"] <= MAX_ERR_FRAC, (what, st)
    assert st["rel_l1"] <= REL_L1, (what, st)
    return st


def check_routing_exact(cfg, logits, gpu, tokens=None):
    """ids, weights, counts, offsets, perm, inv_row of the GPU against the oracle run on the
    same fp32 logits.  Integer results must be identical; weights within 2 fp32 ulp-ish."""
    ids, w = oracle.topk_softmax(logits, cfg.k)
    counts, offsets, perm_tok, inv_row = oracle.permute(ids, cfg.E)
    assert np.array_equal(gpu["ids"], ids), "top-k ids differ"
    assert np.array_equal(gpu["counts"], counts), "counts differ"
    assert np.array_equal(gpu["offsets"], offsets), "offsets differ"
    assert np.array_equal(gpu["perm_tok"][: ids.size], perm_tok), "perm_tok differs"
    assert np.array_equal(gpu["inv_row"], inv_row), "inv_row differs"
    assert np.allclose(gpu["w"], w, rtol=2e-6, atol=1e-7), "weights differ"
    return ids, w, counts, offsets, perm_tok, inv_row


def shadow_mats(source_cfg, qtypes, layer, seed=None):
    """The oracle's own view of a shadow copy: per expert, each projection of `source_cfg`
    whose code family differs from `qtypes` re-quantised by the oracle (its dequantiser and
    round-to-nearest quantiser)."""
    def mats(e):
        out = []
        for m in range(3):
            c, s = synth.gen_matrix(source_cfg, layer, e, m, seed)
            if qtypes[m] != source_cfg.qtypes[m]:
                w = np.ascontiguousarray(oracle.dequant(source_cfg.qtypes[m], c, s).T)
                c, s = oracle.quantize_rtn(qtypes[m], w.astype(np.float32))
            out.append((c, s))
        return out
    return mats


def host_threads() -> int:
    """Worker threads for the oracle: the host's CPU share, at most 16."""
    import os
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def oracle_outputs(cfg, layer, x, logits, tokens, residual, seed=None, threads=None, mats=None,
                   qtypes_of=None):
    """Oracle output rows for `tokens` (bf16 [len(tokens)][d]).

    Routing comes from the oracle on `logits`; only the experts the tokens use
    are regenerated and evaluated.  Tokens are independent given their routing.
    `mats(e)`, if given, supplies expert e's three (codes, scales) in cfg's code
    families instead of the synthetic generator; `qtypes_of(e)`, if given, names the code
    families of expert e's matrices in place of cfg's (per-expert mixed precision).
    Experts are regenerated a chunk at a time (the generator runs on all cores by itself),
    then the chunk's experts are evaluated on `threads` host threads.
    """
    threads = threads or host_threads()
    tokens = np.asarray(tokens)
    ids, w = oracle.topk_softmax(logits[tokens], cfg.k)
    n = len(tokens)
    by_expert = {}
    for i in range(n):
        for j in range(cfg.k):
            by_expert.setdefault(int(ids[i, j]), []).append((i, j))
    y = np.zeros((n * cfg.k, cfg.d), np.uint16)
    inv = np.zeros((n, cfg.k), np.int32)
    ysh = np.zeros((n, cfg.d), np.uint16) if cfg.n_shared else None
    xs = x[tokens]

    def run(item):
        e, mm = item
        qt = qtypes_of(e) if qtypes_of else cfg.qtypes
        if e == cfg.E:
            _, yy = oracle.expert_rows(qt, mm, xs)
            return e, None, yy
        rows = by_expert[e]
        _, yy = oracle.expert_rows(qt, mm, xs[[i for i, _ in rows]])
        return e, rows, yy

    work = sorted(by_expert) + ([cfg.E] if cfg.n_shared else [])
    with ThreadPoolExecutor(threads) as ex:
        for c0 in range(0, len(work), 2 * threads):
            chunk = work[c0:c0 + 2 * threads]
            items = [(e, mats(e) if mats else
                      [synth.gen_matrix(cfg, layer, e, m, seed) for m in range(3)])
                     for e in chunk]
            for e, rows, yy in ex.map(run, items):
                if rows is None:
                    ysh[:] = yy
                else:
                    for (i, j), yrow in zip(rows, yy):
                        y[i * cfg.k + j] = yrow
                        inv[i, j] = i * cfg.k + j
    if residual == "both":  # (without, with) the residual, from one evaluation of the experts
        return (oracle.combine(w, inv, y, ysh, xs, False),
                oracle.combine(w, inv, y, ysh, xs, True))
    return oracle.combine(w, inv, y, ysh, xs, residual)


def stratified_tokens(counts, offsets, perm_tok, inv_row, T, tile_rows, n_shared,
                      min_tokens=256, seed=0):
    """Tokens whose rows reach every row tile of every expert.

    The permuted rows of expert e are cut into tiles of `tile_rows` rows, as
    the grouped GEMMs cut them.  For each tile not yet reached, one row is
    drawn uniformly inside it and its token is taken; a token reaches the
    tiles of all of its k rows at once.  With a shared expert (which sees all
    T tokens in order) every `tile_rows`-token block is reached too.  The
    first and last token are always in, and random tokens pad the sample to
    `min_tokens`.  Returns (sorted tokens, coverage dict).
    """
    rng = np.random.default_rng(seed)
    counts = np.asarray(counts, np.int64)
    offsets = np.asarray(offsets, np.int64)
    E = counts.size
    k = inv_row.shape[1]
    row_exp = np.repeat(np.arange(E), counts)
    row_tile = (np.arange(T * k) - offsets[row_exp]) // tile_rows
    tile_base = np.concatenate([[0], np.cumsum((counts + tile_rows - 1) // tile_rows)])
    row_key = tile_base[row_exp] + row_tile       # global tile id of each permuted row
    n_tiles = int(tile_base[-1])
    tok_keys = row_key[inv_row]                   # [T][k]
    reached = np.zeros(n_tiles, bool)
    sh_blocks = (T + tile_rows - 1) // tile_rows
    sh_reached = np.zeros(sh_blocks, bool)
    chosen = set()

    def take(t):
        chosen.add(int(t))
        reached[tok_keys[t]] = True
        sh_reached[t // tile_rows] = True

    take(0)
    take(T - 1)
    for key in rng.permutation(n_tiles):
        if reached[key]:
            continue
        e = int(np.searchsorted(tile_base, key, side="right") - 1)
        a = offsets[e] + (key - tile_base[e]) * tile_rows
        b = min(offsets[e] + counts[e], a + tile_rows)
        take(perm_tok[int(rng.integers(a, b))])
    if n_shared:
        for blk in np.flatnonzero(~sh_reached):
            take(int(rng.integers(blk * tile_rows, min(T, (blk + 1) * tile_rows))))
    while len(chosen) < min(min_tokens, T):
        take(int(rng.integers(0, T)))
    toks = np.array(sorted(chosen))
    cov = dict(tiles=n_tiles, tiles_reached=int(reached.sum()),
               shared_blocks=sh_blocks if n_shared else 0,
               shared_reached=int(sh_reached.sum()) if n_shared else 0,
               active=int((counts > 0).sum()),
               active_reached=int(np.unique(row_exp[inv_row[toks].ravel()]).size),
               tokens=int(toks.size))
    return toks, cov
