"""The five synthetic workloads (seed i+... is fixed per workload) and a
helper that materialises one of them at a chosen batch size.

1. tiny HMM: 64 states, 8 positions, 32 symbols, batch 16 (fp32-level mode);
2. one dense sum layer: 1024 nodes over 1024 shared children, batch 128, child
   values -U(0,300) per sample - U(0,50) per entry, incoming flows U(0,1);
3. HMM: 4096 states, 32 positions, 512 symbols, batch 128 / 512;
4. HCLT-like: 768 variables x 512 categories, 1024 latents, random tree, batch 512;
5. LowRank exp_sum: HMM with 1024 states, 64 positions, 512 symbols, rank 16,
   batch 64, factor spread 0.3 .. 4 nats;
6. PD (Poon-Domingos region graph) over a 28 x 28 grid of 256-category
   variables, regions on a 4-pixel lattice, 64 latents per region, batch 128:
   general block-sparse sum layers (node blocks of 64 over lists of 64-node
   child blocks).
"""
from __future__ import annotations

import numpy as np

from . import circuits as C
from . import inputs as I

CONFIGS = {
    "tiny_hmm": dict(seed=0, kind="hmm", H=64, T=8, V=32, B=16),
    "dense_layer": dict(seed=1, kind="dense", M=1024, N=1024, groups=1, B=128),
    "hmm4096": dict(seed=2, kind="hmm", H=4096, T=32, V=512, B=512),
    "hclt": dict(seed=3, kind="hclt", num_vars=768, H=1024, K=512, B=512),
    "lowrank": dict(seed=4, kind="hmm", H=1024, T=64, V=512, B=64, rank=16, spread=1.0),
    "pd": dict(seed=5, kind="pd", H=28, W=28, K=64, C=256, split=4, B=128),
}


def make_config(name: str = None, **over):
    """Build circuit and inputs.  ``name`` picks a base config; keyword
    overrides change any field (sizes, B, seed, spread ...).  Returns a dict
    with keys circuit, params, tokens, external, seed_flows, lowrank, B."""
    cfg = dict(CONFIGS[name]) if name else {}
    cfg.update(over)
    rng = np.random.default_rng(cfg.get("seed", 0))
    B = int(cfg["B"])
    kind = cfg["kind"]
    out = dict(B=B, cfg=cfg, tokens=None, external=None, seed_flows=None, lowrank=None)
    if kind == "hmm":
        rank = int(cfg.get("rank", 0))
        circ = C.hmm(cfg["H"], cfg["T"], cfg["V"], lowrank_rank=rank, lowrank_form=cfg.get("form", "exp_sum"))
        out["params"] = I.softmax_rows_params(circ, rng)
        if cfg.get("skew"):
            out["tokens"] = I.skewed_tokens(circ, B, cfg["V"], float(cfg["skew"]), rng)
        else:
            out["tokens"] = I.uniform_tokens(circ, B, cfg["V"], rng)
        if rank > 0:
            sigma = cfg.get("sigma") or I.lowrank_sigma_for_spread(cfg.get("spread", 1.0), rank)
            out["lowrank"] = I.lowrank_factors(circ, B, sigma, rng)
    elif kind == "dense":
        circ = C.dense_layer(cfg["M"], cfg["N"], cfg.get("groups", 1))
        out["params"] = I.softmax_rows_params(circ, rng)
        out["external"] = I.external_values(circ, B, rng)
        out["seed_flows"] = I.uniform_flows(cfg.get("groups", 1) * cfg["M"], B, rng)
    elif kind == "hclt":
        circ = C.hclt(cfg["num_vars"], cfg["H"], cfg["K"], cfg.get("seed", 3))
        out["params"] = I.softmax_rows_params(circ, rng)
        out["tokens"] = I.uniform_tokens(circ, B, cfg["K"], rng)
    elif kind == "pd":
        circ = C.pd(cfg["H"], cfg["W"], cfg["K"], cfg["C"], cfg.get("split", 1))
        out["params"] = I.softmax_rows_params(circ, rng)
        out["tokens"] = I.uniform_tokens(circ, B, cfg["C"], rng)
    elif kind == "block_sparse":
        circ = C.block_sparse(cfg.get("seed", 0), **{k: cfg[k] for k in
                              ("num_vars", "K", "in_blocks", "block", "sum_blocks", "density",
                               "depth_sums") if k in cfg})
        out["params"] = I.softmax_rows_params(circ, rng)
        out["tokens"] = I.uniform_tokens(circ, B, circ.meta["K"], rng)
    elif kind == "block_layer":
        circ = C.random_block_layer(cfg.get("seed", 0), cfg["M_blocks"], cfg["node_block"],
                                    cfg["ch_blocks"], cfg["ch_block"], cfg.get("density", 0.5))
        out["params"] = I.softmax_rows_params(circ, rng)
        out["external"] = I.external_values(circ, B, rng, cfg.get("shift_hi", 300.0),
                                            cfg.get("spread_hi", 50.0))
        outs = circ.output_nodes()
        out["seed_flows"] = I.uniform_flows(len(outs), B, rng)
    else:
        raise ValueError(kind)
    out["circuit"] = circ
    return out
