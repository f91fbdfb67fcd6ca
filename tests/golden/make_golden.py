"""Write the stored expected values under tests/golden/ from the float64
oracle (the only computation this script runs; inputs come from the seeded
workload generators).  The values are pinned, independently of the oracle,
by tests/test_golden.py: the HMM log-likelihoods and parameter flows by the
textbook scaled forward / forward-backward algorithm, the LowRank ones by
the same algorithms on the per-sample time-inhomogeneous HMM the scaled
layers define.

Usage: python tests/golden/make_golden.py   (rewrites the JSON files)
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from workloads import make_config  # noqa: E402

# The small LowRank HMM of the golden file (rank-4 factor pairs per position).
LOWRANK_SMALL = dict(H=40, T=4, V=6, rank=4, B=16)


def tiny_hmm():
    cfg = make_config("tiny_hmm")
    circ, B = cfg["circuit"], cfg["B"]
    p = cfg["params"].astype(np.float64)
    V, ll = oracle.forward(circ, p, B, tokens=cfg["tokens"])
    r = oracle.backward(circ, p, V, tokens=cfg["tokens"])
    m = circ.meta
    H, Vs = m["H"], m["V"]
    F = r["param_flows"]
    return {
        "what": "tiny HMM workload (64 states, 8 positions, 32 symbols, batch 16, seed 0): per-sample "
                "log-likelihood and parameter flows (expected counts) of the initial, transition and "
                "emission tables, summed over the batch",
        "source": "float64 oracle via tests/golden/make_golden.py",
        "ll": ll.tolist(),
        "flows_init": F[m["off_init"]:m["off_init"] + H].tolist(),
        "flows_trans_rowsum": F[m["off_trans"]:m["off_trans"] + H * H].reshape(H, H).sum(1).tolist(),
        "flows_emit_colsum": F[m["off_emit"]:m["off_emit"] + H * Vs].reshape(H, Vs).sum(0).tolist(),
    }


def lowrank_small():
    cfg = make_config("lowrank", **LOWRANK_SMALL)
    circ, B = cfg["circuit"], cfg["B"]
    p = cfg["params"].astype(np.float64)
    V, ll = oracle.forward(circ, p, B, tokens=cfg["tokens"], lowrank=cfg["lowrank"])
    r = oracle.backward(circ, p, V, tokens=cfg["tokens"], lowrank=cfg["lowrank"])
    m = circ.meta
    H = m["H"]
    F = r["param_flows"]
    return {
        "what": "LowRank exp_sum HMM (40 states, 4 positions, 6 symbols, rank 4, batch 16, seed 4): "
                "per-sample log-likelihood, row sums of the transition parameter flows F+ (summed over "
                "the batch and the 3 scaled layers), and dLL/dA, dLL/dB of slot 0, sample 0",
        "source": "float64 oracle via tests/golden/make_golden.py",
        "config": LOWRANK_SMALL,
        "ll": ll.tolist(),
        "fplus_rowsum": F[m["off_trans"]:m["off_trans"] + H * H].reshape(H, H).sum(1).tolist(),
        "dA_slot0_sample0": r["dA"][0][0].tolist(),
        "dB_slot0_sample0": r["dB"][0][0].tolist(),
    }


def main():
    for name, fn in (("tiny_hmm.json", tiny_hmm), ("lowrank_small.json", lowrank_small)):
        with open(os.path.join(HERE, name), "w") as f:
            json.dump(fn(), f, indent=1)
        print("wrote", name)


if __name__ == "__main__":
    main()
