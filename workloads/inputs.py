"""Seeded synthetic inputs for the circuits in ``workloads.circuits``.

Every generator takes a ``numpy.random.Generator`` (``default_rng(seed)``),
draws in float64 and returns float32 / int32 arrays: both the float64 oracle
(after promotion) and the HIP path consume exactly these values.
"""
from __future__ import annotations

import numpy as np

from .circuits import Circuit, InputExternal


def softmax_rows_params(circ: Circuit, rng: np.random.Generator, scale: float = 1.0) -> np.ndarray:
    """Every parameter row = softmax of i.i.d. N(0, scale^2) logits (float32)."""
    p = np.zeros(circ.num_params, dtype=np.float64)
    for off, nrows, rlen in circ.param_row_segments():
        z = rng.standard_normal((nrows, rlen)) * scale
        z -= z.max(axis=1, keepdims=True)
        e = np.exp(z)
        p[off:off + nrows * rlen] = (e / e.sum(axis=1, keepdims=True)).reshape(-1)
    return p.astype(np.float32)


def uniform_tokens(circ: Circuit, B: int, num_cats: int, rng: np.random.Generator) -> np.ndarray:
    """Tokens [B, num_vars] int32, uniform over [0, num_cats)."""
    return rng.integers(0, num_cats, size=(B, circ.num_vars)).astype(np.int32)


def skewed_tokens(circ: Circuit, B: int, num_cats: int, frac: float, rng: np.random.Generator) -> np.ndarray:
    """Tokens [B, num_vars] int32: uniform over [0, num_cats), then each entry
    replaced by the last category with probability ``frac`` (one large bucket
    per variable beside small ones)."""
    tok = rng.integers(0, num_cats, size=(B, circ.num_vars))
    tok[rng.random(tok.shape) < frac] = num_cats - 1
    return tok.astype(np.int32)


def external_values(circ: Circuit, B: int, rng: np.random.Generator,
                    shift_hi: float = 300.0, spread_hi: float = 50.0) -> np.ndarray:
    """Values for every InputExternal layer, stacked in layer order: a
    per-sample shift -U(0, shift_hi) plus a per-entry -U(0, spread_hi)
    (the dense single-layer workload).  Returns float32 [n_ext, B]."""
    n = sum(l.num_nodes for l in circ.layers if isinstance(l, InputExternal))
    shift = -rng.uniform(0.0, shift_hi, size=(1, B))
    spread = -rng.uniform(0.0, spread_hi, size=(n, B))
    return (shift + spread).astype(np.float32)


def uniform_flows(num: int, B: int, rng: np.random.Generator) -> np.ndarray:
    """Incoming element flows U(0, 1), float32 [num, B]."""
    return rng.uniform(0.0, 1.0, size=(num, B)).astype(np.float32)


def lowrank_factors(circ: Circuit, B: int, sigma: float, rng: np.random.Generator):
    """Per LowRank slot s: A_s [B, M, k] and B_s [B, k, N], i.i.d. N(0, sigma^2),
    float32.  Returns a list indexed by slot."""
    k = circ.lowrank_rank
    out = []
    for slot, M, N in circ.lowrank_slots():
        assert slot == len(out)
        A = (rng.standard_normal((B, M, k)) * sigma).astype(np.float32)
        Bf = (rng.standard_normal((B, k, N)) * sigma).astype(np.float32)
        out.append((A, Bf))
    return out


def lowrank_sigma_for_spread(spread_nats: float, rank: int) -> float:
    """sigma such that the standard deviation of (A B)[i, j] = sqrt(k)*sigma^2
    equals ``spread_nats``."""
    return float(np.sqrt(spread_nats / np.sqrt(rank)))
