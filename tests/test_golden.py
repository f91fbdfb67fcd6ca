"""Stored expected values (tests/golden/*.json, written from the float64
oracle by tests/golden/make_golden.py).

CPU: each stored value is pinned independently of the oracle -- the tiny-HMM
log-likelihoods and expected counts by the textbook scaled forward-backward
algorithm, the LowRank ones by the forward algorithm on the per-sample
time-inhomogeneous HMM whose step-t transition is normalize(A * exp(A_b B_b))
(LowRank page, definition) -- and the oracle must still reproduce the file.
GPU: the HIP path (fp32-level mode) against the stored values at the
fp32-level tolerances (2e-6 relative for log-likelihoods, 1e-5 relative per
layer for flows, times the number of sum layers end to end; dLL/dA, dLL/dB
1e-5 normwise)."""
import json
import os

import numpy as np
import pytest

import oracle
from tests import oracle_pins as P
from workloads import make_config

HERE = os.path.dirname(os.path.abspath(__file__))
LOWRANK_SMALL = dict(H=40, T=4, V=6, rank=4, B=16)


def _load(name):
    with open(os.path.join(HERE, "golden", name)) as f:
        return json.load(f)


def _tiny_hmm_from_oracle():
    cfg = make_config("tiny_hmm")
    circ, B = cfg["circuit"], cfg["B"]
    p = cfg["params"].astype(np.float64)
    V, ll = oracle.forward(circ, p, B, tokens=cfg["tokens"])
    r = oracle.backward(circ, p, V, tokens=cfg["tokens"])
    return cfg, ll, r


def test_golden_tiny_hmm_pinned():
    g = _load("tiny_hmm.json")
    cfg = make_config("tiny_hmm")
    circ = cfg["circuit"]
    p = cfg["params"].astype(np.float64)
    A, pi, E = P._hmm_tables(circ, p)
    H = len(pi)
    ll, g0, xi, em = [], np.zeros(H), np.zeros((H, H)), np.zeros(E.shape[1])
    for x in cfg["tokens"]:
        l, gamma, xis = P._forward_backward(A, pi, E, x)
        ll.append(l)
        g0 += gamma[0]
        xi += xis
        for t, sym in enumerate(x):
            em[sym] += gamma[t].sum()
    np.testing.assert_allclose(g["ll"], ll, rtol=1e-12, atol=1e-11)
    np.testing.assert_allclose(g["flows_init"], g0, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["flows_trans_rowsum"], xi.sum(1), rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(g["flows_emit_colsum"], em, rtol=1e-10, atol=1e-12)


def test_golden_tiny_hmm_oracle_reproduces():
    g = _load("tiny_hmm.json")
    cfg, ll, r = _tiny_hmm_from_oracle()
    m = cfg["circuit"].meta
    np.testing.assert_allclose(ll, g["ll"], rtol=1e-13, atol=0)
    np.testing.assert_allclose(r["param_flows"][m["off_init"]:m["off_init"] + m["H"]], g["flows_init"], rtol=1e-12)


def test_golden_lowrank_pinned():
    g = _load("lowrank_small.json")
    cfg = make_config("lowrank", **LOWRANK_SMALL)
    circ, x = cfg["circuit"], cfg["tokens"]
    p = cfg["params"].astype(np.float64)
    fac = [(a.astype(np.float64), b.astype(np.float64)) for a, b in cfg["lowrank"]]
    m = circ.meta
    H, T = m["H"], m["T"]
    A, pi, E = P._hmm_tables(circ, p)
    xi_tot = np.zeros((H, H))
    ll = []
    for b in range(x.shape[0]):
        At = []
        for t in range(T - 1):   # the step from position t to t+1 uses the scaled layer of slot t
            q = A * np.exp(fac[t][0][b] @ fac[t][1][b])
            At.append(q / q.sum(1, keepdims=True))
        alpha = pi * E[:, x[b, 0]]
        al = [alpha]
        for t in range(1, T):
            alpha = (alpha @ At[t - 1]) * E[:, x[b, t]]
            al.append(alpha)
        Pb = alpha.sum()
        ll.append(np.log(Pb))
        beta = np.ones(H)
        for t in range(T - 2, -1, -1):
            xi_tot += al[t][:, None] * At[t] * (E[:, x[b, t + 1]] * beta)[None, :] / Pb
            beta = At[t] @ (E[:, x[b, t + 1]] * beta)
    np.testing.assert_allclose(g["ll"], ll, rtol=1e-12, atol=1e-11)
    np.testing.assert_allclose(g["fplus_rowsum"], xi_tot.sum(1), rtol=1e-10, atol=1e-12)


def test_golden_lowrank_oracle_reproduces():
    g = _load("lowrank_small.json")
    cfg = make_config("lowrank", **LOWRANK_SMALL)
    circ, B = cfg["circuit"], cfg["B"]
    p = cfg["params"].astype(np.float64)
    V, ll = oracle.forward(circ, p, B, tokens=cfg["tokens"], lowrank=cfg["lowrank"])
    r = oracle.backward(circ, p, V, tokens=cfg["tokens"], lowrank=cfg["lowrank"])
    np.testing.assert_allclose(ll, g["ll"], rtol=1e-13, atol=0)
    np.testing.assert_allclose(r["dA"][0][0], g["dA_slot0_sample0"], rtol=1e-12, atol=1e-15)
    np.testing.assert_allclose(r["dB"][0][0], g["dB_slot0_sample0"], rtol=1e-12, atol=1e-15)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.max(np.abs(a - b) / np.maximum(np.abs(b), 1e-6 * np.abs(b).max())))


@pytest.mark.gpu
def test_golden_tiny_hmm_gpu():
    from tests import gpu_util as G
    g = _load("tiny_hmm.json")
    cfg = make_config("tiny_hmm")
    gpu = G.run_gpu(cfg, "fp32")
    m = cfg["circuit"].meta
    H, V = m["H"], m["V"]
    F = gpu["pflows"].astype(np.float64)
    depth = G.num_sum_layers(cfg["circuit"])
    assert np.all(np.abs(gpu["ll"] - np.array(g["ll"])) <= 2e-6 * np.abs(g["ll"]))
    assert _rel(F[m["off_init"]:m["off_init"] + H], g["flows_init"]) <= 1e-5 * depth
    assert _rel(F[m["off_trans"]:m["off_trans"] + H * H].reshape(H, H).sum(1), g["flows_trans_rowsum"]) <= 1e-5 * depth
    assert _rel(F[m["off_emit"]:m["off_emit"] + H * V].reshape(H, V).sum(0), g["flows_emit_colsum"]) <= 1e-5 * depth


@pytest.mark.gpu
def test_golden_lowrank_gpu():
    from tests import gpu_util as G
    g = _load("lowrank_small.json")
    cfg = make_config("lowrank", **LOWRANK_SMALL)
    gpu = G.run_gpu(cfg, "fp32")
    m = cfg["circuit"].meta
    H = m["H"]
    depth = G.num_sum_layers(cfg["circuit"])
    assert np.all(np.abs(gpu["ll"] - np.array(g["ll"])) <= 2e-6 * np.abs(g["ll"]))
    F = gpu["pflows"].astype(np.float64)
    assert _rel(F[m["off_trans"]:m["off_trans"] + H * H].reshape(H, H).sum(1), g["fplus_rowsum"]) <= 1e-5 * depth
    for got, ref in ((gpu["dA"][0][0], g["dA_slot0_sample0"]), (gpu["dB"][0][0], g["dB_slot0_sample0"])):
        ref = np.asarray(ref)
        assert np.linalg.norm(got - ref) <= 1e-5 * np.linalg.norm(ref)
