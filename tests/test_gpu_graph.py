"""A pass recorded as a HIP graph (log_space_sum_amd.StepGraph) replays the
eager pass bit for bit: node values, log-likelihoods, flows, parameter flows,
LowRank gradients and the EM-updated parameters, at every replay, with the
program's own eager passes and synchronizations between replays; after a
precision-mode change the graph is recorded again and matches the eager pass
in the new mode."""
import numpy as np
import pytest

from tests import gpu_util as G
from workloads import make_config

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import log_space_sum_amd as L
    L.lib()


def _buffers(cfg, dev):
    import torch as T
    circ, B = cfg["circuit"], cfg["B"]
    params = T.tensor(cfg["params"], device=dev)
    tokens = T.tensor(cfg["tokens"], device=dev) if cfg.get("tokens") is not None else None
    vals = T.full((circ.num_nodes, B), float("nan"), device=dev)
    flows = T.full((circ.num_nodes, B), float("nan"), device=dev)
    pflows = T.zeros(circ.num_params, device=dev)
    ll = T.empty(B, device=dev) if circ.root >= 0 else None
    lr = grads = None
    if cfg.get("lowrank") is not None:
        lr = [(T.tensor(a[:B], device=dev), T.tensor(b[:B], device=dev)) for a, b in cfg["lowrank"]]
        grads = [(T.full_like(a, float("nan")), T.full_like(b, float("nan"))) for a, b in lr]
    return dict(params=params, tokens=tokens, vals=vals, flows=flows, pflows=pflows, ll=ll, lr=lr, grads=grads)


def _same(a, b, what):
    import torch as T
    T.cuda.synchronize()
    for k in ("params", "vals", "flows", "pflows", "ll"):
        if a[k] is not None:
            np.testing.assert_array_equal(a[k].cpu().numpy(), b[k].cpu().numpy(), err_msg=f"{what}: {k}")
    for x, y in zip(a["grads"] or [], b["grads"] or []):
        for u, v in zip(x, y):
            np.testing.assert_array_equal(u.cpu().numpy(), v.cpu().numpy(), err_msg=f"{what}: LowRank gradient")


@pytest.mark.parametrize("what,cfg_args,mode", [
    ("hmm batch 256 (fused epilogues)", dict(name="hmm4096", H=128, T=5, V=20, B=256), "auto"),
    ("hmm ragged batch", dict(name="hmm4096", H=96, T=4, V=11, B=23), "fp32"),
    ("hclt", dict(name="hclt", num_vars=30, H=48, K=12, B=33), "auto"),
    ("lowrank hmm", dict(name="lowrank", H=40, T=4, V=7, B=23, rank=5), "auto"),
])
def test_graph_replays_match_eager(what, cfg_args, mode):
    import torch as T
    import log_space_sum_amd as L
    cfg = make_config(**cfg_args)
    B, dev = cfg["B"], "cuda:0"
    G.say(f"case graph replay: {what} mode={mode} B={B}")
    h = L.pc_compile_layout(cfg["circuit"], device=0)
    L.pc_set_precision(h, mode)
    eg, gr = _buffers(cfg, dev), _buffers(cfg, dev)
    ws = L.workspace(h, B, dev, all_modes=True)
    em = (0.5, 0.01)

    def eager():
        eg["pflows"].zero_()
        L.pc_forward(h, B, eg["tokens"], eg["params"], eg["vals"], eg["ll"], eg["lr"], ws)
        L.pc_backward(h, B, eg["tokens"], eg["params"], eg["vals"], eg["flows"], eg["pflows"], 0,
                      eg["lr"], eg["grads"], ws)
        L.pc_em_step(h, eg["params"], eg["pflows"], em[0], em[1])

    g = L.StepGraph(h, B, gr["tokens"], gr["params"], gr["vals"], gr["flows"], gr["pflows"], gr["ll"],
                    lowrank=gr["lr"], grads=gr["grads"], em=em)
    for r in range(3):
        g.replay()
        eager()
        T.cuda.synchronize()
        _same(gr, eg, f"{what}, replay {r}")
    G.say(f"  3 replays identical to the eager passes ({mode})")
    other = "fp32" if mode == "auto" else "auto"
    L.pc_set_precision(h, other)
    for r in range(2):
        g.replay()
        eager()
        T.cuda.synchronize()
        _same(gr, eg, f"{what}, {other} replay {r}")
    G.say(f"  recorded again after the mode change: 2 replays identical ({other})")
