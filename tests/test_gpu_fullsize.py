"""GPU parity at the full sizes of the synthetic workloads, in the launch
configuration bench.py times.

* HMM with 4096 states, 32 positions and 512 symbols (the timed workload), at
  batch 512 in both precision modes and at batch 128 in auto mode: the float64
  oracle runs on the whole batch, so node values, log-likelihoods, element
  flows and parameter flows are compared end to end on every entry, and every
  layer's values, flows and parameter flows against the oracle's step from
  that layer's GPU inputs.
* HCLT-like circuit, 768 variables x 1024 latents x 512 categories, batch 512,
  both modes: values, log-likelihoods and element flows end to end and per
  layer on sampled samples (samples are independent); parameter flows end to
  end over the whole batch (the oracle in chunks of samples, whose parameter
  flows add up) on sampled edge blocks, the root and sampled input rows.
* The LowRank workload (HMM 1024 states, 64 positions, rank 16, batch 64):
  see tests/test_gpu_lowrank.py::test_lowrank_full_size_sampled.
"""
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


@pytest.mark.timeout(600)
@pytest.mark.parametrize("B,mode", [(512, "auto"), (512, "fp32"), (128, "auto")])
def test_hmm4096_full_size(B, mode):
    cfg = make_config("hmm4096", B=B)
    circ = cfg["circuit"]
    G.say(f"case hmm4096x32 full size mode={mode} B={B}")
    gpu = G.run_gpu(cfg, mode)
    G.say("  gpu pass done; oracle on the whole batch")
    orc = G.run_oracle(cfg)
    G.check_values(gpu["vals"], orc["vals"], mode, "full-size node values")
    G.check_values(gpu["ll"], orc["ll"], mode, "full-size log-likelihood")
    tol = G.e2e_flow_tol(circ, orc["vals"], mode)
    G.check_flows(gpu["flows"], orc["flows"], mode, "full-size element flows end to end", rtol=tol)
    G.check_flows(gpu["pflows"], orc["pflows"], mode, "full-size parameter flows end to end", rtol=tol)
    G.say("  per-layer oracle on the whole batch")
    G.check_local(cfg, gpu, mode, "full-size")


# ---------------------------------------------------------------------------
# HCLT at full size
# ---------------------------------------------------------------------------

_HCLT = {}


def _hclt_cfg():
    if "cfg" not in _HCLT:
        G.say("  building the full-size HCLT workload (768 x 1024 x 512, batch 512)")
        _HCLT["cfg"] = make_config("hclt")
    return _HCLT["cfg"]


def _hclt_checked_params(circ):
    """Parameter entries compared end to end: every 16th edge block, the root
    row and the input rows of 8 variables (index arrays into the vector)."""
    meta = circ.meta
    H, K = meta["H"], meta["K"]
    idx = []
    edges = sorted(meta["param_off"].items())
    for v, off in edges[::16]:
        idx.append(np.arange(off, off + H * H, dtype=np.int64))
    idx.append(np.arange(meta["off_root"], meta["off_root"] + H, dtype=np.int64))
    for v in (0, 1, 100, 383, 500, 600, 700, 767):
        idx.append(np.arange(v * H * K, (v + 1) * H * K, dtype=np.int64))
    return np.concatenate(idx)


def _hclt_oracle_pflows(cfg, sel, chunk=128):
    """The oracle's parameter flows over the whole batch, in chunks of
    samples (parameter flows are sums over samples), at the entries `sel`;
    computed once for both modes."""
    if "pflows" not in _HCLT:
        B = cfg["B"]
        acc = np.zeros(len(sel))
        for b0 in range(0, B, chunk):
            G.say(f"  oracle parameter flows: samples {b0}..{min(b0 + chunk, B) - 1}")
            r = G.run_oracle(cfg, samples=np.arange(b0, min(b0 + chunk, B)))
            acc += r["pflows"][sel]
            del r
        _HCLT["pflows"] = acc
    return _HCLT["pflows"]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("mode", ["auto", "fp32"])
def test_hclt_full_size(mode):
    cfg = _hclt_cfg()
    circ = cfg["circuit"]
    B = cfg["B"]
    G.say(f"case hclt 768x1024x512 full size mode={mode} B={B}")
    gpu = G.run_gpu(cfg, mode)
    samples = np.array([0, 137, 300, B - 1])
    G.say("  gpu pass done; oracle on sampled samples")
    orc = G.run_oracle(cfg, samples=samples)
    G.check_values(gpu["vals"][:, samples], orc["vals"], mode, "full-size node values (sampled)")
    G.check_values(gpu["ll"][samples], orc["ll"], mode, "full-size log-likelihood (sampled)")
    tol = G.e2e_flow_tol(circ, orc["vals"], mode)
    G.check_flows(gpu["flows"][:, samples], orc["flows"], mode, "full-size element flows (sampled, e2e)", rtol=tol)
    del orc
    G.say("  per-layer oracle on the sampled samples")
    G.check_local(cfg, gpu, mode, "full-size (sampled)", samples=samples, pflows=False)
    sel = _hclt_checked_params(circ)
    ref = _hclt_oracle_pflows(cfg, sel)
    # the fp32-level storage term of the whole batch is bounded by the sampled
    # samples' one only if those carry the largest |v|; take the GPU's own values
    tol = G.e2e_flow_tol(circ, gpu["vals"], mode)
    G.check_flows(gpu["pflows"][sel], ref, mode, "full-size parameter flows (sampled blocks, e2e, all samples)",
                  rtol=tol)
