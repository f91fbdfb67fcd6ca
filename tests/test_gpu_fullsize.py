"""GPU parity at the full size of the timed workload: the HMM with 4096
states, 32 positions and 512 symbols in auto mode, at batch 512 (the launch
configuration bench.py times) and batch 128.  The oracle computes sampled
outputs one by one: node values, log-likelihood and element flows of three
samples end to end (samples are independent), every layer's values and flows
on those samples from the GPU's inputs to the layer, and the tied transition
matrix's parameter flows on sampled rows, over all samples and copies, in
float64 from the GPU's values and flows; plus the row-sum identity of the
parameter flows (sum_j F[i, j] = sum over copies and samples of f[i])."""
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


def _transition_rows(cfg, gpu, rows):
    """F[i, j] = theta[i, j] * sum over positions t and samples b of
    f[s_t(i), b] exp(v[child_j, b] - v[s_t(i), b]) for the given rows i, from
    the GPU's (float32) values and flows, in float64."""
    circ = cfg["circuit"]
    H = circ.meta["H"]
    th = cfg["params"][:H * H].reshape(H, H).astype(np.float64)
    V = gpu["vals"]
    Fl = gpu["flows"]
    F = np.zeros((len(rows), H))
    for ly in circ.layers:
        if type(ly).__name__ != "Sum" or ly.groups[0].param_offset != circ.meta["off_trans"]:
            continue
        g = ly.groups[0]
        ch = g.child_ids()
        vc = V[ch].astype(np.float64)                      # [H, B]
        for k, i in enumerate(rows):
            vi = V[g.out_start + i].astype(np.float64)
            fi = Fl[g.out_start + i].astype(np.float64)
            w = np.where((fi != 0) & np.isfinite(vi), fi, 0.0)
            with np.errstate(over="ignore", invalid="ignore"):
                F[k] += (np.exp(vc - np.where(np.isfinite(vi), vi, 0.0)[None, :]) * w[None, :]).sum(axis=1)
    return th[rows] * F


@pytest.mark.parametrize("B", [512, 128])
def test_hmm4096_full_size(B):
    cfg = make_config("hmm4096", B=B)
    mode = "auto"
    G.say(f"case hmm4096x32 full size mode={mode} B={B}")
    gpu = G.run_gpu(cfg, mode)
    samples = np.array([0, B // 2 + 1, B - 1])
    orc = G.run_oracle(cfg, samples=samples)
    G.check_values(gpu["vals"][:, samples], orc["vals"], mode, "full-size node values (sampled)")
    G.check_values(gpu["ll"][samples], orc["ll"], mode, "full-size log-likelihood (sampled)")
    depth = G.num_sum_layers(cfg["circuit"])
    G.check_flows(gpu["flows"][:, samples], orc["flows"], mode, "full-size element flows (sampled, e2e)", scale=depth)
    G.check_local(cfg, gpu, mode, "full-size", samples=samples, pflows=False)
    H = cfg["circuit"].meta["H"]
    rows = [0, 1777, H - 1]
    ref = _transition_rows(cfg, gpu, rows)
    got = gpu["pflows"][:H * H].reshape(H, H)[rows]
    G.check_flows(got, ref, mode, "full-size transition parameter flows (sampled rows, all samples)")
    # row sums: sum_j F[i, j] = sum over copies and samples of the flow of s_t(i)
    circ = cfg["circuit"]
    fsum = np.zeros(H)
    for ly in circ.layers:
        if type(ly).__name__ == "Sum" and ly.groups[0].param_offset == circ.meta["off_trans"]:
            g = ly.groups[0]
            fsum += gpu["flows"][g.out_start:g.out_start + H].astype(np.float64).sum(axis=1)
    rs = gpu["pflows"][:H * H].reshape(H, H).astype(np.float64).sum(axis=1)
    G.check_flows(rs, fsum, mode, "full-size transition parameter-flow row sums vs node flows")
