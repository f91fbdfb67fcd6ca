"""pc_forward_static (the forward that allocates nothing and takes no
workspace) against pc_forward on the same inputs: two calls in a row, the
second with a smaller batch (the static scratch keeps the first call's
content), in both precision modes, on a plain HMM, a block-sparse circuit and
a LowRank HMM; and the host-side rejection of a forward too large for the
static scratch (no device work).  Same kernels, so the results are expected
bit for bit; the comparison also holds them to the stated tolerances."""
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


def _forward_both(h, cfg, B, dev):
    """node values and log-likelihoods of pc_forward (own workspace) and of
    pc_forward_static on the first B samples."""
    import torch
    import log_space_sum_amd as L
    circ = cfg["circuit"]
    params = torch.tensor(cfg["params"], device=dev)
    tokens = torch.tensor(np.ascontiguousarray(cfg["tokens"][:B]), device=dev) if cfg.get("tokens") is not None else None
    lr = None
    if cfg.get("lowrank") is not None:
        lr = [(torch.tensor(np.ascontiguousarray(a[:B]), device=dev),
               torch.tensor(np.ascontiguousarray(b[:B]), device=dev)) for a, b in cfg["lowrank"]]
    out = []
    for static in (False, True):
        vals = torch.full((circ.num_nodes, B), float("nan"), device=dev)
        ll = torch.full((B,), float("nan"), device=dev)
        if static:
            L.pc_forward_static(h, B, tokens, params, vals, ll, lr)
        else:
            ws = L.workspace(h, B, dev)
            L.pc_forward(h, B, tokens, params, vals, ll, lr, ws)
        torch.cuda.synchronize()
        out.append((vals.cpu().numpy(), ll.cpu().numpy()))
    return out


@pytest.mark.parametrize("mode", ["auto", "fp32"])
@pytest.mark.parametrize("what,cfg_args,B1,B2", [
    ("hmm", dict(name="hmm4096", H=320, T=7, V=50, B=300), 300, 70),
    ("block-sparse", dict(kind="block_sparse", seed=2, num_vars=6, K=5, in_blocks=3, block=24,
                          sum_blocks=3, depth_sums=2, B=64), 64, 29),
    ("lowrank hmm", dict(name="lowrank", H=64, T=5, V=16, B=37, rank=16), 37, 20),
])
def test_static_forward_matches_forward(what, cfg_args, B1, B2, mode):
    import log_space_sum_amd as L
    cfg = make_config(**cfg_args)
    h = L.pc_compile_layout(cfg["circuit"], device=0)
    L.pc_set_precision(h, mode)
    for B in (B1, B2):
        G.say(f"case static forward: {what} mode={mode} B={B}")
        (v0, l0), (v1, l1) = _forward_both(h, cfg, B, "cuda:0")
        m = mode if B >= 16 else "fp32"
        G.check_values(v1, v0, m, f"{what} B={B} static vs workspace node values")
        G.check_values(l1, l0, m, f"{what} B={B} static vs workspace log-likelihood")
        np.testing.assert_array_equal(v1, v0, err_msg=f"{what} B={B}: node values differ in bits")
        np.testing.assert_array_equal(l1, l0, err_msg=f"{what} B={B}: log-likelihoods differ in bits")


def test_static_forward_rejects_oversized():
    """A forward whose scratch exceeds the static array is refused on the host
    with PC_ERR_WORKSPACE (nothing is launched); the same handle then still
    runs a forward that fits."""
    import torch
    import log_space_sum_amd as L
    from workloads import circuits as W
    circ = W.dense_layer(8192, 8192, 1)     # two 128 MiB weight planes in auto mode
    h = L.pc_compile_layout(circ, device=0)
    vals = torch.zeros((circ.num_nodes, 16), device="cuda:0")
    params = torch.zeros(circ.num_params, device="cuda:0")
    with pytest.raises(L.PCError) as ei:
        L.pc_forward_static(h, 16, None, params, vals)
    assert ei.value.code == L.PC_ERR_WORKSPACE, str(ei.value)
    G.say(f"  rejected: {ei.value}")
    small = make_config("hmm4096", H=96, T=4, V=11, B=23)
    hs = L.pc_compile_layout(small["circuit"], device=0)
    (v0, l0), (v1, l1) = _forward_both(hs, small, 23, "cuda:0")
    np.testing.assert_array_equal(v1, v0)
    np.testing.assert_array_equal(l1, l0)
