"""Planted mistakes in the HIP path must fail parity: every mutant library
built by tests/hip_mutants.py (one wrong line each) runs a parity case through
the C ABI, and at least one of the value / flow / parameter-flow checks
against the float64 oracle must reject its results.  The real library passes
the same case (checked first, so a failure here is the mutant's)."""
import numpy as np
import pytest

from tests import gpu_util as G
from tests import hip_mutants as HM
from workloads import make_config

pytestmark = pytest.mark.gpu

# mutation -> (parity case, mode, what it is caught by)
CASES = {
    "fp32_one_term": (dict(name="dense_layer", M=256, N=256, groups=1, B=64), "fp32"),
    "no_column_max_shift": (dict(name="dense_layer", M=200, N=136, groups=1, B=37), "auto"),
    "shift_of_other_samples": (dict(name="dense_layer", M=200, N=136, groups=1, B=37), "auto"),
    "param_flow_without_theta": (dict(name="hmm4096", H=320, T=7, V=50, B=70), "auto"),
    "ties_not_accumulated": (dict(name="hmm4096", H=320, T=7, V=50, B=70), "auto"),
    "no_neg_inf_guard": ("edge", "auto"),
    "strided_group_offset": (dict(name="dense_layer", M=96, N=160, groups=3, B=48), "auto"),
    # square transition blocks (both weight layouts have the same shape)
    "element_flows_untransposed": (dict(name="hmm4096", H=320, T=7, V=50, B=70), "auto"),
    # batch 15 in auto mode must still meet the fp32-level bar
    "small_batch_rule_ignored": (dict(name="dense_layer", M=130, N=70, groups=1, B=15), "auto"),
}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import log_space_sum_amd as L
    L.lib()


def _cfg(spec):
    if spec == "edge":
        cfg = make_config("dense_layer", M=70, N=90, groups=2, B=20)
        ext = cfg["external"]
        ext[:90, 0] = -np.inf          # an all -inf column of the first group
        ext[:, 1] = -np.inf
        ext[7, 1] = -2.0
        return cfg
    return make_config(**spec)


def _failures(cfg, mode, gpu, orc):
    """The checks (values, log-likelihood, flows, parameter flows end to end at
    the stated bar; fp32-level for batches below 16) that reject `gpu`."""
    m = "fp32" if cfg["B"] < 16 else mode
    tol = G.e2e_flow_tol(cfg["circuit"], orc["vals"], m)
    checks = [("values", lambda: G.check_values(gpu["vals"], orc["vals"], m, "values")),
              ("flows", lambda: G.check_flows(gpu["flows"], orc["flows"], m, "flows", rtol=tol)),
              ("parameter flows", lambda: G.check_flows(gpu["pflows"], orc["pflows"], m, "parameter flows", rtol=tol))]
    if orc["ll"] is not None:
        checks.append(("log-likelihood", lambda: G.check_values(gpu["ll"], orc["ll"], m, "log-likelihood")))
    bad = []
    for what, fn in checks:
        try:
            with np.errstate(invalid="ignore", over="ignore"):
                fn()
        except AssertionError:
            bad.append(what)
    return bad


@pytest.mark.parametrize("name", list(HM.MUTATIONS))
def test_mutant_is_caught(name):
    import log_space_sum_amd as L
    spec, mode = CASES[name]
    cfg = _cfg(spec)
    G.say(f"case mutation {name}: mode={mode} B={cfg['B']}")
    orc = G.run_oracle(cfg)
    good = G.run_gpu(cfg, mode)
    assert _failures(cfg, mode, good, orc) == [], "the real library fails this case"
    with L.using_library(HM.library_path(name)):
        bad = G.run_gpu(cfg, mode)
    caught = _failures(cfg, mode, bad, orc)
    G.say(f"  mutation {name} caught by: {', '.join(caught) or 'nothing'}")
    assert caught, f"mutation {name} passed every parity check"
