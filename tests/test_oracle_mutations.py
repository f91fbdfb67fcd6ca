"""Each planted mistake in a copy of the oracle must be caught by at least one
pin (the pins are strong enough to tell a plausible slip from the truth).
The mutated copies are built from the oracle's source text on the CPU; the
real oracle is never modified."""
import os
import types

import pytest

from tests import oracle_pins as P

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "pc_oracle.py")

# (name, text to replace, replacement, count of occurrences to replace (0 = all))
MUTATIONS = [
    ("no_column_max_shift", "m = _colmax(C)", "m = np.zeros(C.shape[1])", 0),
    ("no_neg_inf_guard", "return np.where(np.isfinite(m), m, 0.0)", "return m", 0),
    ("max_over_wrong_axis", "m = C.max(axis=0) if", "m = C.max(axis=1).mean() + 0 * C.max(axis=0) if", 0),
    ("transposed_theta_forward", "S = th @ E", "S = th.T @ E", 0),
    ("element_flow_without_e", "F[ch] += E * (th.T @ gm)", "F[ch] += (th.T @ gm)", 0),
    ("element_flow_untransposed", "F[ch] += E * (th.T @ gm)", "F[ch] += E * (th @ gm)", 0),
    ("param_flow_without_theta", "(th * (gm @ E.T))", "(gm @ E.T)", 0),
    ("param_flow_overwrites_ties", "PF[g.param_offset:g.param_offset + th.size] += (th", "PF[g.param_offset:g.param_offset + th.size] = (th", 0),
    ("flow_shift_sign", "f * np.exp(m - n)", "f * np.exp(n - m)", 0),
    ("product_backward_dropped", "np.add.at(F, layer.ch_ids.astype(np.int64), F[parents])", "pass", 0),
    ("input_flow_wrong_category", "np.add.at(PF, idx.reshape(-1)", "np.add.at(PF, (idx + 1).reshape(-1)", 0),
    ("em_not_normalised", "/ tot[ok][:, None]", "/ 1.0", 0),
    ("em_pseudocount_dropped", "(fl[ok] + pseudocount / rlen)", "(fl[ok])", 0),
    ("lowrank_no_z", "q / Z[:, None]", "q", 0),
    ("lowrank_grad_sign", "D = eps - fi[:, None] * tb", "D = eps + fi[:, None] * tb", 0),
    ("lowrank_dB_without_z_term", "dBg[b] = Ab.T @ D", "dBg[b] = Ab.T @ eps", 0),
    ("lowrank_dA_wrong_factor", "dAg[b] = D @ Bb.T", "dAg[b] = D @ Bb.T[::-1]", 0),
    ("zstat_without_z", "fz = np.where((fi != 0) & (Z > 0), fi / Z, 0.0)", "fz = fi", 0),
    ("zstat_without_scale", "zf += fz[:, None] * gb", "zf += fz[:, None] * np.ones_like(th)", 0),
    ("sumexp_scale_as_exp_of_sum", "return np.exp(A_b) @ np.exp(B_b)", "return np.exp(A_b @ B_b)", 0),
    ("sumexp_dA_without_expA", "dAg[b] = eA * (G @ eB.T)", "dAg[b] = (G @ eB.T)", 0),
    ("sumexp_dB_without_expB", "dBg[b] = eB * (eA.T @ G)", "dBg[b] = (eA.T @ G)", 0),
    ("sumexp_grad_through_h", "G = D / gb", "G = D", 0),
    ("zstat_per_copy_overwrite", "ZF[g.param_offset:g.param_offset + th.size] += zf", "ZF[g.param_offset:g.param_offset + th.size] = zf", 0),
    ("em_corrected_not_ratio", "np.where((th > 0) & (w > 0), fp / w, 0.0)", "np.where((th > 0) & (w > 0), fp, 0.0)", 0),
    ("em_corrected_inverted", "np.where((th > 0) & (w > 0), fp / w, 0.0)", "np.where((th > 0) & (w > 0), w / np.maximum(fp, 1e-300), 0.0)", 0),
]


def _mutant(old, new, count):
    src = open(SRC).read()
    assert old in src, f"mutation anchor not found: {old!r}"
    src = src.replace(old, new) if count == 0 else src.replace(old, new, count)
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = SRC
    exec(compile(src, SRC + " (mutant)", "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new,count", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_mutation_is_caught(name, old, new, count):
    mod = _mutant(old, new, count)
    caught = []
    for check in P.ALL_CHECKS:
        try:
            with __import__("numpy").errstate(all="ignore"):
                check(mod)
        except Exception as e:  # noqa: BLE001 - any failure counts as caught
            caught.append((check.__name__, type(e).__name__))
            break
    assert caught, f"mutation {name} passed every pin"
