"""Helpers of the GPU parity tests: run a workload through the C ABI (via the
binding) and through the float64 oracle, and compare them element by element
with the stated tolerances.

Tolerances (the stated accuracy bar of the two precision modes):
  node values / log-likelihood:  fp32-level |x - x*| <= 2e-6 |x*|;  auto (bf16) <= 1e-2 absolute
  element and parameter flows:   fp32-level 1e-5 relative;           auto 5e-3 relative
A relative comparison uses max(|x*|, 1e-6 * max|x*|) as the scale, so exact
zeros and underflowed entries are compared against the array's magnitude.
"""
from __future__ import annotations

import sys

import numpy as np

import log_space_sum_amd as L
import oracle

TOL = {
    "fp32": dict(val_rel=2e-6, val_abs=0.0, flow_rel=1e-5),
    "auto": dict(val_rel=0.0, val_abs=1e-2, flow_rel=5e-3),
}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch():
    import torch as T
    return T


def run_gpu(cfg, mode="auto", splits=None, B=None, em=None, timing=False, device=0, repeat=1, options=None,
            z_init=None, em_corrected=None):
    """Forward + backward (+ optional EM) on the GPU.  Returns numpy arrays
    (with timing: also the per-kind kernel counts and times, key "times").
    z_init: initial contents of the LowRank denominator statistic's buffer
    (key "z_flows" after the pass); em_corrected = (step, pseudocount): the
    conditional M-step from the pass's F+ and W (key "em_corrected")."""
    T = torch()
    circ = cfg["circuit"]
    B = B or cfg["B"]
    dev = f"cuda:{device}"
    h = L.pc_compile_layout(circ, device=device)
    L.pc_set_precision(h, mode)
    for (m, k, pa, pb) in (splits or []):
        L.pc_set_split(h, m, k, pa, pb)
    for (name, value) in (options or []):
        L.pc_set_option(h, name, value)
    if timing:
        L.pc_set_timing(h, True)
    params = T.tensor(cfg["params"], device=dev)
    tokens = T.tensor(cfg["tokens"], device=dev) if cfg.get("tokens") is not None else None
    vals = T.full((circ.num_nodes, B), float("nan"), device=dev)
    ext_rows = _external_rows(circ)
    if cfg.get("external") is not None:
        vals[T.tensor(ext_rows, device=dev)] = T.tensor(cfg["external"], device=dev)
    flows = T.full((circ.num_nodes, B), float("nan"), device=dev)
    flags = 0
    if cfg.get("seed_flows") is not None:
        outs = circ.output_nodes()
        flows[T.tensor(outs, device=dev)] = T.tensor(cfg["seed_flows"], device=dev)
        flags = L.PC_BWD_SEEDED
    pflows = T.zeros(circ.num_params, device=dev)
    ll = T.empty(B, device=dev) if circ.root >= 0 else None
    ws = L.workspace(h, B, dev)
    lr = grads = None
    if cfg.get("lowrank") is not None:
        lr = [(T.tensor(a[:B], device=dev), T.tensor(b[:B], device=dev)) for a, b in cfg["lowrank"]]
        grads = [(T.full_like(a, float("nan")), T.full_like(b, float("nan"))) for a, b in lr]
    zf = T.tensor(np.asarray(z_init, np.float32), device=dev) if z_init is not None else None
    out = []
    for _ in range(repeat):
        pflows.zero_()
        L.pc_forward(h, B, tokens, params, vals, ll, lr, ws)
        L.pc_backward(h, B, tokens, params, vals, flows, pflows, flags, lr, grads, ws, z_flows=zf)
        T.cuda.synchronize()
        r = dict(vals=vals.cpu().numpy().copy(), flows=flows.cpu().numpy().copy(),
                 pflows=pflows.cpu().numpy().copy(), ll=None if ll is None else ll.cpu().numpy().copy())
        if timing:
            r["times"] = L.pc_kernel_times(h)
        if grads is not None:
            r["dA"] = [a.cpu().numpy().copy() for a, _ in grads]
            r["dB"] = [b.cpu().numpy().copy() for _, b in grads]
        if zf is not None:
            r["z_flows"] = zf.cpu().numpy().copy()
        out.append(r)
    if em_corrected is not None:
        newp = params.clone()
        L.pc_em_step_corrected(h, newp, pflows, zf, em_corrected[0], em_corrected[1])
        T.cuda.synchronize()
        out[-1]["em_corrected"] = newp.cpu().numpy()
    if em is not None:
        newp = params.clone()
        L.pc_em_step(h, newp, pflows, em[0], em[1])
        T.cuda.synchronize()
        out[-1]["em"] = newp.cpu().numpy()
    return out if repeat > 1 else out[0]


def _external_rows(circ):
    rows = []
    for l in circ.layers:
        if type(l).__name__ == "InputExternal":
            rows.extend(range(l.node_start, l.node_start + l.num_nodes))
    return np.array(rows, dtype=np.int64)


def run_oracle(cfg, B=None, samples=None):
    circ = cfg["circuit"]
    p = cfg["params"].astype(np.float64)
    tok = cfg.get("tokens")
    ext = cfg.get("external")
    seeds = cfg.get("seed_flows")
    if samples is not None:
        tok = None if tok is None else tok[samples]
        ext = None if ext is None else ext[:, samples]
        seeds = None if seeds is None else seeds[:, samples]
    Bo = (len(samples) if samples is not None else (B or cfg["B"]))
    lr = cfg.get("lowrank")
    if lr is not None:
        sel = samples if samples is not None else slice(0, Bo)
        lr = [(a[sel], b[sel]) for a, b in lr]
    V, ll = oracle.forward(circ, p, Bo, tokens=tok, external=ext, lowrank=lr)
    r = oracle.backward(circ, p, V, tokens=tok, seed_flows=seeds, lowrank=lr)
    out = dict(vals=V, ll=ll, flows=r["flows"], pflows=r["param_flows"])
    if lr is not None:
        out["dA"] = [r["dA"][s] for s in range(len(lr))]
        out["dB"] = [r["dB"][s] for s in range(len(lr))]
        out["z_flows"] = r["z_flows"]
    return out


def rel_err(got, ref, floor=1e-6):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    scale = np.maximum(np.abs(ref), floor * max(np.abs(ref).max(), 1e-300))
    both_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    e = np.where(both_inf, 0.0, np.abs(got - ref) / scale)
    e[np.isnan(got) | np.isnan(ref)] = np.inf
    return e


def check_values(got, ref, mode, what):
    t = TOL[mode]
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    both_inf = np.isinf(got) & np.isinf(ref) & (np.sign(got) == np.sign(ref))
    err = np.where(both_inf, 0.0, np.abs(got - ref))
    err[np.isnan(got) | np.isnan(ref)] = np.inf
    bound = t["val_abs"] + t["val_rel"] * np.where(np.isfinite(ref), np.abs(ref), 0.0)
    bad = err > bound
    worst = float(np.max(err)) if err.size else 0.0
    say(f"  {what}: max abs err {worst:.3e} (mode {mode})")
    assert not bad.any(), f"{what}: {int(bad.sum())} entries out of tolerance, worst {worst:.3e} at {np.argwhere(bad)[0]}"
    return worst


# dLL/dA and dLL/dB of LowRank slots: compared normwise and against the
# largest entry of the magnitude `mag` of the terms the gradient is a
# difference of (dLL/dA_b = X B_b^T with X = eps - f theta_b, the edge flows
# minus the normaliser's part: mag = |eps| |B_b|^T + |f theta_b| |B_b|^T, and
# likewise for dB and for the "sum_exp" form; without mag, |x*| itself):
# the products round each term, so where the two nearly cancel (wide or
# offset factors) the error is relative to the terms, not to the difference:
#   auto (gradient products in one bfloat16 term): ||x - x*|| <= 1e-2 ||mag||
#     and max|x - x*| <= 3e-2 max mag;
#   fp32-level (six-term products): 1e-5 of |x*| itself, normwise and max.
GRAD_TOL = {"fp32": (1e-5, 1e-5), "auto": (1e-2, 3e-2)}


def check_grads(got, ref, mode, what, e2e_tol=None, mag=None):
    """e2e_tol: for gradients compared end to end at fp32 level, the flows'
    end-to-end bound (gpu_util.e2e_flow_tol) replaces 1e-5: the gradients are
    built from the end-to-end flows and carry their float32-storage term."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    if mode != "auto":
        mag = None               # fp32-level: against |x*| itself
    m = np.abs(ref) if mag is None else np.asarray(mag, np.float64)
    scale = max(m.max(), 1e-300)
    en = float(np.linalg.norm(got - ref) / max(np.linalg.norm(m), 1e-300))
    em = float(np.abs(got - ref).max() / scale)
    tn, tm = GRAD_TOL[mode]
    if e2e_tol is not None and mode == "fp32":
        tn = tm = e2e_tol
    say(f"  {what}: normwise {en:.3e}, max/max {em:.3e} of {'|ref|' if mag is None else 'the terms'} "
        f"(mode {mode}, bounds {tn:.3e} {tm:.3e})")
    assert np.isfinite(got).all(), f"{what}: non-finite entries"
    assert en <= tn and em <= tm, f"{what}: normwise {en:.3e} (bound {tn}), max {em:.3e} (bound {tm})"
    return en, em


def num_sum_layers(circ):
    return sum(1 for l in circ.layers if type(l).__name__ == "Sum")


def check_flows(got, ref, mode, what, rtol=None):
    """Per-entry relative error (scale max(|x*|, 1e-6 max|x*|)) within rtol
    (default: the mode's stated flow tolerance)."""
    rtol = TOL[mode]["flow_rel"] if rtol is None else rtol
    e = rel_err(got, ref)
    worst = float(e.max()) if e.size else 0.0
    med = float(np.median(e)) if e.size else 0.0
    say(f"  {what}: max rel err {worst:.3e}, median {med:.3e} (mode {mode}, bound {rtol:.3e})")
    bad = e > rtol
    assert not bad.any(), f"{what}: {int(bad.sum())}/{e.size} entries out of tolerance, worst {worst:.3e}"
    return worst


# End-to-end flows (every layer's rounding compounded from the root down).
# auto: the stated 5e-3.  fp32-level: the stated 1e-5 plus what float32
# storage of the node values costs: every stored log-value v carries an
# absolute rounding of up to |v| 2^-24, and a flow through a sum layer is a
# product of exp(v_child - v_node) terms, so each sum layer adds at most
# 2 max|v| 2^-24 relative (child and node), whatever the products' precision:
#     rtol = 1e-5 + 2^-23 * sum over sum layers l of max |v| over l's nodes.
def sum_layer_value_mass(circ, vals):
    """sum over sum layers of the largest finite |v| of the layer's nodes."""
    tot = 0.0
    for layer in circ.layers:
        if type(layer).__name__ != "Sum":
            continue
        rows = np.concatenate([np.arange(g.out_start, g.out_start + g.num_nodes) for g in layer.groups])
        v = np.asarray(vals[rows], np.float64)
        v = np.abs(v[np.isfinite(v)])
        tot += float(v.max()) if v.size else 0.0
    return tot


def e2e_flow_tol(circ, ref_vals, mode):
    if mode == "auto":
        return TOL["auto"]["flow_rel"]
    return TOL["fp32"]["flow_rel"] + 2.0 ** -23 * sum_layer_value_mass(circ, ref_vals)


def compare(cfg, mode, gpu=None, orc=None, samples=None, what=""):
    """Full comparison of values, flows and parameter flows."""
    gpu = gpu or run_gpu(cfg, mode)
    orc = orc or run_oracle(cfg)
    circ = cfg["circuit"]
    if samples is None:
        check_values(gpu["vals"], orc["vals"], mode, f"{what} node values")
        check_flows(gpu["flows"], orc["flows"], mode, f"{what} element flows")
    else:
        check_values(gpu["vals"][:, samples], orc["vals"], mode, f"{what} node values (sampled)")
        check_flows(gpu["flows"][:, samples], orc["flows"], mode, f"{what} element flows (sampled)")
    return gpu, orc


# ---------------------------------------------------------------------------
# Per-layer ("one layer against float64") oracle: every layer's outputs are
# recomputed by the oracle from the GPU's own inputs to that layer (children
# values, incoming flows), so the comparison measures that layer's kernels
# alone, as the precision pull request measures flows on one HMM layer.
# ---------------------------------------------------------------------------

def _sub_sum_circuit(circ, layer):
    """The sum layer alone over external copies of its distinct children,
    with its own weight blocks packed into a compact parameter vector.
    Returns (sub, kids, outs, blocks) with blocks = [(old_offset,
    new_offset, size)] of the distinct (tied groups: shared) weight blocks."""
    from workloads import circuits as W
    kids = np.unique(np.concatenate([g.child_ids() for g in layer.groups]))
    remap = {int(c): i for i, c in enumerate(kids)}
    n_ext = len(kids)
    groups = []
    nxt = n_ext
    outs = []
    blocks = {}
    pcur = 0
    for g in layer.groups:
        key = int(g.param_offset)
        if key not in blocks:
            size = int(g.num_nodes) * int(g.num_children)
            blocks[key] = (key, pcur, size)
            pcur += size
        starts = np.array([remap[int(s)] for s in g.ch_block_start], dtype=np.int32)
        groups.append(W.SumGroup(nxt, g.num_nodes, starts, g.ch_block_size, blocks[key][1], g.lowrank))
        outs.append(np.arange(g.out_start, g.out_start + g.num_nodes))
        nxt += g.num_nodes
    sub = W.Circuit("sub", nxt, 0, pcur, [W.InputExternal(0, n_ext), W.Sum(groups)],
                    root=-1, lowrank_rank=circ.lowrank_rank, lowrank_form=circ.lowrank_form)
    return sub, kids, np.concatenate(outs), list(blocks.values())


def _sub_params(p, blocks):
    return np.concatenate([p[o:o + n] for o, _, n in blocks]) if blocks else np.zeros(0)


def local_oracle(cfg, gpu, samples=None, own_values=False, want_pflows=True):
    """Expected values, flows and parameter flows, layer by layer, from the
    GPU's own inputs to each step: a sum layer's values are recomputed by the
    oracle from the GPU's children values; its backward step (contributions
    to its children's flows, parameter flows, LowRank gradients) from the
    GPU's children values, the GPU's values of the layer's own nodes and the
    GPU's flows at its outputs -- the inputs of that step; products and
    inputs likewise from theirs.  The layer's own values enter the backward
    step as the exact recomputation (own_values=False: the GPU keeps the scaled
    sums S of the forward and divides by them, so for fp32-level products its
    backward sees S to float32 precision, while its stored float32 node values
    carry an absolute rounding of |v| 2^-24 that it does not use), or as the
    GPU's own stored values (own_values=True: the step given the forward's
    outputs, for bf16 products whose forward error the value check covers).
    want_pflows=False skips the parameter flows (pflows is then None)."""
    from workloads import circuits as W
    circ = cfg["circuit"]
    p = cfg["params"]
    cols = np.arange(gpu["vals"].shape[1]) if samples is None else np.asarray(samples)
    GV = gpu["vals"][:, cols].astype(np.float64)
    GF = gpu["flows"][:, cols].astype(np.float64)
    Bs = len(cols)
    vals = GV.copy()
    flows = np.zeros_like(GF)
    seeds = cfg.get("seed_flows")
    if seeds is not None:
        flows[circ.output_nodes()] = seeds[:, cols]
    else:
        flows[circ.root] = 1.0
    pflows = np.zeros(circ.num_params) if want_pflows else None
    tok = cfg.get("tokens")
    tok = None if tok is None else tok[cols]
    lr = cfg.get("lowrank")
    if lr is not None:
        lr = [(a[cols], b[cols]) for a, b in lr]
    dA, dB, magA, magB = {}, {}, {}, {}
    for layer in circ.layers:
        if isinstance(layer, W.Sum):
            sub, kids, outs, blocks = _sub_sum_circuit(circ, layer)
            ps = _sub_params(p, blocks).astype(np.float64)
            V, _ = oracle.forward(sub, ps, Bs, external=GV[kids], lowrank=lr)
            vals[outs] = V[len(kids):]
            # the backward step of the layer from its GPU inputs: children
            # values, the layer's own output values and its output flows
            Vb = V.copy()
            if own_values:
                Vb[len(kids):] = GV[outs]
            r = oracle.backward(sub, ps, Vb, seed_flows=GF[outs], lowrank=lr)
            flows[kids] += r["flows"][:len(kids)]
            if want_pflows:
                for o, q, n in blocks:
                    pflows[o:o + n] += r["param_flows"][q:q + n]
            dA.update(r["dA"])
            dB.update(r["dB"])
            for g in sub.layers[1].groups:
                if g.lowrank >= 0:
                    ma, mb = _lowrank_grad_terms(sub, ps, Vb, _seed_rows(sub, GF[outs]), g, lr, circ.lowrank_form)
                    magA[g.lowrank], magB[g.lowrank] = ma, mb
        elif isinstance(layer, W.Product):
            ptr = layer.ch_ptr.astype(np.int64)
            ids = layer.ch_ids.astype(np.int64)
            rng_ = slice(layer.node_start, layer.node_start + layer.num_nodes)
            vals[rng_] = np.add.reduceat(GV[ids], ptr[:-1], axis=0)
            par = np.repeat(np.arange(layer.node_start, layer.node_start + layer.num_nodes), np.diff(ptr))
            np.add.at(flows, ids, GF[par])
        elif isinstance(layer, W.InputCat):
            # the layer alone, over its own parameter table
            n = layer.num_nodes
            size = layer.num_rows * layer.num_cats
            sub = W.Circuit("in", n, circ.num_vars, size,
                            [W.InputCat(0, n, layer.num_cats, layer.var, layer.row, 0, layer.num_rows)], root=-1)
            ps = np.asarray(p[layer.param_offset:layer.param_offset + size], np.float64)
            V, _ = oracle.forward(sub, ps, Bs, tokens=tok)
            rng_ = slice(layer.node_start, layer.node_start + n)
            vals[rng_] = V
            if want_pflows:
                r = oracle.backward(sub, ps, V, tokens=tok, seed_flows=GF[rng_])
                pflows[layer.param_offset:layer.param_offset + size] += r["param_flows"]
    return dict(vals=vals, flows=flows, pflows=pflows, dA=dA, dB=dB, magA=magA, magB=magB)


def _seed_rows(sub, seeds):
    """Flows of the sub-circuit with the seeds on its output rows."""
    F = np.zeros((sub.num_nodes, seeds.shape[1]))
    F[sub.output_nodes()] = seeds
    return F


def _lowrank_grad_terms(sub, ps, V, F, g, lowrank, form):
    """Magnitudes of the two terms dLL/dA_b and dLL/dB_b are differences of
    (per sample, from the layer's inputs): with theta_b, edge flows eps and
    the node's flow f as in the oracle's LowRank backward,
      exp_sum: |eps| |B_b|^T + |f theta_b| |B_b|^T  and  |A_b|^T (|eps| + |f theta_b|);
      sum_exp: exp(A_b) (theta (c1 e + c2) exp(B_b)^T), exp(B_b) (exp(A_b)^T theta (c1 e + c2))
    with c1 = f / S, c2 = f / Z.  Returns ([B, M, k], [B, k, N])."""
    import oracle
    th = ps[g.param_offset:g.param_offset + g.num_nodes * g.num_children].reshape(g.num_nodes, g.num_children)
    ch = g.child_ids()
    C = V[ch]
    m = C.max(axis=0)
    m = np.where(np.isfinite(m), m, 0.0)
    E = np.exp(C - m)
    n = V[g.out_start:g.out_start + g.num_nodes]
    f = F[g.out_start:g.out_start + g.num_nodes]
    A, Bf = lowrank[g.lowrank]
    Bn = V.shape[1]
    MA = np.zeros(A.shape)
    MB = np.zeros(Bf.shape)
    for b in range(Bn):
        Ab = np.asarray(A[b], np.float64)
        Bb = np.asarray(Bf[b], np.float64)
        tb, q, Z = oracle.lowrank_effective(th, Ab, Bb, form)
        fi = np.where(np.isfinite(n[:, b]), f[:, b], 0.0)
        S = tb @ E[:, b]
        with np.errstate(divide="ignore", invalid="ignore"):
            c1 = np.where((fi != 0) & (S > 0), fi / S, 0.0)
        eps = tb * E[:, b][None, :] * c1[:, None]
        norm = np.abs(fi)[:, None] * tb
        if form == "exp_sum":
            MA[b] = (np.abs(eps) + norm) @ np.abs(Bb).T
            MB[b] = np.abs(Ab).T @ (np.abs(eps) + norm)
        else:
            with np.errstate(divide="ignore", invalid="ignore"):
                c2 = np.where((fi != 0) & (Z > 0), fi / Z, 0.0)
            Gm = th * (np.abs(c1)[:, None] * E[:, b][None, :] + np.abs(c2)[:, None])
            eA, eB = np.exp(Ab), np.exp(Bb)
            MA[b] = eA * (Gm @ eB.T)
            MB[b] = eB * (eA.T @ Gm)
    return MA, MB


def check_local(cfg, gpu, mode, what, samples=None, pflows=True):
    """Per-layer parity at the stated tolerances (the backward steps of auto
    mode from the GPU's own forward outputs, see local_oracle)."""
    loc = local_oracle(cfg, gpu, samples, own_values=(mode == "auto"), want_pflows=pflows)
    cols = slice(None) if samples is None else np.asarray(samples)
    check_values(gpu["vals"][:, cols], loc["vals"], mode, f"{what} per-layer values")
    check_flows(gpu["flows"][:, cols], loc["flows"], mode, f"{what} per-layer element flows")
    if pflows:
        check_flows(gpu["pflows"], loc["pflows"], mode, f"{what} per-layer parameter flows")
    return loc
