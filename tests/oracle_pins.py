"""Pins for the float64 oracle: checks against things other than the oracle
itself (library closed forms, brute-force enumeration, textbook HMM and tree
algorithms, finite differences, invariants).

Every check takes the oracle module as its argument so that the mutation test
can run the same checks against deliberately broken copies of the oracle.
Each check raises AssertionError (or any exception) on failure.
"""
from __future__ import annotations

import itertools

import numpy as np
from scipy.special import logsumexp

from workloads import circuits as C
from workloads import inputs as I
from workloads import make_config

F64 = np.float64


def _renorm(circ, p):
    """Rows renormalised in float64 (the float32 inputs sum to one only to
    about 1e-7), so that sum-to-one checks can be exact to 1e-12."""
    p = np.array(p, dtype=F64)
    for off, nr, rl in circ.param_row_segments():
        blk = p[off:off + nr * rl].reshape(nr, rl)
        p[off:off + nr * rl] = (blk / blk.sum(1, keepdims=True)).reshape(-1)
    return p


def _close(a, b, rtol, atol, what):
    a = np.asarray(a, F64)
    b = np.asarray(b, F64)
    assert a.shape == b.shape, (what, a.shape, b.shape)
    same_inf = (np.isinf(a) & np.isinf(b) & (np.sign(a) == np.sign(b)))
    with np.errstate(invalid="ignore"):
        ok = same_inf | (np.abs(a - b) <= atol + rtol * np.abs(b))
    assert not np.isnan(a).any(), f"{what}: NaN"
    if not ok.all():
        i = np.argwhere(~ok)[0]
        raise AssertionError(f"{what}: mismatch at {tuple(i)}: {a[tuple(i)]} vs {b[tuple(i)]}")


# ---------------------------------------------------------------------------
# Dense sum layer: closed form and finite differences
# ---------------------------------------------------------------------------

def check_dense_logsumexp(orc):
    """Sum layer = logsumexp(log theta[i,:] + c[:,b]) (scipy), including the
    per-group column-maximum edge cases: a column of -inf children, a column
    with a single finite child, a column shifted by -1e4 nats, a column far
    above the others."""
    for groups in (1, 3):
        cfg = make_config(kind="dense", M=37, N=53, groups=groups, B=9, seed=11)
        circ = cfg["circuit"]
        M, N, B = 37, 53, 9
        p = cfg["params"].astype(F64)
        p[3] = 0.0                                   # a zero weight
        ext = cfg["external"].astype(F64)
        ext[:N, 0] = -np.inf
        ext[:N, 1] = -np.inf
        ext[5, 1] = -3.0
        ext[:, 2] -= 1e4
        ext[:, 3] += 700.0
        V, _ = orc.forward(circ, p, B, external=ext)
        for g in range(groups):
            th = p[g * M * N:(g + 1) * M * N].reshape(M, N)
            c = ext[g * N:(g + 1) * N]
            with np.errstate(divide="ignore"):
                lt = np.log(th)
            expect = logsumexp(lt[:, :, None] + c[None, :, :], axis=1)
            got = V[groups * N + g * M: groups * N + (g + 1) * M]
            _close(got, expect, 1e-13, 1e-12, f"dense group {g}")


def _fd(fun, x, idx, h):
    xp = x.copy()
    xm = x.copy()
    xp[idx] += h
    xm[idx] -= h
    return (fun(xp) - fun(xm)) / (2 * h)


def check_dense_flows_fd(orc):
    """Element flows of the children = dJ/dc and parameter flows =
    theta * dJ/dtheta for J = sum of seed flows times output values
    (central finite differences)."""
    cfg = make_config(kind="dense", M=5, N=7, groups=2, B=3, seed=5)
    circ = cfg["circuit"]
    B = 3
    p = cfg["params"].astype(F64)
    ext = cfg["external"].astype(F64) * 0.05
    seeds = cfg["seed_flows"].astype(F64)
    outs = circ.output_nodes()

    def J_of(pp, ee):
        V, _ = orc.forward(circ, pp, B, external=ee)
        return float((seeds * V[outs]).sum())

    V, _ = orc.forward(circ, p, B, external=ext)
    r = orc.backward(circ, p, V, seed_flows=seeds)
    for idx in [(0, 0), (3, 1), (6, 2), (9, 0), (13, 2)]:
        d = _fd(lambda e: J_of(p, e), ext, idx, 1e-5)
        _close(r["flows"][idx], d, 1e-6, 1e-9, f"dense element flow {idx}")
    for k in [0, 4, 17, 34, 35, 50, 69]:
        d = _fd(lambda q: J_of(q, ext), p, k, 1e-6)
        _close(r["param_flows"][k], p[k] * d, 1e-6, 1e-9, f"dense param flow {k}")


# ---------------------------------------------------------------------------
# HMM: brute force, forward algorithm, forward-backward, Baum-Welch
# ---------------------------------------------------------------------------

def _hmm_tables(circ, p):
    m = circ.meta
    H, V = m["H"], m["V"]
    A = p[m["off_trans"]:m["off_trans"] + H * H].reshape(H, H)
    pi = p[m["off_init"]:m["off_init"] + H]
    E = p[m["off_emit"]:m["off_emit"] + H * V].reshape(H, V)
    return A, pi, E


def check_hmm_bruteforce(orc):
    """LL of every sequence = log of the sum over all hidden paths, and the
    probabilities of all sequences sum to one (H=3, T=4, V=3)."""
    H, T, V = 3, 4, 3
    circ = C.hmm(H, T, V)
    p = _renorm(circ, I.softmax_rows_params(circ, np.random.default_rng(7)))
    A, pi, E = _hmm_tables(circ, p)
    xs = np.array(list(itertools.product(range(V), repeat=T)), dtype=np.int32)
    _, ll = orc.forward(circ, p, len(xs), tokens=xs)
    expect = []
    for x in xs:
        tot = 0.0
        for z in itertools.product(range(H), repeat=T):
            pr = pi[z[0]] * E[z[0], x[0]]
            for t in range(1, T):
                pr *= A[z[t - 1], z[t]] * E[z[t], x[t]]
            tot += pr
        expect.append(np.log(tot))
    _close(ll, expect, 1e-12, 1e-12, "hmm brute force")
    assert abs(np.exp(ll).sum() - 1.0) < 1e-12


def _forward_backward(A, pi, E, x):
    """Scaled forward-backward for one sequence: (loglik, gamma [T,H], xi_sum [H,H])."""
    T = len(x)
    H = len(pi)
    alpha = np.zeros((T, H))
    c = np.zeros(T)
    a = pi * E[:, x[0]]
    c[0] = a.sum()
    alpha[0] = a / c[0]
    for t in range(1, T):
        a = (alpha[t - 1] @ A) * E[:, x[t]]
        c[t] = a.sum()
        alpha[t] = a / c[t]
    beta = np.zeros((T, H))
    beta[T - 1] = 1.0
    for t in range(T - 2, -1, -1):
        beta[t] = (A @ (E[:, x[t + 1]] * beta[t + 1])) / c[t + 1]
    gamma = alpha * beta
    xi = np.zeros((H, H))
    for t in range(T - 1):
        xi += alpha[t][:, None] * A * (E[:, x[t + 1]] * beta[t + 1])[None, :] / c[t + 1]
    return np.log(c).sum(), gamma, xi


def check_hmm_forward_algorithm(orc):
    """LL of the tiny-HMM workload = textbook scaled forward algorithm."""
    cfg = make_config("tiny_hmm")
    circ, B = cfg["circuit"], cfg["B"]
    p = cfg["params"].astype(F64)
    A, pi, E = _hmm_tables(circ, p)
    _, ll = orc.forward(circ, p, B, tokens=cfg["tokens"])
    expect = [_forward_backward(A, pi, E, x)[0] for x in cfg["tokens"]]
    _close(ll, expect, 1e-12, 1e-11, "hmm forward algorithm")


def check_hmm_posteriors(orc):
    """Element flows = posterior state marginals gamma_t; transition parameter
    flows = summed xi; emission flows = summed gamma by symbol; initial flows =
    summed gamma_0 (forward-backward)."""
    cfg = make_config("tiny_hmm", H=6, T=5, V=4, B=7, seed=3)
    circ, B = cfg["circuit"], cfg["B"]
    m = circ.meta
    H, T, V = m["H"], m["T"], m["V"]
    p = cfg["params"].astype(F64)
    A, pi, E = _hmm_tables(circ, p)
    x = cfg["tokens"]
    Vv, _ = orc.forward(circ, p, B, tokens=x)
    r = orc.backward(circ, p, Vv, tokens=x)
    Fl, PF = r["flows"], r["param_flows"]
    xi_tot = np.zeros((H, H))
    em_tot = np.zeros((H, V))
    init_tot = np.zeros(H)
    for b in range(B):
        _, gamma, xi = _forward_backward(A, pi, E, x[b])
        xi_tot += xi
        init_tot += gamma[0]
        for t in range(T):
            em_tot[:, x[b, t]] += gamma[t]
            _close(Fl[t * H:(t + 1) * H, b], gamma[t], 1e-10, 1e-12, f"input flow t={t}")
            if t < T - 1:
                ps = m["prod_starts"][t]
                ss = m["sum_starts"][t]
                _close(Fl[ps:ps + H, b], gamma[t], 1e-10, 1e-12, f"product flow t={t}")
                _close(Fl[ss:ss + H, b], gamma[t], 1e-10, 1e-12, f"sum flow t={t}")
    _close(PF[m["off_trans"]:m["off_trans"] + H * H].reshape(H, H), xi_tot, 1e-10, 1e-12, "transition flows")
    _close(PF[m["off_emit"]:m["off_emit"] + H * V].reshape(H, V), em_tot, 1e-10, 1e-12, "emission flows")
    _close(PF[m["off_init"]:m["off_init"] + H], init_tot, 1e-10, 1e-12, "initial flows")


def check_baum_welch(orc):
    """EM on flows = Baum-Welch M-step; full-batch EM never lowers the LL."""
    cfg = make_config("tiny_hmm", H=5, T=6, V=4, B=9, seed=4)
    circ, B = cfg["circuit"], cfg["B"]
    m = circ.meta
    H, T, V = m["H"], m["T"], m["V"]
    x = cfg["tokens"]
    p = cfg["params"].astype(F64)
    prev = -np.inf
    for it in range(4):
        A, pi, E = _hmm_tables(circ, p)
        xi_tot = np.zeros((H, H))
        em_tot = np.zeros((H, V))
        init_tot = np.zeros(H)
        for b in range(B):
            _, gamma, xi = _forward_backward(A, pi, E, x[b])
            xi_tot += xi
            init_tot += gamma[0]
            for t in range(T):
                em_tot[:, x[b, t]] += gamma[t]
        Vv, ll = orc.forward(circ, p, B, tokens=x)
        assert ll.sum() >= prev - 1e-9, "EM lowered the log-likelihood"
        prev = ll.sum()
        r = orc.backward(circ, p, Vv, tokens=x)
        newp = orc.em_step(circ, p, r["param_flows"])
        A2, pi2, E2 = _hmm_tables(circ, newp)
        _close(A2, xi_tot / xi_tot.sum(1, keepdims=True), 1e-10, 1e-12, "BW transition")
        _close(E2, em_tot / em_tot.sum(1, keepdims=True), 1e-10, 1e-12, "BW emission")
        _close(pi2, init_tot / init_tot.sum(), 1e-10, 1e-12, "BW initial")
        p = newp


def check_em_blend_and_pseudocount(orc):
    """EM with step size eta and pseudocount alpha on a hand-computed row."""
    circ = C.dense_layer(2, 3, 1)
    p = np.array([0.2, 0.3, 0.5, 0.1, 0.1, 0.8])
    Fl = np.array([1.0, 2.0, 3.0, 0.0, 0.0, 0.0])
    out = orc.em_step(circ, p, Fl, step_size=0.5, pseudocount=0.3)
    r0 = (np.array([1.0, 2.0, 3.0]) + 0.1) / 6.3
    r1 = np.array([0.1, 0.1, 0.1]) / 0.3
    expect = np.concatenate([0.5 * p[:3] + 0.5 * r0, 0.5 * p[3:] + 0.5 * r1])
    _close(out, expect, 1e-14, 1e-15, "em blend")
    out0 = orc.em_step(circ, p, Fl)                   # alpha = 0: zero row keeps theta
    _close(out0, np.concatenate([[1 / 6, 2 / 6, 3 / 6], p[3:]]), 1e-14, 1e-15, "em zero row")


# ---------------------------------------------------------------------------
# HCLT: brute force and tree message passing
# ---------------------------------------------------------------------------

def _hclt_tables(circ, p):
    m = circ.meta
    H, K = m["H"], m["K"]
    nv = circ.num_vars
    Em = p[:nv * H * K].reshape(nv, H, K)
    th = {v: p[o:o + H * H].reshape(H, H) for v, o in m["param_off"].items()}
    pi = p[m["off_root"]:m["off_root"] + H]
    return Em, th, pi


def check_hclt_bruteforce(orc):
    """4 variables, 3 latents, 3 categories: LL = log of the sum over all
    latent assignments of the tree factorisation; probabilities sum to one."""
    circ = C.hclt(4, 3, 3, seed=2)
    p = _renorm(circ, I.softmax_rows_params(circ, np.random.default_rng(9)))
    Em, th, pi = _hclt_tables(circ, p)
    par = circ.meta["parent"]
    xs = np.array(list(itertools.product(range(3), repeat=4)), dtype=np.int32)
    _, ll = orc.forward(circ, p, len(xs), tokens=xs)
    expect = []
    for x in xs:
        tot = 0.0
        for z in itertools.product(range(3), repeat=4):
            pr = pi[z[0]]
            for v in range(4):
                pr *= Em[v, z[v], x[v]]
                if v:
                    pr *= th[v][z[par[v]], z[v]]
            tot += pr
        expect.append(np.log(tot))
    _close(ll, expect, 1e-12, 1e-12, "hclt brute force")
    assert abs(np.exp(ll).sum() - 1.0) < 1e-12


def check_hclt_tree_recursion(orc):
    """Upward message passing on a 12-variable tree = oracle LL."""
    cfg = make_config(kind="hclt", num_vars=12, H=5, K=4, B=7, seed=6)
    circ, B = cfg["circuit"], cfg["B"]
    p = cfg["params"].astype(F64)
    Em, th, pi = _hclt_tables(circ, p)
    kids = circ.meta["children"]
    x = cfg["tokens"]

    def up(v, xb):
        msg = Em[v, :, xb[v]].copy()
        for c in kids[v]:
            msg = msg * (th[c] @ up(c, xb))
        return msg

    _, ll = orc.forward(circ, p, B, tokens=x)
    expect = [np.log(pi @ up(0, x[b])) for b in range(B)]
    _close(ll, expect, 1e-12, 1e-12, "hclt tree recursion")


# ---------------------------------------------------------------------------
# Block-sparse circuits: normalisation and finite differences
# ---------------------------------------------------------------------------

def check_block_sparse_normalized(orc):
    """Random smooth decomposable block-sparse circuits sum to one over all
    27 assignments of 3 ternary variables."""
    for seed in range(4):
        circ = C.block_sparse(seed, num_vars=3, K=3, in_blocks=2, block=2, sum_blocks=2)
        p = _renorm(circ, I.softmax_rows_params(circ, np.random.default_rng(seed)))
        xs = np.array(list(itertools.product(range(3), repeat=3)), dtype=np.int32)
        _, ll = orc.forward(circ, p, len(xs), tokens=xs)
        assert abs(np.exp(ll).sum() - 1.0) < 1e-12, (seed, np.exp(ll).sum())


def check_pd_normalized(orc):
    """PD region-graph circuits (2 x 2 pixel grid, three categories; 2 x 3 with
    two; a 4 x 4 grid on a 2-pixel lattice whose leaf cells are products of
    four pixels, two categories) sum to one over every assignment of their
    variables, and every sample's LL equals the log of the brute-force sum over
    the region graph's latent choices for the 2 x 2 grid."""
    for (H, W, K, nc, split, seed) in [(2, 2, 2, 3, 1, 0), (2, 3, 3, 2, 1, 1), (4, 4, 2, 2, 2, 2)]:
        circ = C.pd(H, W, K, nc, split)
        p = _renorm(circ, I.softmax_rows_params(circ, np.random.default_rng(seed)))
        xs = np.array(list(itertools.product(range(nc), repeat=H * W)), dtype=np.int32)
        _, ll = orc.forward(circ, p, len(xs), tokens=xs)
        assert abs(np.exp(ll).sum() - 1.0) < 1e-12, ((H, W, K), np.exp(ll).sum())
    # 2 x 2 grid: regions are the 4 pixels, 2 + 2 dominoes and the square;
    # the square's root mixes 2 cuts (rows, columns) x K latents, each cut's
    # latent k multiplying the two dominoes' latent k, each domino mixing
    # its one cut's latent k' of the two pixels.
    circ = C.pd(2, 2, 2, 3, 1)
    p = _renorm(circ, I.softmax_rows_params(circ, np.random.default_rng(0)))
    xs = np.array(list(itertools.product(range(3), repeat=4)), dtype=np.int32)
    _, ll = orc.forward(circ, p, len(xs), tokens=xs)
    K = 2
    emit = p[:4 * K * 3].reshape(4, K, 3)                  # pixel v, latent k, category
    sums = {}
    for layer in circ.layers:
        if isinstance(layer, C.Sum):
            for g in layer.groups:
                sums[int(g.out_start)] = (g, p[g.param_offset:g.param_offset + g.num_nodes * g.num_children]
                                          .reshape(g.num_nodes, g.num_children))
    root_g, root_w = sums[circ.root]
    # the domino sum groups, keyed by their pixel pairs, in the order the builder
    # creates regions: sorted by (area, y0, y1, x0, x1)
    dominoes = sorted([(0, 1, 0, 2), (1, 2, 0, 2), (0, 2, 0, 1), (0, 2, 1, 2)])
    pix = {(0, 1, 0, 2): (0, 1), (1, 2, 0, 2): (2, 3), (0, 2, 0, 1): (0, 2), (0, 2, 1, 2): (1, 3)}
    dom_groups = sorted([g for g, _ in sums.values() if g.num_nodes == K], key=lambda g: g.out_start)
    dom_w = {r: sums[int(g.out_start)][1] for r, g in zip(dominoes, dom_groups)}
    cuts = [((0, 1, 0, 2), (1, 2, 0, 2)), ((0, 2, 0, 1), (0, 2, 1, 2))]   # rows, then columns
    expect = []
    for x in xs:
        def dom(r, k):
            a, b = pix[r]
            return sum(dom_w[r][k, q] * emit[a, q, x[a]] * emit[b, q, x[b]] for q in range(K))
        tot = 0.0
        for c, (r1, r2) in enumerate(cuts):
            for k in range(K):
                tot += root_w[0, c * K + k] * dom(r1, k) * dom(r2, k)
        expect.append(np.log(tot))
    _close(ll, expect, 1e-12, 1e-12, "pd 2x2 brute force")


def check_flows_fd(orc):
    """On a block-sparse circuit: parameter flows = theta * dLL/dtheta (sum and
    input parameters) and element flows = dLL/dv (node-value perturbation)."""
    circ = C.block_sparse(1, num_vars=4, K=3, in_blocks=2, block=2, sum_blocks=2)
    B = 4
    rng = np.random.default_rng(1)
    p = I.softmax_rows_params(circ, rng).astype(F64)
    x = rng.integers(0, 3, size=(B, 4)).astype(np.int32)

    def L(pp, perturb=None):
        return float(orc.forward(circ, pp, B, tokens=x, perturb=perturb)[1].sum())

    V, _ = orc.forward(circ, p, B, tokens=x)
    r = orc.backward(circ, p, V, tokens=x)
    for k in np.linspace(0, circ.num_params - 1, 23).astype(int):
        d = _fd(lambda q: L(q), p, int(k), 1e-6)
        _close(r["param_flows"][k], p[k] * d, 1e-6, 1e-9, f"param flow {k}")
    for node in np.linspace(0, circ.num_nodes - 1, 17).astype(int):
        for b in (0, 3):
            h = 1e-5
            dv = np.zeros(B)
            dv[b] = h
            d = (L(p, {int(node): dv}) - L(p, {int(node): -dv})) / (2 * h)
            _close(r["flows"][node, b], d, 1e-6, 1e-9, f"element flow node {node} b {b}")


def check_pd_flows_fd(orc):
    """On a PD circuit (3 x 3 grid, 3 latents): parameter flows = theta *
    dLL/dtheta and element flows = dLL/dv by central differences."""
    circ = C.pd(3, 3, 3, 3, 1)
    B = 3
    rng = np.random.default_rng(4)
    p = I.softmax_rows_params(circ, rng).astype(F64)
    x = rng.integers(0, 3, size=(B, 9)).astype(np.int32)

    def L(pp, perturb=None):
        return float(orc.forward(circ, pp, B, tokens=x, perturb=perturb)[1].sum())

    V, _ = orc.forward(circ, p, B, tokens=x)
    r = orc.backward(circ, p, V, tokens=x)
    for k in np.linspace(0, circ.num_params - 1, 19).astype(int):
        d = _fd(lambda q: L(q), p, int(k), 1e-6)
        _close(r["param_flows"][k], p[k] * d, 1e-6, 1e-9, f"pd param flow {k}")
    for node in np.linspace(0, circ.num_nodes - 1, 13).astype(int):
        h = 1e-5
        dv = np.zeros(B)
        dv[1] = h
        d = (L(p, {int(node): dv}) - L(p, {int(node): -dv})) / (2 * h)
        _close(r["flows"][node, 1], d, 1e-6, 1e-9, f"pd element flow node {node}")


# ---------------------------------------------------------------------------
# LowRank exp_sum
# ---------------------------------------------------------------------------

def _lowrank_case(B=5, seed=8, H=4, T=4, V=3, rank=2, sigma=0.7, form="exp_sum"):
    circ = C.hmm(H, T, V, lowrank_rank=rank, lowrank_form=form)
    rng = np.random.default_rng(seed)
    p = _renorm(circ, I.softmax_rows_params(circ, rng))
    x = I.uniform_tokens(circ, B, V, rng)
    fac = [(a.astype(F64), b.astype(F64)) for a, b in I.lowrank_factors(circ, B, sigma, rng)]
    return circ, p, x, fac


def check_lowrank_reductions(orc):
    """A = 0, or B constant along the children, leaves theta unchanged: the
    scaled circuit equals the plain one (values and flows)."""
    circ, p, x, fac = _lowrank_case()
    plain = C.hmm(4, 4, 3)
    B = x.shape[0]
    V0, ll0 = orc.forward(plain, p, B, tokens=x)
    r0 = orc.backward(plain, p, V0, tokens=x)
    zeroA = [(np.zeros_like(a), b) for a, b in fac]
    constB = [(a, np.repeat(b[:, :, :1], b.shape[2], axis=2)) for a, b in fac]
    for f in (zeroA, constB):
        V1, ll1 = orc.forward(circ, p, B, tokens=x, lowrank=f)
        r1 = orc.backward(circ, p, V1, tokens=x, lowrank=f)
        _close(ll1, ll0, 1e-12, 1e-12, "lowrank reduction LL")
        _close(r1["param_flows"], r0["param_flows"], 1e-10, 1e-12, "lowrank reduction param flows")
        _close(r1["flows"], r0["flows"], 1e-10, 1e-12, "lowrank reduction flows")


def _scale(a, b, form):
    """The scale of pyjuice.parameterizations.LowRank, definition, per form."""
    return np.exp(a @ b) if form == "exp_sum" else np.exp(a) @ np.exp(b)


def check_lowrank_inhomogeneous_hmm(orc, form="exp_sum"):
    """Scaled HMM = a per-sample time-inhomogeneous HMM with transition
    normalize(A * g_b) at each step (g_b the form's scale): LL by the forward
    algorithm, F+ by summed xi, probabilities of all sequences (one sample's
    factors) sum to one."""
    circ, p, x, fac = _lowrank_case(B=5, form=form)
    m = circ.meta
    H, T = m["H"], m["T"]
    A, pi, E = _hmm_tables(circ, p)
    B = x.shape[0]
    V, ll = orc.forward(circ, p, B, tokens=x, lowrank=fac)
    r = orc.backward(circ, p, V, tokens=x, lowrank=fac)
    xi_tot = np.zeros((H, H))
    for b in range(B):
        # transition from position t to t+1 uses the slot of sum layer t
        At = []
        for t in range(T - 1):
            q = A * _scale(fac[t][0][b], fac[t][1][b], form)
            At.append(q / q.sum(1, keepdims=True))
        alpha = pi * E[:, x[b, 0]]
        al = [alpha]
        for t in range(1, T):
            alpha = (alpha @ At[t - 1]) * E[:, x[b, t]]
            al.append(alpha)
        Pb = alpha.sum()
        _close(ll[b], np.log(Pb), 1e-12, 1e-12, "lowrank LL")
        beta = np.ones(H)
        for t in range(T - 2, -1, -1):
            xi_tot += al[t][:, None] * At[t] * (E[:, x[b, t + 1]] * beta)[None, :] / Pb
            beta = At[t] @ (E[:, x[b, t + 1]] * beta)
    _close(r["param_flows"][m["off_trans"]:m["off_trans"] + H * H].reshape(H, H), xi_tot,
           1e-10, 1e-12, "lowrank F+")
    # normalisation with one sample's factors for every sequence
    xs = np.array(list(itertools.product(range(3), repeat=T)), dtype=np.int32)
    fac1 = [(np.repeat(a[:1], len(xs), 0), np.repeat(b_[:1], len(xs), 0)) for a, b_ in fac]
    _, lla = orc.forward(circ, p, len(xs), tokens=xs, lowrank=fac1)
    assert abs(np.exp(lla).sum() - 1.0) < 1e-12


def check_lowrank_grad_fd(orc, form="exp_sum"):
    """dLL/dA and dLL/dB and the element flows of the scaled layer's children
    against central finite differences."""
    circ, p, x, fac = _lowrank_case(B=3, form=form)
    B = x.shape[0]

    def L(f, perturb=None):
        return float(orc.forward(circ, p, B, tokens=x, lowrank=f, perturb=perturb)[1].sum())

    V, _ = orc.forward(circ, p, B, tokens=x, lowrank=fac)
    r = orc.backward(circ, p, V, tokens=x, lowrank=fac)
    h = 1e-6
    for slot in (0, 2):
        for which, idx in (("A", (1, 2, 1)), ("A", (0, 3, 0)), ("B", (2, 0, 3)), ("B", (1, 1, 0))):
            k = 0 if which == "A" else 1
            fp = [(a.copy(), b.copy()) for a, b in fac]
            fm = [(a.copy(), b.copy()) for a, b in fac]
            fp[slot][k][idx] += h
            fm[slot][k][idx] -= h
            d = (L(fp) - L(fm)) / (2 * h)
            got = (r["dA"] if which == "A" else r["dB"])[slot][idx]
            _close(got, d, 1e-6, 1e-9, f"d{which} slot {slot} {idx}")
    for node in (0, 5, 13, 20):
        dv = np.zeros(B)
        dv[1] = 1e-5
        d = (L(fac, {node: dv}) - L(fac, {node: -dv})) / 2e-5
        _close(r["flows"][node, 1], d, 1e-6, 1e-9, f"lowrank element flow {node}")


def check_lowrank_sumexp_inhomogeneous_hmm(orc):
    """The "sum_exp" form (g = sum_r exp(A_b[:, r]) exp(B_b[r, :])) against the
    per-sample inhomogeneous HMM."""
    check_lowrank_inhomogeneous_hmm(orc, "sum_exp")


def check_lowrank_sumexp_grad_fd(orc):
    """The "sum_exp" form's dLL/dA, dLL/dB and element flows against central
    finite differences."""
    check_lowrank_grad_fd(orc, "sum_exp")


def check_lowrank_sumexp_reduction(orc):
    """"sum_exp" with B = 0: g[i, j] = sum_r exp(A_b[i, r]) is constant along a
    row and cancels in the normalisation, so the circuit equals the plain
    one (values, flows, parameter flows)."""
    circ, p, x, fac = _lowrank_case(form="sum_exp")
    plain = C.hmm(4, 4, 3)
    B = x.shape[0]
    V0, ll0 = orc.forward(plain, p, B, tokens=x)
    r0 = orc.backward(plain, p, V0, tokens=x)
    zeroB = [(a, np.zeros_like(b)) for a, b in fac]
    V1, ll1 = orc.forward(circ, p, B, tokens=x, lowrank=zeroB)
    r1 = orc.backward(circ, p, V1, tokens=x, lowrank=zeroB)
    _close(ll1, ll0, 1e-12, 1e-12, "sum_exp reduction LL")
    _close(r1["param_flows"], r0["param_flows"], 1e-10, 1e-12, "sum_exp reduction param flows")
    _close(r1["flows"], r0["flows"], 1e-10, 1e-12, "sum_exp reduction flows")


def check_lowrank_zstat_fd(orc, form="exp_sum"):
    """LowRank denominator statistic (pyjuice.parameterizations.LowRank,
    Training): with the element flows f held fixed, W = dJ/dtheta for
    J(theta) = sum over LowRank layers, samples and nodes of
    f_b[i] log Z_b[i](theta), Z_b[i] = sum_j theta[i,j] exp(A_b B_b)[i,j]
    (central differences on the tied transition block)."""
    circ, p, x, fac = _lowrank_case(B=3, form=form)
    B = x.shape[0]
    V, _ = orc.forward(circ, p, B, tokens=x, lowrank=fac)
    r = orc.backward(circ, p, V, tokens=x, lowrank=fac)
    groups = [g for ly in circ.layers if isinstance(ly, C.Sum) for g in ly.groups if g.lowrank >= 0]
    off, M, N = groups[0].param_offset, groups[0].num_nodes, groups[0].num_children

    def J(theta):
        tot = 0.0
        for g in groups:
            f = r["flows"][g.out_start:g.out_start + M]
            A, Bf = fac[g.lowrank]
            for b in range(B):
                Z = (theta * _scale(A[b], Bf[b], form)).sum(axis=1)
                tot += float((f[:, b] * np.log(Z)).sum())
        return tot

    th = p[off:off + M * N].reshape(M, N)
    h = 1e-6
    for (i, j) in ((0, 0), (1, 3), (3, 2), (2, 1)):
        tp, tm = th.copy(), th.copy()
        tp[i, j] += h
        tm[i, j] -= h
        _close(r["z_flows"][off + i * N + j], (J(tp) - J(tm)) / (2 * h), 1e-6, 1e-9, f"W[{i},{j}]")
    # nothing outside the LowRank blocks
    mask = np.ones(circ.num_params, bool)
    mask[off:off + M * N] = False
    assert not r["z_flows"][mask].any()


def check_lowrank_sumexp_zstat_fd(orc):
    """W of the "sum_exp" form against finite differences of sum f log Z."""
    check_lowrank_zstat_fd(orc, "sum_exp")


def check_lowrank_zstat_reduction(orc):
    """With A = 0 (no scale) Z_b[i] is the row sum of theta (1), so W[i, :] is
    the node's flow summed over samples and copies, and the conditional
    M-step without pseudocount is the plain EM step."""
    circ, p, x, fac = _lowrank_case()
    B = x.shape[0]
    zeroA = [(np.zeros_like(a), b) for a, b in fac]
    V, _ = orc.forward(circ, p, B, tokens=x, lowrank=zeroA)
    r = orc.backward(circ, p, V, tokens=x, lowrank=zeroA)
    groups = [g for ly in circ.layers if isinstance(ly, C.Sum) for g in ly.groups if g.lowrank >= 0]
    off, M, N = groups[0].param_offset, groups[0].num_nodes, groups[0].num_children
    fsum = sum(r["flows"][g.out_start:g.out_start + M].sum(axis=1) for g in groups)
    _close(r["z_flows"][off:off + M * N].reshape(M, N), np.repeat(fsum[:, None], N, axis=1), 1e-12, 1e-12,
           "W with A = 0")
    # (without a pseudocount: alpha / n does not scale with the row)
    for eta in (1.0, 0.5):
        _close(orc.em_step_corrected(circ, p, r["param_flows"], r["z_flows"], eta, 0.0),
               orc.em_step(circ, p, r["param_flows"], eta, 0.0), 1e-12, 1e-14, "corrected M-step with A = 0")


def check_em_corrected_row(orc):
    """Conditional M-step on a hand-computed row of a one-node LowRank layer:
    theta = (0.5, 0.25, 0.25, 0), F+ = (1, 2, 0.5, 0), W = (4, 2, 1, 3):
    F+ / W = (0.25, 1, 0.5, 0) -> (1/7, 4/7, 2/7, 0); with eta = 0.5 and
    alpha = 0.2: (0.5 theta + 0.5 (R + 0.05) / 1.95)."""
    ext = C.InputExternal(0, 4)
    g = C.SumGroup(4, 1, np.array([0]), 4, 0, lowrank=0)
    circ = C.Circuit("row", 5, 0, 4, [ext, C.Sum([g])], root=4, lowrank_rank=1)
    th = np.array([0.5, 0.25, 0.25, 0.0])
    Fp = np.array([1.0, 2.0, 0.5, 0.0])
    W = np.array([4.0, 2.0, 1.0, 3.0])
    _close(orc.em_step_corrected(circ, th, Fp, W, 1.0, 0.0), np.array([1, 4, 2, 0]) / 7.0, 1e-15, 1e-15,
           "corrected row")
    R = np.array([0.25, 1.0, 0.5, 0.0])
    _close(orc.em_step_corrected(circ, th, Fp, W, 0.5, 0.2), 0.5 * th + 0.5 * (R + 0.05) / 1.95, 1e-15, 1e-15,
           "corrected row with step and pseudocount")


# ---------------------------------------------------------------------------
# Invariants
# ---------------------------------------------------------------------------

def check_invariants(orc):
    """HMM: flows of each position's product nodes sum to 1 per sample; row
    sums of transition flows = summed flows of the sum nodes over copies and
    samples; LL <= 0; EM rows sum to one."""
    cfg = make_config("tiny_hmm")
    circ, B = cfg["circuit"], cfg["B"]
    m = circ.meta
    H = m["H"]
    p = _renorm(circ, cfg["params"])
    V, ll = orc.forward(circ, p, B, tokens=cfg["tokens"])
    assert (ll <= 0).all()
    r = orc.backward(circ, p, V, tokens=cfg["tokens"])
    Fl = r["flows"]
    tot = np.zeros(H)
    for t, ps in m["prod_starts"].items():
        _close(Fl[ps:ps + H].sum(0), np.ones(B), 1e-12, 1e-12, f"flow sum t={t}")
        ss = m["sum_starts"][t]
        tot += Fl[ss:ss + H].sum(1)
    rows = r["param_flows"][:H * H].reshape(H, H).sum(1)
    _close(rows, tot, 1e-11, 1e-12, "flow conservation")
    newp = orc.em_step(circ, p, r["param_flows"])
    for off, nr, rl in circ.param_row_segments():
        _close(newp[off:off + nr * rl].reshape(nr, rl).sum(1), np.ones(nr), 1e-13, 1e-13, "em rows")


def check_neg_inf_flows(orc):
    """A column whose children are all -inf: value -inf, zero flows, no NaN."""
    cfg = make_config(kind="dense", M=4, N=6, groups=1, B=3, seed=2)
    circ = cfg["circuit"]
    p = cfg["params"].astype(F64)
    ext = cfg["external"].astype(F64)
    ext[:, 1] = -np.inf
    V, _ = orc.forward(circ, p, 3, external=ext)
    assert np.isneginf(V[6:, 1]).all()
    r = orc.backward(circ, p, V, seed_flows=cfg["seed_flows"])
    assert not np.isnan(r["flows"]).any() and not np.isnan(r["param_flows"]).any()
    assert (r["flows"][:6, 1] == 0).all()


ALL_CHECKS = [check_dense_logsumexp, check_dense_flows_fd, check_hmm_bruteforce,
              check_hmm_forward_algorithm, check_hmm_posteriors, check_baum_welch,
              check_em_blend_and_pseudocount, check_hclt_bruteforce, check_hclt_tree_recursion,
              check_block_sparse_normalized, check_pd_normalized, check_flows_fd, check_pd_flows_fd,
              check_lowrank_reductions,
              check_lowrank_inhomogeneous_hmm, check_lowrank_grad_fd, check_lowrank_zstat_fd,
              check_lowrank_sumexp_inhomogeneous_hmm, check_lowrank_sumexp_grad_fd,
              check_lowrank_sumexp_reduction, check_lowrank_sumexp_zstat_fd,
              check_lowrank_zstat_reduction, check_em_corrected_row, check_invariants,
              check_neg_inf_flows]
