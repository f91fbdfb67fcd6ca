"""Float64 CPU oracle for the probabilistic-circuit sum-layer hot path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports, calls or links
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg do.  It shares no code with the HIP path; both read the same circuit
structures and seeded inputs from ``workloads``.

What it computes (plain definitions, float64, numpy):

* categorical input node:  v[u,b] = log theta_in[row(u), x[b, var(u)]];
* product node:            v[p,b] = sum of its children's values;
* sum node (PyJuice pull request #62, Summary item 2: a sum layer
  exponentiates its children, multiplies by the weights and takes the log):
                           v[i,b] = log sum_j theta[i,j] exp(v[j,b]),
  evaluated as m[b] + log(theta @ exp(v_ch - m)) with m the per-sample
  maximum over the group's children (the "per-group column maximum" of the
  pull request's Tests section).  The shift is an exact identity; a column
  whose children are all -inf takes m = 0 so that its value is -inf;
* element flows (the "element flows" of Summary item 3): f = dLL/dv with
  f[root] = 1 (or caller-given seeds on output nodes), pushed to children in
  reverse layer order: a product passes its flow to each child, a sum node
  passes f[i]*theta[i,j]*exp(v[j]-v[i]) to child j;
* parameter flows (Summary item 3): F[i,j] = sum over samples and tied copies
  of f[i]*theta[i,j]*exp(v[j]-v[i]) (expected edge counts); input rows:
  F_in[row,k] = sum of f[u,b] over nodes u of the row and samples b with
  x[b,var(u)] = k;
* EM (pyjuice.parameterizations.LowRank, Training: plain EM is normalize(F)):
  theta <- (1-eta)*theta + eta*(F + alpha/n)/(sum F + alpha) per row; a row with
  zero total keeps its weights;
* LowRank (pyjuice.parameterizations.LowRank, definition):
  theta_b = theta * g_b / Z_b, Z_b[i] = sum_j theta[i,j] g_b[i,j], with the
  scale g_b = exp(A_b B_b) ("exp_sum") or g_b[i,j] = sum_r exp(A_b[i,r])
  exp(B_b[r,j]) ("sum_exp"), built explicitly per sample; the layer is the sum
  layer above with theta_b.  The gradients go through dLL/dg (chain rule).
  Its backward (Training) writes the element flows, the parameter flows
  F+ = sum_b of the edge flows under theta_b, and dLL/dA, dLL/dB;
* LowRank denominator statistic (pyjuice.parameterizations.LowRank, Training,
  apply_z_correction): W[i,j] = sum over samples and tied copies of
  f_b[i] * exp(A_b B_b)[i,j] / Z_b[i], in the parameter flows' layout, and the
  conditional M-step theta <- normalize(theta * F+ / F-) with F- = theta * W,
  i.e. normalize(F+ / W) on the entries with theta > 0 and W > 0 (0 elsewhere),
  normalised as the plain EM step (same step size and pseudocount).
"""
from __future__ import annotations

import numpy as np

from workloads.circuits import Circuit, InputCat, InputExternal, Product, Sum


def _log(x):
    with np.errstate(divide="ignore"):
        return np.log(x)


def _colmax(C):
    """Per-sample maximum over the children (axis 0); -inf columns -> 0."""
    m = C.max(axis=0) if C.shape[0] else np.zeros(C.shape[1])
    return np.where(np.isfinite(m), m, 0.0)


def _theta(params, g):
    M, N = g.num_nodes, g.num_children
    return params[g.param_offset:g.param_offset + M * N].reshape(M, N)


def lowrank_scale(A_b, B_b, form="exp_sum"):
    """g_b of pyjuice.parameterizations.LowRank: exp(A_b B_b) for "exp_sum",
    sum_r exp(A_b[:, r]) exp(B_b[r, :]) for "sum_exp"."""
    if form == "exp_sum":
        return np.exp(A_b @ B_b)
    if form == "sum_exp":
        return np.exp(A_b) @ np.exp(B_b)
    raise ValueError(form)


def lowrank_effective(theta, A_b, B_b, form="exp_sum"):
    """theta_b = theta * g_b normalised over each row's children
    (pyjuice.parameterizations.LowRank, definition).  Returns (theta_b, q, Z)
    with q = theta * g_b and Z its row sums."""
    q = theta * lowrank_scale(A_b, B_b, form)
    Z = q.sum(axis=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        tb = np.where(Z[:, None] > 0, q / Z[:, None], 0.0)
    return tb, q, Z


def forward(circ: Circuit, params, B: int, tokens=None, external=None, lowrank=None,
            perturb=None):
    """Node values [num_nodes, B] (float64) and the root's log-likelihood [B].

    ``external``: float [n_ext, B] values of the InputExternal layers in layer
    order.  ``lowrank``: list of (A [B,M,k], B [B,k,N]) per slot.  ``perturb``:
    optional {node id: delta [B]} added to a node's value right after its layer
    computes it (used by the finite-difference checks)."""
    p = np.asarray(params, dtype=np.float64)
    V = np.full((circ.num_nodes, B), np.nan)
    ext_off = 0
    for layer in circ.layers:
        if isinstance(layer, InputCat):
            x = np.asarray(tokens)[:, layer.var].T.astype(np.int64)        # [n, B]
            idx = layer.param_offset + layer.row.astype(np.int64)[:, None] * layer.num_cats + x
            V[layer.node_start:layer.node_start + layer.num_nodes] = _log(p[idx])
            rng_nodes = [(layer.node_start, layer.num_nodes)]
        elif isinstance(layer, InputExternal):
            ext = np.asarray(external, dtype=np.float64)
            V[layer.node_start:layer.node_start + layer.num_nodes] = ext[ext_off:ext_off + layer.num_nodes]
            ext_off += layer.num_nodes
            rng_nodes = [(layer.node_start, layer.num_nodes)]
        elif isinstance(layer, Product):
            ptr = layer.ch_ptr.astype(np.int64)
            vals = V[layer.ch_ids.astype(np.int64)]
            V[layer.node_start:layer.node_start + layer.num_nodes] = np.add.reduceat(vals, ptr[:-1], axis=0)
            rng_nodes = [(layer.node_start, layer.num_nodes)]
        elif isinstance(layer, Sum):
            rng_nodes = []
            for g in layer.groups:
                C = V[g.child_ids()]                                     # [N, B]
                m = _colmax(C)
                E = np.exp(C - m)
                th = _theta(p, g)
                if g.lowrank >= 0:
                    A, Bf = lowrank[g.lowrank]
                    S = np.empty((g.num_nodes, B))
                    for b in range(B):
                        tb, _, _ = lowrank_effective(th, np.asarray(A[b], np.float64),
                                                     np.asarray(Bf[b], np.float64), circ.lowrank_form)
                        S[:, b] = tb @ E[:, b]
                else:
                    S = th @ E
                V[g.out_start:g.out_start + g.num_nodes] = m + _log(S)
                rng_nodes.append((g.out_start, g.num_nodes))
        else:
            raise TypeError(layer)
        if perturb:
            for s, n in rng_nodes:
                for node, d in perturb.items():
                    if s <= node < s + n:
                        V[node] = V[node] + d
    ll = V[circ.root].copy() if circ.root >= 0 else None
    return V, ll


def backward(circ: Circuit, params, V, tokens=None, lowrank=None, seed_flows=None):
    """Element flows [num_nodes, B], parameter flows [num_params] and, for
    LowRank slots, dLL/dA and dLL/dB.

    Seeds: flow 1 at the root per sample, or ``seed_flows`` [n_out, B] on the
    circuit's output nodes in ascending node order."""
    p = np.asarray(params, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    B = V.shape[1]
    F = np.zeros_like(V)
    if seed_flows is not None:
        F[circ.output_nodes()] = np.asarray(seed_flows, dtype=np.float64)
    else:
        F[circ.root] = 1.0
    PF = np.zeros(circ.num_params)
    ZF = np.zeros(circ.num_params)
    dA = {}
    dB = {}
    for layer in reversed(circ.layers):
        if isinstance(layer, Sum):
            for g in layer.groups:
                ch = g.child_ids()
                C = V[ch]
                m = _colmax(C)
                E = np.exp(C - m)                                        # e[j,b]
                n = V[g.out_start:g.out_start + g.num_nodes]
                f = F[g.out_start:g.out_start + g.num_nodes]
                # f[i,b] * exp(m[b] - v[i,b]) (= f / S); zero where f = 0 or v = -inf
                with np.errstate(over="ignore", invalid="ignore"):
                    gm = np.where((f != 0) & np.isfinite(n), f * np.exp(m - n), 0.0)
                th = _theta(p, g)
                if g.lowrank >= 0:
                    A, Bf = lowrank[g.lowrank]
                    dAg = np.zeros(A.shape)
                    dBg = np.zeros(Bf.shape)
                    pf = np.zeros_like(th)
                    zf = np.zeros_like(th)
                    fc = np.zeros_like(C)
                    for b in range(B):
                        Ab = np.asarray(A[b], np.float64)
                        Bb = np.asarray(Bf[b], np.float64)
                        gb = lowrank_scale(Ab, Bb, circ.lowrank_form)
                        tb, _, Z = lowrank_effective(th, Ab, Bb, circ.lowrank_form)
                        eps = tb * E[:, b][None, :] * gm[:, b][:, None]  # edge flows
                        fc[:, b] = eps.sum(axis=0)
                        pf += eps
                        fi = np.where(np.isfinite(n[:, b]), f[:, b], 0.0)
                        D = eps - fi[:, None] * tb                       # dLL/dg * g
                        if circ.lowrank_form == "exp_sum":               # g = exp(h), h = A_b B_b
                            dAg[b] = D @ Bb.T
                            dBg[b] = Ab.T @ D
                        else:                                            # g = exp(A_b) exp(B_b)
                            G = D / gb                                   # dLL/dg (g > 0)
                            eA, eB = np.exp(Ab), np.exp(Bb)
                            dAg[b] = eA * (G @ eB.T)
                            dBg[b] = eB * (eA.T @ G)
                        # denominator statistic: f_b[i] exp(A_b B_b)[i, j] / Z_b[i]
                        with np.errstate(divide="ignore", invalid="ignore"):
                            fz = np.where((fi != 0) & (Z > 0), fi / Z, 0.0)
                        zf += fz[:, None] * gb
                    F[ch] += fc
                    PF[g.param_offset:g.param_offset + th.size] += pf.reshape(-1)
                    ZF[g.param_offset:g.param_offset + th.size] += zf.reshape(-1)
                    dA[g.lowrank] = dAg
                    dB[g.lowrank] = dBg
                else:
                    F[ch] += E * (th.T @ gm)
                    PF[g.param_offset:g.param_offset + th.size] += (th * (gm @ E.T)).reshape(-1)
        elif isinstance(layer, Product):
            ptr = layer.ch_ptr.astype(np.int64)
            counts = np.diff(ptr)
            parents = np.repeat(np.arange(layer.node_start, layer.node_start + layer.num_nodes), counts)
            np.add.at(F, layer.ch_ids.astype(np.int64), F[parents])
        elif isinstance(layer, InputCat):
            x = np.asarray(tokens)[:, layer.var].T.astype(np.int64)
            idx = layer.param_offset + layer.row.astype(np.int64)[:, None] * layer.num_cats + x
            np.add.at(PF, idx.reshape(-1), F[layer.node_start:layer.node_start + layer.num_nodes].reshape(-1))
        elif isinstance(layer, InputExternal):
            pass
    return dict(flows=F, param_flows=PF, dA=dA, dB=dB, z_flows=ZF)


def lowrank_param_ranges(circ: Circuit):
    """(offset, length) of the weight block of every LowRank group."""
    out = []
    for layer in circ.layers:
        if isinstance(layer, Sum):
            for g in layer.groups:
                if g.lowrank >= 0:
                    out.append((g.param_offset, g.num_nodes * g.num_children))
    return sorted(set(out))


def em_step_corrected(circ: Circuit, params, param_flows, z_flows, step_size: float = 1.0,
                      pseudocount: float = 0.0):
    """The EM update with the LowRank conditional M-step: the rows of LowRank
    weight blocks take R = F+ / W (entries with theta > 0 and W > 0, else 0)
    in place of F, every other row the plain step."""
    p = np.asarray(params, dtype=np.float64)
    F = np.array(param_flows, dtype=np.float64)
    W = np.asarray(z_flows, dtype=np.float64)
    for off, n in lowrank_param_ranges(circ):
        th, fp, w = p[off:off + n], F[off:off + n], W[off:off + n]
        with np.errstate(divide="ignore", invalid="ignore"):
            F[off:off + n] = np.where((th > 0) & (w > 0), fp / w, 0.0)
    return em_step(circ, p, F, step_size, pseudocount)


def em_step(circ: Circuit, params, param_flows, step_size: float = 1.0, pseudocount: float = 0.0):
    """One EM update of every parameter row (tied rows once):
    theta <- (1-eta) theta + eta (F + alpha/n) / (sum F + alpha)."""
    p = np.array(params, dtype=np.float64)
    F = np.asarray(param_flows, dtype=np.float64)
    for off, nrows, rlen in circ.param_row_segments():
        th = p[off:off + nrows * rlen].reshape(nrows, rlen)
        fl = F[off:off + nrows * rlen].reshape(nrows, rlen)
        tot = fl.sum(axis=1) + pseudocount
        new = th.copy()
        ok = tot > 0
        new[ok] = (fl[ok] + pseudocount / rlen) / tot[ok][:, None]
        p[off:off + nrows * rlen] = ((1.0 - step_size) * th + step_size * new).reshape(-1)
    return p
