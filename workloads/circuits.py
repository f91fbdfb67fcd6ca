"""Circuit structures for the synthetic workloads.

A circuit is a list of layers in topological order over a global node
numbering.  Every node value is a log-probability per sample.  Three layer
kinds compute values, one kind receives them:

* ``InputCat``      categorical input nodes: node u reads category
                    ``tokens[b, var[u]]`` of its own parameter row ``row[u]``
                    (rows with the same index are tied);
* ``InputExternal`` nodes whose values the caller supplies (used to drive a
                    lone sum layer, as the dense-layer tests on the PyJuice
                    precision pull request do);
* ``Product``       node value = sum of its children's values (CSR child list);
* ``Sum``           groups of sum nodes; group g has ``M`` nodes over the
                    ``N = nblocks * block`` children listed as blocks of
                    consecutive node ids, and a row-major ``[M, N]`` weight
                    matrix at ``param_offset`` in the flat parameter vector.
                    Two groups with the same ``param_offset`` share (tie) their
                    weights.  ``lowrank`` >= 0 names the per-sample factor pair
                    that scales the group (PyJuice ``LowRank`` exp_sum form).

This module only describes structure and draws seeded inputs; it computes
nothing of the circuit itself.  It is shared by the float64 oracle and by the
HIP path's tests and benchmark.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np


@dataclass
class InputCat:
    node_start: int
    num_nodes: int
    num_cats: int
    var: np.ndarray          # int32 [num_nodes]
    row: np.ndarray          # int32 [num_nodes]
    param_offset: int        # row r of this layer's table starts at param_offset + r*num_cats
    num_rows: int


@dataclass
class InputExternal:
    node_start: int
    num_nodes: int


@dataclass
class Product:
    node_start: int
    num_nodes: int
    ch_ptr: np.ndarray       # int32 [num_nodes + 1]
    ch_ids: np.ndarray       # int32 [nnz]


@dataclass
class SumGroup:
    out_start: int
    num_nodes: int           # M
    ch_block_start: np.ndarray  # int32 [nblocks]
    ch_block_size: int
    param_offset: int
    lowrank: int = -1

    @property
    def num_children(self) -> int:
        return int(len(self.ch_block_start)) * int(self.ch_block_size)

    def child_ids(self) -> np.ndarray:
        s = np.asarray(self.ch_block_start, dtype=np.int64)
        return (s[:, None] + np.arange(self.ch_block_size, dtype=np.int64)[None, :]).reshape(-1)


@dataclass
class Sum:
    groups: List[SumGroup]


@dataclass
class Circuit:
    name: str
    num_nodes: int
    num_vars: int
    num_params: int
    layers: list
    root: int = -1                      # node whose value is the log-likelihood (-1: none)
    lowrank_rank: int = 0               # rank k of every LowRank factor pair
    lowrank_form: str = "exp_sum"       # how the factors make the scale: "exp_sum" or "sum_exp"
    meta: dict = field(default_factory=dict)

    # --- structural helpers (no arithmetic of the method) -----------------
    def param_row_segments(self):
        """Unique parameter row blocks as (offset, num_rows, row_len), each a
        run of rows that EM normalises independently."""
        seen = {}
        for layer in self.layers:
            if isinstance(layer, Sum):
                for g in layer.groups:
                    key = int(g.param_offset)
                    seg = (key, int(g.num_nodes), int(g.num_children))
                    if key in seen and seen[key] != seg:
                        raise ValueError("partially overlapping tied parameters")
                    seen[key] = seg
            elif isinstance(layer, InputCat):
                key = int(layer.param_offset)
                seg = (key, int(layer.num_rows), int(layer.num_cats))
                if key in seen and seen[key] != seg:
                    raise ValueError("partially overlapping tied parameters")
                seen[key] = seg
        return sorted(seen.values())

    def lowrank_slots(self):
        """[(slot, M, N)] for every LowRank-scaled group, ordered by slot."""
        out = {}
        for layer in self.layers:
            if isinstance(layer, Sum):
                for g in layer.groups:
                    if g.lowrank >= 0:
                        out[int(g.lowrank)] = (int(g.num_nodes), int(g.num_children))
        return [(s, *out[s]) for s in sorted(out)]

    def output_nodes(self) -> np.ndarray:
        """Nodes that no layer uses as a child."""
        used = np.zeros(self.num_nodes, dtype=bool)
        for layer in self.layers:
            if isinstance(layer, Product):
                used[layer.ch_ids] = True
            elif isinstance(layer, Sum):
                for g in layer.groups:
                    used[g.child_ids()] = True
        defined = np.zeros(self.num_nodes, dtype=bool)
        for layer in self.layers:
            for s, n in _node_ranges(layer):
                defined[s:s + n] = True
        return np.nonzero(defined & ~used)[0].astype(np.int64)


def _node_ranges(layer):
    if isinstance(layer, Sum):
        return [(g.out_start, g.num_nodes) for g in layer.groups]
    return [(layer.node_start, layer.num_nodes)]


def node_ranges(layer):
    return _node_ranges(layer)


# ---------------------------------------------------------------------------
# Builders
# ---------------------------------------------------------------------------

def hmm(H: int, T: int, V: int, lowrank_rank: int = 0, lowrank_form: str = "exp_sum") -> Circuit:
    """Homogeneous HMM with H hidden states, T positions, V symbols, written as
    a circuit in backward-recursion form.

    Position t has H emission input nodes I_t[z] (tied rows: emission row z),
    for t < T-1 a sum layer s_t[z] = log sum_z' A[z,z'] exp(p_{t+1}[z']) over the
    next position (one dense group: every node shares all children) and a
    product p_t[z] = I_t[z] + s_t[z]; p_{T-1} is I_{T-1}.  The root is a one-node
    sum over p_0 with the initial distribution.  The transition matrix A is tied
    across the T-1 positions.

    Parameter layout: A [H, H] at 0, initial [1, H] at H*H, emission [H, V]
    after it.  With ``lowrank_rank`` > 0 every transition group gets its own
    LowRank factor slot (slot = position index t).
    """
    off_trans = 0
    off_init = H * H
    off_emit = off_init + H
    num_params = off_emit + H * V
    layers = []
    inp = InputCat(node_start=0, num_nodes=T * H, num_cats=V,
                   var=np.repeat(np.arange(T, dtype=np.int32), H),
                   row=np.tile(np.arange(H, dtype=np.int32), T),
                   param_offset=off_emit, num_rows=H)
    layers.append(inp)
    nxt = T * H
    child_start = (T - 1) * H          # I_{T-1}
    slot = 0
    sum_starts = {}
    prod_starts = {}
    for t in range(T - 2, -1, -1):
        s_start = nxt
        nxt += H
        g = SumGroup(out_start=s_start, num_nodes=H,
                     ch_block_start=np.array([child_start], dtype=np.int32),
                     ch_block_size=H, param_offset=off_trans,
                     lowrank=(t if lowrank_rank > 0 else -1))
        layers.append(Sum([g]))
        p_start = nxt
        nxt += H
        ptr = np.arange(0, 2 * H + 1, 2, dtype=np.int32)
        ids = np.empty(2 * H, dtype=np.int32)
        ids[0::2] = t * H + np.arange(H, dtype=np.int32)
        ids[1::2] = s_start + np.arange(H, dtype=np.int32)
        layers.append(Product(node_start=p_start, num_nodes=H, ch_ptr=ptr, ch_ids=ids))
        sum_starts[t] = s_start
        prod_starts[t] = p_start
        child_start = p_start
        slot += 1
    root = nxt
    nxt += 1
    layers.append(Sum([SumGroup(out_start=root, num_nodes=1,
                                ch_block_start=np.array([child_start], dtype=np.int32),
                                ch_block_size=H, param_offset=off_init)]))
    c = Circuit(name=f"hmm{H}x{T}v{V}", num_nodes=nxt, num_vars=T, num_params=num_params,
                layers=layers, root=root, lowrank_rank=lowrank_rank, lowrank_form=lowrank_form)
    c.meta = dict(kind="hmm", H=H, T=T, V=V, off_trans=off_trans, off_init=off_init,
                  off_emit=off_emit, sum_starts=sum_starts, prod_starts=prod_starts)
    return c


def dense_layer(M: int, N: int, groups: int = 1) -> Circuit:
    """One sum layer over externally supplied child values.

    ``groups`` independent groups, each M nodes over its own N children; group
    g's children are nodes [g*N, (g+1)*N), its outputs follow all children and
    its weights are the g-th [M, N] block of the parameter vector, so the
    groups are evenly strided in children, outputs and parameters.
    """
    ext = InputExternal(node_start=0, num_nodes=groups * N)
    gl = []
    for g in range(groups):
        gl.append(SumGroup(out_start=groups * N + g * M, num_nodes=M,
                           ch_block_start=np.array([g * N], dtype=np.int32),
                           ch_block_size=N, param_offset=g * M * N))
    c = Circuit(name=f"dense{M}x{N}g{groups}", num_nodes=groups * (N + M), num_vars=0,
                num_params=groups * M * N, layers=[ext, Sum(gl)], root=-1)
    c.meta = dict(kind="dense", M=M, N=N, groups=groups)
    return c


def prufer_tree(n: int, rng: np.random.Generator) -> np.ndarray:
    """Uniform random labelled tree on n vertices (Pruefer sequence), returned
    as a parent array with vertex 0 as the root (parent[0] = -1)."""
    if n == 1:
        return np.array([-1])
    if n == 2:
        return np.array([-1, 0])
    seq = rng.integers(0, n, size=n - 2)
    degree = np.ones(n, dtype=np.int64)
    for v in seq:
        degree[v] += 1
    adj = [[] for _ in range(n)]
    import heapq
    leaves = [v for v in range(n) if degree[v] == 1]
    heapq.heapify(leaves)
    for v in seq:
        leaf = heapq.heappop(leaves)
        adj[leaf].append(int(v))
        adj[int(v)].append(leaf)
        degree[v] -= 1
        if degree[v] == 1:
            heapq.heappush(leaves, int(v))
    u = heapq.heappop(leaves)
    w = heapq.heappop(leaves)
    adj[u].append(w)
    adj[w].append(u)
    parent = np.full(n, -1, dtype=np.int64)
    seen = np.zeros(n, dtype=bool)
    stack = [0]
    seen[0] = True
    while stack:
        v = stack.pop()
        for w in adj[v]:
            if not seen[w]:
                seen[w] = True
                parent[w] = v
                stack.append(w)
    return parent


def hclt(num_vars: int, H: int, K: int, seed: int) -> Circuit:
    """HCLT-like circuit: a latent tree with H latent states per variable over a
    random spanning tree of the variables (root = variable 0).

    Per variable v: H categorical input nodes I_v[z] with their own rows (row
    v*H + z of a [num_vars*H, K] table); a product P_v[z] = I_v[z] + sum over
    tree children c of S_c[z]; per non-root v an edge sum S_v[z] = log sum_z'
    theta_v[z, z'] exp(P_v[z']) with its own [H, H] matrix.  Root = one-node sum
    over P_0.  Products and sums are layered by tree height; within a height
    level the edge groups are evenly strided in outputs, children and
    parameters (node ids and parameter offsets are assigned in level order).
    """
    rng = np.random.default_rng(seed)
    parent = prufer_tree(num_vars, rng)
    children = [[] for _ in range(num_vars)]
    for v in range(1, num_vars):
        children[parent[v]].append(v)
    height = np.zeros(num_vars, dtype=np.int64)
    order = []
    stack = [(0, False)]
    while stack:
        v, done = stack.pop()
        if done:
            order.append(v)
            height[v] = 0 if not children[v] else 1 + max(height[c] for c in children[v])
        else:
            stack.append((v, True))
            for c in children[v]:
                stack.append((c, False))
    maxh = int(height.max())
    levels = [[v for v in range(num_vars) if height[v] == h] for h in range(maxh + 1)]
    # node id assignment
    in_off = 0
    inp = InputCat(node_start=0, num_nodes=num_vars * H, num_cats=K,
                   var=np.repeat(np.arange(num_vars, dtype=np.int32), H),
                   row=np.arange(num_vars * H, dtype=np.int32),
                   param_offset=0, num_rows=num_vars * H)
    emit_params = num_vars * H * K
    nxt = num_vars * H
    layers = [inp]
    p_start = {}
    s_start = {}
    param_off = {}
    pcur = emit_params
    for h in range(maxh + 1):
        lvl = levels[h]
        # products of this level
        base = nxt
        ptr = [0]
        ids = []
        for i, v in enumerate(lvl):
            p_start[v] = base + i * H
        for i, v in enumerate(lvl):
            for z in range(H):
                ids.append(v * H + z)
                for c in children[v]:
                    ids.append(s_start[c] + z)
                ptr.append(len(ids))
        layers.append(Product(node_start=base, num_nodes=len(lvl) * H,
                              ch_ptr=np.array(ptr, dtype=np.int32),
                              ch_ids=np.array(ids, dtype=np.int32)))
        nxt = base + len(lvl) * H
        # edge sums of this level (every non-root variable)
        edge_vars = [v for v in lvl if v != 0]
        if edge_vars:
            sbase = nxt
            groups = []
            for i, v in enumerate(edge_vars):
                s_start[v] = sbase + i * H
                param_off[v] = pcur
                groups.append(SumGroup(out_start=s_start[v], num_nodes=H,
                                       ch_block_start=np.array([p_start[v]], dtype=np.int32),
                                       ch_block_size=H, param_offset=pcur))
                pcur += H * H
            layers.append(Sum(groups))
            nxt = sbase + len(edge_vars) * H
    root = nxt
    nxt += 1
    layers.append(Sum([SumGroup(out_start=root, num_nodes=1,
                                ch_block_start=np.array([p_start[0]], dtype=np.int32),
                                ch_block_size=H, param_offset=pcur)]))
    pcur += H
    c = Circuit(name=f"hclt{num_vars}x{H}k{K}", num_nodes=nxt, num_vars=num_vars,
                num_params=pcur, layers=layers, root=root)
    c.meta = dict(kind="hclt", H=H, K=K, parent=parent, children=children, height=height,
                  p_start=p_start, s_start=s_start, param_off=param_off,
                  off_root=pcur - H, emit_params=emit_params)
    return c


def block_sparse(seed: int, num_vars: int = 3, K: int = 3, in_blocks: int = 2,
                 block: int = 2, sum_blocks: int = 2, density: float = 0.6,
                 depth_sums: int = 2) -> Circuit:
    """Random smooth and decomposable circuit whose sum layers are block-sparse.

    Each variable gets ``in_blocks`` blocks of ``block`` categorical input nodes.
    Scopes are merged pairwise along a random binary tree: for a merge of scope
    L and R, product blocks pair a block of L with a block of R elementwise; then
    ``depth_sums`` (first level) sum layers over all blocks of the same scope,
    where every output block connects to a random non-empty subset of the scope's
    blocks (density ``density``).  The final scope gets a one-node root sum over
    all its blocks.  Node blocks are contiguous and child blocks are
    ``block`` consecutive nodes, so every sum group is a (node block, child-block
    list) pair: the general block-sparse layout.
    """
    rng = np.random.default_rng(seed)
    layers = []
    nxt = 0
    pcur = 0
    # inputs
    ninp = num_vars * in_blocks * block
    var = np.repeat(np.arange(num_vars, dtype=np.int32), in_blocks * block)
    inp = InputCat(node_start=0, num_nodes=ninp, num_cats=K, var=var,
                   row=np.arange(ninp, dtype=np.int32), param_offset=0, num_rows=ninp)
    layers.append(inp)
    pcur = ninp * K
    nxt = ninp
    # scope -> list of block start node ids
    scopes = {(v,): [v * in_blocks * block + i * block for i in range(in_blocks)]
              for v in range(num_vars)}

    def sum_layer(blocks_in, n_out_blocks, out_block):
        nonlocal nxt, pcur
        groups = []
        outs = []
        for ob in range(n_out_blocks):
            mask = rng.random(len(blocks_in)) < density
            if not mask.any():
                mask[rng.integers(len(blocks_in))] = True
            chosen = np.array(blocks_in, dtype=np.int32)[mask]
            groups.append(SumGroup(out_start=nxt, num_nodes=out_block,
                                   ch_block_start=chosen, ch_block_size=block,
                                   param_offset=pcur))
            outs.append(nxt)
            pcur += out_block * len(chosen) * block
            nxt += out_block
        layers.append(Sum(groups))
        return outs

    keys = list(scopes.keys())
    # one sum layer over the inputs of each variable
    new = {}
    for k in keys:
        new[k] = sum_layer(scopes[k], sum_blocks, block)
    scopes = new
    while len(scopes) > 1:
        keys = list(scopes.keys())
        rng.shuffle(keys)
        a, b = keys[0], keys[1]
        la, lb = scopes.pop(a), scopes.pop(b)
        n = min(len(la), len(lb))
        ptr = [0]
        ids = []
        start = nxt
        for i in range(n):
            for z in range(block):
                ids.extend([la[i] + z, lb[i] + z])
                ptr.append(len(ids))
        layers.append(Product(node_start=start, num_nodes=n * block,
                              ch_ptr=np.array(ptr, dtype=np.int32),
                              ch_ids=np.array(ids, dtype=np.int32)))
        nxt += n * block
        blocks = [start + i * block for i in range(n)]
        for _ in range(depth_sums):
            blocks = sum_layer(blocks, sum_blocks, block)
        scopes[tuple(sorted(a + b))] = blocks
    (last,) = scopes.values()
    root = nxt
    layers.append(Sum([SumGroup(out_start=root, num_nodes=1,
                                ch_block_start=np.array(last, dtype=np.int32),
                                ch_block_size=block, param_offset=pcur)]))
    pcur += len(last) * block
    nxt += 1
    c = Circuit(name=f"bsparse_s{seed}", num_nodes=nxt, num_vars=num_vars, num_params=pcur,
                layers=layers, root=root)
    c.meta = dict(kind="block_sparse", K=K)
    return c


def random_block_layer(seed: int, M_blocks: int, node_block: int, ch_blocks: int,
                       ch_block: int, density: float = 0.5) -> Circuit:
    """A lone block-sparse sum layer over external children (unnormalised
    structure, for layer-level parity): ``ch_blocks`` child blocks of
    ``ch_block`` nodes, ``M_blocks`` node blocks of ``node_block`` nodes, each
    connected to a random non-empty subset of the child blocks."""
    rng = np.random.default_rng(seed)
    Nt = ch_blocks * ch_block
    ext = InputExternal(node_start=0, num_nodes=Nt)
    groups = []
    nxt = Nt
    pcur = 0
    for _ in range(M_blocks):
        mask = rng.random(ch_blocks) < density
        if not mask.any():
            mask[rng.integers(ch_blocks)] = True
        chosen = (np.nonzero(mask)[0] * ch_block).astype(np.int32)
        rng.shuffle(chosen)
        groups.append(SumGroup(out_start=nxt, num_nodes=node_block, ch_block_start=chosen,
                               ch_block_size=ch_block, param_offset=pcur))
        pcur += node_block * len(chosen) * ch_block
        nxt += node_block
    c = Circuit(name=f"blocklayer_s{seed}", num_nodes=nxt, num_vars=0, num_params=pcur,
                layers=[ext, Sum(groups)], root=-1)
    c.meta = dict(kind="block_layer")
    return c


def pd(H: int, W: int, K: int, num_cats: int, split: int = 1) -> Circuit:
    """Poon-Domingos (PD) region-graph circuit over an H x W grid of
    categorical variables (variable r*W + c), with K latents per region.

    Regions are the axis-aligned rectangles whose edges lie on multiples of
    ``split`` (and on the grid's border); a region of one cell is a leaf.  A
    leaf cell of one pixel is K categorical input nodes with their own rows; a
    leaf cell of several pixels is K products of its pixels' input nodes
    (node k of every pixel).  Every way of cutting a region in two along a
    row or column line gives a product block of K nodes, node k adding node k
    of the two halves; the region's K sum nodes mix all of its product blocks
    (one sum group: node block K over a list of K-node child blocks, its own
    [K, splits*K] weights).  The full grid's region is one root sum node over
    its product blocks.  Sum and product layers are levelled by depth, so each
    sum layer holds many groups with different child-block lists (the general
    block-sparse layout).
    """
    ys = sorted(set(list(range(0, H, split)) + [H]))
    xs = sorted(set(list(range(0, W, split)) + [W]))
    regions = [(y0, y1, x0, x1) for i, y0 in enumerate(ys) for y1 in ys[i + 1:]
               for j, x0 in enumerate(xs) for x1 in xs[j + 1:]]
    # children before parents: by area, then position
    regions.sort(key=lambda r: ((r[1] - r[0]) * (r[3] - r[2]), r))
    nvar = H * W
    inp = InputCat(node_start=0, num_nodes=nvar * K, num_cats=num_cats,
                   var=np.repeat(np.arange(nvar, dtype=np.int32), K),
                   row=np.arange(nvar * K, dtype=np.int32), param_offset=0, num_rows=nvar * K)
    pcur = nvar * K * num_cats
    nxt = nvar * K
    block = {}     # region -> first node of its K-node block (value of the region)
    level = {}     # region -> sum level (leaf pixels: 0)
    prod_levels = {}   # level -> list of (first node placeholder, [child starts...]) filled later
    sum_levels = {}    # level -> list of (region, [product block ids])
    cell_prods = []    # leaf cells of several pixels: (region, [pixel input starts])
    leaf = lambda r: len([y for y in ys if r[0] < y < r[1]]) == 0 and len([x for x in xs if r[2] < x < r[3]]) == 0
    prod_blocks = []   # (level, child region a, child region b, owner region)
    for r in regions:
        y0, y1, x0, x1 = r
        if leaf(r):
            pix = [(y, x) for y in range(y0, y1) for x in range(x0, x1)]
            if len(pix) == 1:
                block[r] = (pix[0][0] * W + pix[0][1]) * K
                level[r] = 0
            else:
                cell_prods.append((r, [(y * W + x) * K for y, x in pix]))
                level[r] = 0
            continue
        cuts = [((y0, y, x0, x1), (y, y1, x0, x1)) for y in ys if y0 < y < y1] + \
               [((y0, y1, x0, x), (y0, y1, x, x1)) for x in xs if x0 < x < x1]
        lv = 1 + max(max(level[a], level[b]) for a, b in cuts)
        level[r] = lv
        for a, b in cuts:
            prod_blocks.append((lv, a, b, r))
    layers = [inp]
    # leaf cells of several pixels: one product layer before everything else
    if cell_prods:
        start = nxt
        ptr, ids = [0], []
        for r, pstarts in cell_prods:
            block[r] = nxt
            for k in range(K):
                ids.extend(s + k for s in pstarts)
                ptr.append(len(ids))
            nxt += K
        layers.append(Product(node_start=start, num_nodes=nxt - start,
                              ch_ptr=np.array(ptr, dtype=np.int32), ch_ids=np.array(ids, dtype=np.int32)))
    maxlv = max(level.values())
    full = (0, H, 0, W)
    for lv in range(1, maxlv + 1):
        # products of this level: node k of the block = node k of both halves
        owners = {}
        start = nxt
        ptr, ids = [0], []
        for (l, a, b, r) in prod_blocks:
            if l != lv:
                continue
            owners.setdefault(r, []).append(nxt)
            for k in range(K):
                ids.extend([block[a] + k, block[b] + k])
                ptr.append(len(ids))
            nxt += K
        if nxt > start:
            layers.append(Product(node_start=start, num_nodes=nxt - start,
                                  ch_ptr=np.array(ptr, dtype=np.int32), ch_ids=np.array(ids, dtype=np.int32)))
        groups = []
        for r in sorted(owners):
            M = 1 if r == full else K
            chs = np.array(owners[r], dtype=np.int32)
            groups.append(SumGroup(out_start=nxt, num_nodes=M, ch_block_start=chs, ch_block_size=K,
                                   param_offset=pcur))
            block[r] = nxt
            pcur += M * len(chs) * K
            nxt += M
        if groups:
            layers.append(Sum(groups))
    root = block[full]
    c = Circuit(name=f"pd{H}x{W}k{K}c{num_cats}s{split}", num_nodes=nxt, num_vars=nvar, num_params=pcur,
                layers=layers, root=root)
    c.meta = dict(kind="pd", H=H, W=W, K=K, num_cats=num_cats, split=split, regions=len(regions),
                  product_blocks=len(prod_blocks))
    return c
