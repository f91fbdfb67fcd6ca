"""GPU parity: the HIP path through the C ABI against the float64 oracle,
element by element, in both precision modes, on the synthetic workloads and
their edge cases (ragged sizes, -inf columns, batches around the small-batch
rule, overlapping block-sparse children, tied weights)."""
import numpy as np
import pytest

from tests import gpu_util as G
from workloads import make_config

pytestmark = pytest.mark.gpu

MODES = ["auto", "fp32"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import log_space_sum_amd as L
    L.lib()          # fails loudly when libpc.so is missing


def _full(cfg, mode, what, em=None, options=None):
    """Values and log-likelihood end to end at the stated tolerances; element
    and parameter flows per layer (each layer's flows recomputed by the
    oracle from that layer's GPU inputs) at the stated tolerances; flows end
    to end at the stated tolerance in auto mode and at the stated tolerance
    plus the float32-storage term in fp32-level mode (gpu_util.e2e_flow_tol)."""
    G.say(f"case {what} mode={mode} B={cfg['B']}")
    gpu = G.run_gpu(cfg, mode, em=em, options=options)
    orc = G.run_oracle(cfg)
    G.check_values(gpu["vals"], orc["vals"], mode, f"{what} node values")
    if orc["ll"] is not None:
        G.check_values(gpu["ll"], orc["ll"], mode, f"{what} log-likelihood")
    G.check_local(cfg, gpu, mode, what)
    tol = G.e2e_flow_tol(cfg["circuit"], orc["vals"], mode)
    G.check_flows(gpu["flows"], orc["flows"], mode, f"{what} element flows end to end", rtol=tol)
    G.check_flows(gpu["pflows"], orc["pflows"], mode, f"{what} parameter flows end to end", rtol=tol)
    return gpu, orc


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,N,groups,B", [(200, 136, 1, 37), (96, 160, 3, 48), (1024, 1024, 1, 128)])
def test_dense_layer(mode, M, N, groups, B):
    cfg = make_config("dense_layer", M=M, N=N, groups=groups, B=B)
    _full(cfg, mode, f"dense {M}x{N} g{groups}")


@pytest.mark.parametrize("mode", MODES)
def test_dense_edge_columns(mode):
    """Per-group column-maximum edge cases: all-(-inf) column, single finite
    child, far-shifted columns, zero weights."""
    cfg = make_config("dense_layer", M=70, N=90, groups=2, B=20)
    ext = cfg["external"]
    ext[:90, 0] = -np.inf
    ext[:, 1] = -np.inf
    ext[7, 1] = -2.0
    ext[:, 2] -= 1e4
    ext[:, 3] += 80.0
    cfg["params"][5:40] = 0.0
    _full(cfg, mode, "dense edge columns")


@pytest.mark.parametrize("B", [1, 15, 16, 17])
def test_small_batches(B):
    """Batches below 16 run fp32-level products even in auto mode."""
    cfg = make_config("dense_layer", M=130, N=70, groups=1, B=B)
    gpu, orc = _full(cfg, "fp32" if B < 16 else "auto", f"dense small batch B={B}")
    if B < 16:
        gpu_auto = G.run_gpu(cfg, "auto")
        np.testing.assert_array_equal(gpu_auto["vals"], gpu["vals"])


@pytest.mark.parametrize("mode", ["fp32"])
def test_tiny_hmm(mode):
    cfg = make_config("tiny_hmm")
    _full(cfg, mode, "tiny hmm", em=(1.0, 0.0))


@pytest.mark.parametrize("mode", MODES)
def test_hmm_medium(mode):
    cfg = make_config("hmm4096", H=320, T=7, V=50, B=70)
    gpu, orc = _full(cfg, mode, "hmm 320x7")
    # EM step
    newp_or = __import__("oracle").em_step(cfg["circuit"], cfg["params"], orc["pflows"])
    gpu2 = G.run_gpu(cfg, mode, em=(1.0, 0.0))
    G.check_flows(gpu2["em"], newp_or, mode, "hmm EM parameters")


@pytest.mark.parametrize("step,pseudo", [(1.0, 0.0), (0.6, 0.0), (1.0, 0.2)])
def test_em_rows_without_flow(step, pseudo):
    """EM on parameter flows whose every other row is zero: without a
    pseudocount such rows keep their weights (also under a plain step of 1,
    which writes the other rows without reading the old weights); with one
    they move toward the uniform row."""
    import torch
    import log_space_sum_amd as L
    cfg = make_config("hmm4096", H=96, T=3, V=40, B=16)
    circ = cfg["circuit"]
    G.say(f"case EM rows without flow: step={step} pseudocount={pseudo}")
    h = L.pc_compile_layout(circ, device=0)
    rng = np.random.default_rng(5)
    F = rng.uniform(0.0, 2.0, size=circ.num_params)
    for off, nrows, rlen in circ.param_row_segments():
        F[off:off + nrows * rlen].reshape(nrows, rlen)[::2] = 0.0
    F = F.astype(np.float32)
    params = torch.tensor(cfg["params"], device="cuda")
    pflows = torch.tensor(F, device="cuda")
    L.pc_em_step(h, params, pflows, step, pseudo, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    ref = __import__("oracle").em_step(circ, cfg["params"], F.astype(np.float64),
                                       step_size=step, pseudocount=pseudo)
    G.check_flows(params.cpu().numpy(), ref, "fp32", "EM with rows without flow")
    if pseudo == 0.0:
        kept = np.zeros(circ.num_params, dtype=bool)
        for off, nrows, rlen in circ.param_row_segments():
            kept[off:off + nrows * rlen].reshape(nrows, rlen)[::2] = True
        np.testing.assert_array_equal(params.cpu().numpy()[kept], cfg["params"][kept])


@pytest.mark.parametrize("mode", MODES)
def test_em_pseudocount(mode):
    cfg = make_config("hmm4096", H=64, T=5, V=20, B=32)
    gpu = G.run_gpu(cfg, mode, em=(0.7, 0.3))
    orc = G.run_oracle(cfg)
    ref = __import__("oracle").em_step(cfg["circuit"], cfg["params"], gpu["pflows"].astype(np.float64),
                                       step_size=0.7, pseudocount=0.3)
    G.check_flows(gpu["em"], ref, "fp32", "EM blend + pseudocount")
    G.check_flows(gpu["pflows"], orc["pflows"], mode, "parameter flows")


@pytest.mark.parametrize("mode", MODES)
def test_hclt_small(mode):
    cfg = make_config("hclt", num_vars=30, H=48, K=12, B=33)
    _full(cfg, mode, "hclt 30x48")


@pytest.mark.parametrize("tile", [0, 1])
@pytest.mark.parametrize("mode", MODES)
def test_hclt_wide_level_tiles(mode, tile):
    """A strided level with many product tiles per CU (at least 4 x 256
    128 x 128 tiles: 69 groups x 2 row tiles x 8 column tiles at batch 1024)
    next to narrow levels, in one pass, on the automatic tiles and on
    128 x 128 tiles (layer_tile 1)."""
    cfg = make_config("hclt", num_vars=180, H=256, K=16, B=1024)
    widths = [len(ly.groups) * 2 * (cfg["B"] // 128) for ly in cfg["circuit"].layers if type(ly).__name__ == "Sum"]
    assert max(widths) >= 1024 and min(widths) < 1024
    _full(cfg, mode, f"hclt 180x256 wide level, layer tile {tile}", options=[("layer_tile", tile)])


@pytest.mark.parametrize("mode", MODES)
def test_hclt_multi_unit_groups(mode):
    """Evenly strided (batched) layers whose groups span two 256-row units
    (320 latents per variable) in layers of several groups, with a ragged
    batch: the per-group tile addressing past a group's first unit."""
    import log_space_sum_amd as L
    cfg = make_config("hclt", num_vars=40, H=320, K=16, B=300)
    circ = cfg["circuit"]
    h = L.pc_compile_layout(circ, device=-1)
    strided = [i for i, ly in enumerate(circ.layers)
               if type(ly).__name__ == "Sum" and L.pc_layer_class(h, i) == L.PC_CLASS_STRIDED]
    assert any(len(circ.layers[i].groups) >= 3 for i in strided), "no multi-group strided layer"
    _full(cfg, mode, "hclt 40x320")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("what,cfg_args", [
    # node blocks of 16, every pixel a leaf, a full batch of 512
    ("pd 6x6 k16", dict(name="pd", H=6, W=6, K=16, C=8, split=1, B=512)),
    # node blocks of 32, leaf cells of 2 x 2 pixels, ragged batch
    ("pd 8x8 k32", dict(name="pd", H=8, W=8, K=32, C=16, split=2, B=37)),
    # node blocks of 128 over 4-pixel leaf cells
    ("pd 12x12 k128", dict(name="pd", H=12, W=12, K=128, C=4, split=4, B=64)),
    # the measured PD workload at its own size
    ("pd 28x28 k64", dict(name="pd")),
])
def test_pd(what, cfg_args, mode):
    """Poon-Domingos region-graph circuits: general block-sparse sum layers
    whose groups (one per region) mix lists of K-node product blocks."""
    import log_space_sum_amd as L
    cfg = make_config(**cfg_args)
    circ = cfg["circuit"]
    h = L.pc_compile_layout(circ, device=-1)
    cls = {L.pc_layer_class(h, i) for i, ly in enumerate(circ.layers) if type(ly).__name__ == "Sum"}
    assert L.PC_CLASS_GENERAL in cls, cls
    _full(cfg, mode, what)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("seed", [0, 1])
def test_block_sparse_layer(mode, seed):
    cfg = make_config(kind="block_layer", seed=seed, M_blocks=9, node_block=48, ch_blocks=7,
                      ch_block=40, B=41, spread_hi=20.0)
    _full(cfg, mode, f"block layer s{seed}")


@pytest.mark.parametrize("mode", MODES)
def test_block_sparse_circuit(mode):
    cfg = make_config(kind="block_sparse", seed=2, num_vars=6, K=5, in_blocks=3, block=24,
                      sum_blocks=3, depth_sums=2, B=29)
    _full(cfg, mode, "block-sparse circuit")


@pytest.mark.parametrize("what,cfg_args,mode", [
    ("block layer", dict(kind="block_layer", seed=4, M_blocks=6, node_block=40, ch_blocks=5, ch_block=32, B=33),
     "auto"),
    # wide strided level with the weights in registers (a wait that counted
    # loads of both kinds made these flows differ from run to run)
    ("hclt 180x256 wide level", dict(name="hclt", num_vars=180, H=256, K=16, B=1024), "fp32"),
    ("hclt 180x256 wide level", dict(name="hclt", num_vars=180, H=256, K=16, B=1024), "auto"),
    # K split over four workgroups (batch 128)
    ("hmm 1024x6", dict(name="hmm4096", H=1024, T=6, B=128), "auto"),
])
def test_deterministic(what, cfg_args, mode):
    """Three runs give bitwise identical values, flows and parameter flows."""
    args = dict(cfg_args)
    cfg = make_config(args.pop("name", None), **args)
    G.say(f"case determinism {what} mode={mode} B={cfg['B']}")
    r = G.run_gpu(cfg, mode, repeat=3)
    for k in ("vals", "flows", "pflows"):
        for i in (1, 2):
            np.testing.assert_array_equal(r[0][k], r[i][k], err_msg=f"{what}: {k}, run {i} vs run 0")


@pytest.mark.parametrize("kind", ["fwd", "elem", "param"])
def test_fp32_needs_split(kind):
    """Downgrading any one of the three products of the fp32-level mode to a
    single bf16 term breaks the fp32-level tolerance."""
    cfg = make_config("dense_layer", M=256, N=256, groups=1, B=64)
    gpu = G.run_gpu(cfg, "fp32", splits=[("fp32", kind, 1, 1)])
    orc = G.run_oracle(cfg)
    errs = []
    for (what, fn, a, b) in [("vals", G.check_values, gpu["vals"], orc["vals"]),
                             ("flows", G.check_flows, gpu["flows"], orc["flows"]),
                             ("pflows", G.check_flows, gpu["pflows"], orc["pflows"])]:
        try:
            fn(a, b, "fp32", f"downgraded {kind}: {what}")
        except AssertionError as e:
            errs.append(str(e))
    assert errs, f"a 1-term {kind} product still met the fp32-level tolerance"


@pytest.mark.parametrize("what,cfg_args,mode,all_fused", [
    ("hmm", dict(name="hmm4096", H=320, T=7, V=50, B=70), "auto", True),
    ("hmm ragged batch", dict(name="hmm4096", H=96, T=4, V=11, B=23), "fp32", True),
    # batches of multiples of 64: the element-flow products also pack the
    # next layer's scaled flows (at 320 and 192 the last 128-sample column
    # tile is half padding)
    ("hmm batch 256", dict(name="hmm4096", H=320, T=6, V=50, B=256), "auto", True),
    ("hmm batch 320", dict(name="hmm4096", H=320, T=6, V=50, B=320), "auto", True),
    ("hmm batch 192", dict(name="hmm4096", H=128, T=5, V=20, B=192), "fp32", True),
    ("hmm batch 512", dict(name="hmm4096", H=128, T=5, V=20, B=512), "fp32", True),
    ("hclt", dict(name="hclt", num_vars=30, H=48, K=12, B=33), "auto", False),
    ("block-sparse", dict(kind="block_sparse", seed=2, num_vars=6, K=5, in_blocks=3, block=24,
                          sum_blocks=3, depth_sums=2, B=29), "auto", False),
    ("lowrank hmm", dict(name="lowrank", H=40, T=4, V=7, B=23, rank=5), "auto", True),
])
def test_fused_product_layers_identical(what, cfg_args, mode, all_fused):
    """Product layers evaluated inside the adjacent sum layers' column-max and
    scaled-flow kernels give the same bits as their own launches: values,
    log-likelihoods, flows and parameter flows (and LowRank gradients)."""
    cfg = make_config(**cfg_args)
    G.say(f"case fused product layers: {what} mode={mode} B={cfg['B']}")
    fused = G.run_gpu(cfg, mode, timing=True)
    plain = G.run_gpu(cfg, mode, timing=True, options=[("fuse", 0)])
    for k in ("vals", "ll", "flows", "pflows"):
        if fused[k] is not None:
            np.testing.assert_array_equal(fused[k], plain[k], err_msg=f"{what}: {k}")
    for k in ("dA", "dB"):
        for x, y in zip(fused.get(k, []), plain.get(k, [])):
            np.testing.assert_array_equal(x, y, err_msg=f"{what}: {k}")
    tf, tp = fused["times"], plain["times"]
    G.say(f"  launches fused/plain: product fwd {tf['product_fwd'][0]}/{tp['product_fwd'][0]}, "
          f"product bwd {tf['product_bwd'][0]}/{tp['product_bwd'][0]}")
    assert tp["product_fwd"][0] > 0 and tp["product_bwd"][0] > 0
    if all_fused:   # every product layer of an HMM (LowRank or not) sits between two sum layers
        assert tf["product_fwd"][0] == 0 and tf["product_bwd"][0] == 0
    if all_fused and cfg["B"] % 64 == 0:
        # every sum layer below a product layer is packed by the layer above
        G.say(f"  scaled-flow launches fused/plain: {tf['scaled_flows'][0]}/{tp['scaled_flows'][0]}")
        assert tf["scaled_flows"][0] < tp["scaled_flows"][0]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("H,T,V,B,skew", [(96, 6, 37, 264, 0.0), (64, 5, 500, 512, 0.5), (80, 4, 512, 256, 0.9)])
def test_input_rows_of_several_nodes(mode, H, T, V, B, skew):
    """Input-layer parameter flows of rows shared by several nodes (an HMM's
    emission row of a hidden state, one node per position) at the batches
    taken one row per wave (256 to 512 samples, a multiple of 8), with
    uniform categories and with one large bucket per variable."""
    cfg = make_config("hmm4096", H=H, T=T, V=V, B=B, skew=skew)
    _full(cfg, mode, f"hmm {H}x{T} V={V} skew={skew} input rows")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("tile", [1, 2, 3, 4, 5])
def test_layer_tile_options(tile, mode):
    """Every per-layer product tile shape (128x128, 256x128, 128x256, 128x64, 64x128)
    meets the tolerances; a batch of 300 leaves a ragged last column tile."""
    cfg = make_config("hmm4096", H=320, T=5, V=50, B=300)
    _full(cfg, mode, f"hmm 320x5 layer tile {tile}", options=[("layer_tile", tile)])


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("tile", [1, 2, 3])
@pytest.mark.parametrize("what,cfg_args", [
    ("hmm", dict(name="hmm4096", H=320, T=5, V=50, B=300)),
    ("hclt", dict(name="hclt", num_vars=30, H=48, K=12, B=33)),
])
def test_param_tile_options(what, cfg_args, tile, mode):
    """Every parameter-flow tile shape (128x128, 256x256 where the operand
    split allows it, 128x256) meets the tolerances, on one tied block (HMM)
    and on many blocks (HCLT)."""
    cfg = make_config(**cfg_args)
    _full(cfg, mode, f"{what} param tile {tile}", options=[("param_tile", tile)])


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("what,cfg_args,chunk", [
    ("hmm", dict(name="hmm4096", H=320, T=7, V=50, B=70), 1),
    ("hmm", dict(name="hmm4096", H=320, T=7, V=50, B=70), 4),
    ("block-sparse", dict(kind="block_sparse", seed=2, num_vars=6, K=5, in_blocks=3, block=24,
                          sum_blocks=3, depth_sums=2, B=29), 2),
    ("hclt", dict(name="hclt", num_vars=30, H=48, K=12, B=33), 3),
])
def test_param_flow_chunks(what, cfg_args, chunk, mode):
    """Parameter flows in chunks of tied copies on the handle's second stream
    meet the tolerances, and repeat bit for bit."""
    cfg = make_config(**cfg_args)
    opts = [("param_chunk", chunk)]
    gpu, orc = _full(cfg, mode, f"{what} parameter flows in chunks of {chunk}", options=opts)
    again = G.run_gpu(cfg, mode, options=opts)
    np.testing.assert_array_equal(gpu["pflows"], again["pflows"])
    np.testing.assert_array_equal(gpu["flows"], again["flows"])


@pytest.mark.parametrize("what,cfg_args", [
    ("hmm", dict(name="hmm4096", H=320, T=7, V=50, B=70)),                      # tied: one chunk per block
    ("hclt", dict(name="hclt", num_vars=30, H=48, K=12, B=33)),                 # many blocks: one product
])
def test_param_flow_automatic_chunks_agree(what, cfg_args):
    """The automatic choice (one chunk of all copies per block on the second
    stream, or the single product after the layers) agrees with the single
    product to float32 summation order (the two launch groupings can split
    K differently), and repeats bit for bit."""
    cfg = make_config(**cfg_args)
    G.say(f"case automatic parameter-flow chunks: {what} B={cfg['B']}")
    auto = G.run_gpu(cfg, "auto")
    again = G.run_gpu(cfg, "auto")
    single = G.run_gpu(cfg, "auto", options=[("param_chunk", 0)])
    np.testing.assert_array_equal(auto["pflows"], again["pflows"], err_msg=f"{what}: parameter flows repeat")
    np.testing.assert_array_equal(auto["flows"], single["flows"], err_msg=f"{what}: flows")
    G.check_flows(auto["pflows"], single["pflows"].astype(np.float64), "fp32",
                  f"{what}: automatic chunks vs the single product", rtol=1e-6)
