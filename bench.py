"""Benchmark: one pass of the sum-layer hot path on the HMM workload.

Workload: HMM with 4096 latent states, 32 positions, 512 symbols, batch 512
(tied 4096 x 4096 transition, softmax(N(0,1)) rows, uniform tokens; seeded
synthetic data).  A step = forward (input layer, 31 shared-children sum
layers, products, root) + backward (element flows, parameter flows) + EM
update, all through the C ABI on one GPU, inputs resident in HBM.

Prints one JSON line.  `value` is the sum layers' algorithmic throughput:
3 products (forward, element flows, parameter flows) x 2*M*N*B flops per sum
group, divided by the whole step's wall time.  The roofline object describes
the dominant kernel: algorithmic flops per launch over its mean launch time
(in a second timed pass over the same number of steps, every kernel is
launched with a HIP event pair that its own dispatch packet stamps at the
kernel's start and end, on the stream it runs on), against the bf16 dense MFMA
peak of MI355X.
The CPU baseline times the float64 oracle on a bounded sample of the same
workload (a subset of the batch) on the host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 matrix peak
PEAK_HBM_GBS = 8000.0


def sum_flops(circ, B):
    """Algorithmic flops of the sum layers per pass (3 products each)."""
    tot = 0
    per_kind = 0
    for layer in circ.layers:
        if type(layer).__name__ == "Sum":
            for g in layer.groups:
                tot += 3 * 2 * g.num_nodes * g.num_children * B
    return tot


def kernel_traffic(kernel_kind):
    """HBM bytes per launch of `kernel_kind` from the committed counter
    summary (profiles/traffic_<kind>.json), if it was taken on the current
    source of the kernel's file; else None."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_kind}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    src = os.path.join(ROOT, rec.get("source_file", "log_space_sum_amd/csrc/k_gemm.hip"))
    sha = hashlib.sha256(open(src, "rb").read()).hexdigest()
    if rec.get("source_sha256") != sha:
        return None
    return rec["bytes_per_launch"]


def cpu_baseline(cfg, sample_B, min_s=10.0, max_passes=100000):
    """The float64 oracle (as it stands) on the first `sample_B` samples,
    repeated (at most `max_passes` passes) until `min_s` seconds have passed;
    the rate is per pass."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # noqa: BLE001
        threads = os.cpu_count()
    circ = cfg["circuit"]
    p = cfg["params"].astype(np.float64)
    tok = cfg["tokens"][:sample_B] if cfg.get("tokens") is not None else None
    ext = cfg["external"][:, :sample_B] if cfg.get("external") is not None else None
    seeds = cfg["seed_flows"][:, :sample_B] if cfg.get("seed_flows") is not None else None
    t0 = time.perf_counter()
    passes = 0
    while passes < max_passes and (passes == 0 or time.perf_counter() - t0 < min_s):
        V, ll = oracle.forward(circ, p, sample_B, tokens=tok, external=ext)
        oracle.backward(circ, p, V, tokens=tok, seed_flows=seeds)
        passes += 1
    total = time.perf_counter() - t0
    dt = total / passes
    fl = sum_flops(circ, sample_B)
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"float64 oracle forward+backward on {sample_B} of the {cfg['B']} samples "
                      f"(the whole circuit), {passes} pass(es) in {total:.2f} s; sum-layer algorithmic "
                      f"flops per pass / time per pass",
            "seconds": total}


# MI355X exp rate: 256 CUs x 4 SIMDs x 16 lanes = 16384 fp32 lane operations
# per clock; CDNA4 issues transcendentals (v_exp_f32) at half that rate, so
# 8192 exps per clock x 2.4 GHz = 19.66 T exp/s.  (A probe of independent exp
# chains measured 13.0 T exp/s next to 52 T packed FMA/s = 26 T FMA issue/s:
# the same 1:2 ratio at a 1.6 GHz clock under load.)
PEAK_EXP_G = 19660.0


def bench_lowrank(args):
    """The LowRank exp_sum workload: HMM 1024 states x 64 positions, 512
    symbols, rank 16, batch 64, a (A, B) factor pair per position copy.  A step
    is forward + backward (+ dLL/dA, dLL/dB) + EM.  The fused kernels are
    bound by the exp rate: one exp per (sample, node, child) in the forward
    and one in the backward's recomputation."""
    import torch
    import log_space_sum_amd as L
    from workloads import make_config
    cfg = make_config("lowrank", form=args.lowrank_form)
    circ, B = cfg["circuit"], cfg["B"]
    dev = "cuda:0"
    h = L.pc_compile_layout(circ, device=0)
    L.pc_set_precision(h, args.mode)
    L.pc_set_option(h, "lr_pack", args.lr_pack)
    L.pc_set_option(h, "flow_fp8", args.flow_fp8)
    params = torch.tensor(cfg["params"], device=dev)
    tokens = torch.tensor(cfg["tokens"], device=dev)
    vals = torch.empty((circ.num_nodes, B), device=dev)
    flows = torch.empty((circ.num_nodes, B), device=dev)
    pflows = torch.zeros(circ.num_params, device=dev)
    ll = torch.empty(B, device=dev)
    lr = [(torch.tensor(a, device=dev), torch.tensor(b, device=dev)) for a, b in cfg["lowrank"]]
    grads = [(torch.empty_like(a), torch.empty_like(b)) for a, b in lr]
    ws = L.workspace(h, B, dev)
    stream = torch.cuda.current_stream()
    # with --z-correction: the denominator statistic and the conditional M-step
    zf = torch.zeros(circ.num_params, device=dev) if args.z_correction else None

    def step():
        pflows.zero_()
        L.pc_forward(h, B, tokens, params, vals, ll, lr, ws, stream.cuda_stream)
        if zf is None:
            L.pc_backward(h, B, tokens, params, vals, flows, pflows, 0, lr, grads, ws, stream.cuda_stream)
            L.pc_em_step(h, params, pflows, 1.0, 0.0, stream.cuda_stream)
        else:
            zf.zero_()
            L.pc_backward(h, B, tokens, params, vals, flows, pflows, 0, lr, grads, ws, stream.cuda_stream,
                          z_flows=zf)
            L.pc_em_step_corrected(h, params, pflows, zf, 1.0, 0.0, stream.cuda_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    run = step
    if args.graph and zf is None:
        g = L.StepGraph(h, B, tokens, params, vals, flows, pflows, ll, 0, lowrank=lr, grads=grads, ws=ws,
                        em=(1.0, 0.0))
        run = g.replay
        run()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / args.steps * 1e3
    L.pc_set_timing(h, True)
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = L.pc_kernel_times(h)
    L.pc_set_timing(h, False)
    pairs_per_sample = sum(g.num_nodes * g.num_children for ly in circ.layers if type(ly).__name__ == "Sum"
                           for g in ly.groups if g.lowrank >= 0)
    pairs = B * pairs_per_sample                       # (sample, node, child) triples per pass
    exps = 2 * pairs                                   # forward + backward recomputation
    value = exps / (ms * 1e-3) / 1e9
    if args.lowrank_form == "sum_exp":
        # the virtual-batch products with the shared weights dominate: per
        # LowRank group one forward product theta [X | C]^T and one backward
        # product theta^T [Y1 | Y2]^T, 2 * M * N * (2 B k) flops each
        rank = int(cfg["cfg"]["rank"])
        kind_flops = {"sum_fwd_gemm": 4 * pairs * rank, "elem_flow_gemm": 4 * pairs * rank}
        dom = max(kind_flops, key=lambda k: kt[k][1])
        n_launch, tot_ms = kt[dom]
        avg_ms = tot_ms / max(n_launch, 1)
        per_launch = kind_flops[dom] * args.steps / max(n_launch, 1)
        roofline = {"kernel": dom, "bound": "mfma", "achieved": round(per_launch / (avg_ms * 1e-3) / 1e12, 3),
                    "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(per_launch / (avg_ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
                    "traffic": kernel_traffic("lowrank_" + dom), "per_launch_gflop": round(per_launch / 1e9, 4),
                    "avg_launch_ms": round(avg_ms, 5)}
    else:
        dom = max(("lowrank_fwd", "lowrank_bwd", "lowrank_coef"), key=lambda k: kt[k][1])
        n_launch, tot_ms = kt[dom]
        per_launch_exps = pairs * args.steps / max(n_launch, 1)
        avg_ms = tot_ms / max(n_launch, 1)
        achieved = per_launch_exps / (avg_ms * 1e-3) / 1e9
        roofline = {"kernel": dom, "bound": "alu", "achieved": round(achieved, 2), "peak": PEAK_EXP_G,
                    "unit": "Gexp/s", "frac": round(achieved / PEAK_EXP_G, 4), "traffic": kernel_traffic(dom),
                    "avg_launch_ms": round(avg_ms, 5)}
    out = {
        "metric": f"LowRank {args.lowrank_form} fwd+bwd exp throughput, HMM 1024 lat x 64 pos, rank 16, batch 64",
        "value": round(value, 2), "unit": "Gexp/s", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16-split" if args.mode == "auto" else "bf16x6-split", "data": "synthetic",
        "config": {"workload": f"lowrank {args.lowrank_form} hmm1024x64 symbols 512 rank 16 batch 64 fwd+bwd+em"
                               + (" (z-corrected)" if args.z_correction else "")
                               + (" (fp8 end products)" if args.flow_fp8 and args.lowrank_form == "sum_exp" else ""),
                   "precision_mode": args.mode,
                   "hip_graph": bool(args.graph and zf is None),
                   "global_batch": B},
        "kernel_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in kt.items() if v[0]},
        "roofline": roofline,
    }
    if not args.no_cpu:
        import numpy as np
        import oracle
        try:
            from threadpoolctl import threadpool_info
            threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
        except Exception:  # noqa: BLE001
            threads = os.cpu_count()
        sb = min(args.lr_cpu_sample, B)   # about 10-20 s on a 16-core host
        p = cfg["params"].astype(np.float64)
        lrs = [(a[:sb], b[:sb]) for a, b in cfg["lowrank"]]
        t0 = time.perf_counter()
        V, _ = oracle.forward(circ, p, sb, tokens=cfg["tokens"][:sb], lowrank=lrs)
        oracle.backward(circ, p, V, tokens=cfg["tokens"][:sb], lowrank=lrs)
        dt = time.perf_counter() - t0
        out["cpu_baseline"] = {"value": round(2 * pairs_per_sample * sb / dt / 1e9, 4),
                               "unit": "Gexp/s", "cores": int(threads), "kind": "oracle",
                               "sample": f"float64 oracle forward+backward on {sb} of the {B} samples, {dt:.1f} s"}
    print(json.dumps(out))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="hmm4096", choices=["hmm4096", "lowrank", "hclt", "dense", "pd"],
                    help="hmm4096: the metric's workload (default); lowrank: the LowRank exp_sum HMM "
                         "(1024 states, 64 positions, rank 16, batch 64); hclt: the HCLT-like circuit (768 "
                         "variables x 1024 latents x 512 categories, batch 512); dense: one 1024 x 1024 dense "
                         "layer over external children, batch 128; pd: a Poon-Domingos region graph over a 28 x 28 "
                         "grid of 256-category variables (4-pixel region lattice, 64 latents per region), batch 128")
    ap.add_argument("--mode", default="auto", choices=["auto", "fp32"])
    ap.add_argument("--batch", type=int, default=None, help="batch (default: the workload's)")
    ap.add_argument("--H", type=int, default=4096)
    ap.add_argument("--T", type=int, default=32)
    ap.add_argument("--cpu-sample", type=int, default=512,
                    help="samples of the batch the float64 oracle baseline runs on (the default, the whole "
                         "batch of 512, is about 10-20 s on a 16-core host)")
    ap.add_argument("--cpu-sample-other", type=int, default=None,
                    help="samples the oracle baseline of the hclt / dense workloads runs on "
                         "(default: 8 for hclt, the whole batch for dense)")
    ap.add_argument("--lr-cpu-sample", type=int, default=24,
                    help="samples of the LowRank workload the oracle baseline runs on")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--lowrank-form", default="exp_sum", choices=["exp_sum", "sum_exp"],
                    help="LowRank workload: how the factors make the scale")
    ap.add_argument("--z-correction", type=int, default=0, choices=[0, 1],
                    help="LowRank workload: also accumulate the denominator statistic W and take the conditional M-step")
    ap.add_argument("--flow-fp8", type=int, default=0, choices=[0, 1],
                    help="LowRank sum_exp: parameter flows and W from e4m3 operands (auto mode)")
    ap.add_argument("--graph", type=int, default=0, choices=[0, 1],
                    help="time replays of the step recorded as a HIP graph (1) or eager launches (0; measured the same: the queue already runs ahead of the host)")
    ap.add_argument("--layer-tile", type=int, default=0, help="product-kernel option: 0 auto, 1 128x128, 2 256x128, 3 128x256, 4 128x64, 5 64x128")
    ap.add_argument("--param-tile", type=int, default=0, help="product-kernel option: 0 auto, 1 128x128, 2 256x256, 3 128x256")
    ap.add_argument("--split-max", type=int, default=8, help="largest K split of a per-layer product")
    ap.add_argument("--param-chunk", type=int, default=-1,
                    help="tied copies per parameter-flow launch on a second stream (-1: automatic, 0: one launch at the end)")
    ap.add_argument("--lr-pack", type=int, default=0, choices=[0, 1],
                    help="LowRank factor records: 0 made once per forward, 1 per layer and pass")
    ap.add_argument("--splits", default="",
                    help="operand splits of the current mode, e.g. 'fwd=2,2;elem=2,1' (product kind = planes of "
                         "the first, second operand; default: the library's)")
    ap.add_argument("--fuse", type=int, default=1, choices=[0, 1],
                    help="1: product layers inside the adjacent sum layers' memory-bound kernels; 0: own launches")
    ap.add_argument("--copy-calibration", type=int, default=0,
                    help="only run a plain device copy of this many bytes (3 times): the reference "
                         "dispatch for scaling FETCH_SIZE / WRITE_SIZE counters to bytes")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: the library has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    if args.copy_calibration:
        n = args.copy_calibration // 4
        src = torch.ones(n, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n * 4}))
        return

    import log_space_sum_amd as L
    from workloads import make_config

    if args.workload == "lowrank":
        return bench_lowrank(args)
    bsz = {} if args.batch is None else {"B": args.batch}
    if args.workload == "hmm4096":
        cfg = make_config("hmm4096", H=args.H, T=args.T, **bsz)
        metric = (f"sum-layer fwd+bwd ms & TFLOP/s (frac of MFMA peak), HMM {args.H} lat×{args.T} pos, "
                  f"batch {cfg['B']}")
        workload = f"hmm{args.H}x{args.T} symbols 512 batch {cfg['B']} fwd+bwd+em"
        context = "pages (RTX PRO 6000, whole circuit, auto): 32.1 ms fwd+bwd at batch 512"
    elif args.workload == "hclt":
        print("building the HCLT workload (768 variables x 1024 latents, 512 categories; about a minute)",
              file=sys.stderr, flush=True)
        cfg = make_config("hclt", **bsz)
        metric = "sum-layer fwd+bwd TFLOP/s (frac of MFMA peak), HCLT 768 vars x 1024 latents x 512 cats"
        workload = f"hclt 768 vars x 1024 latents x 512 categories, random tree, batch {cfg['B']} fwd+bwd+em"
        context = "pages (RTX PRO 6000, whole circuit, auto): 48.1 ms fwd+bwd at batch 512"
    elif args.workload == "pd":
        cfg = make_config("pd", **bsz)
        metric = ("sum-layer fwd+bwd TFLOP/s (frac of MFMA peak), PD 28x28 grid x 256 cats, 4-pixel regions, "
                  f"64 latents, batch {cfg['B']}")
        workload = (f"pd 28x28 grid, 256 categories, region lattice 4, 64 latents per region, batch {cfg['B']} "
                    "fwd+bwd+em")
        context = "pages: PD layouts are not taken by the dense path (forward and fwd+bwd x1.00)"
    else:
        cfg = make_config("dense_layer", **bsz)
        metric = "sum-layer fwd+bwd TFLOP/s (frac of MFMA peak), one dense 1024x1024 layer"
        workload = f"dense layer 1024 nodes x 1024 shared children, batch {cfg['B']} fwd+bwd+em"
        context = None
    return bench_circuit(args, cfg, metric, workload, context)


def bench_circuit(args, cfg, metric, workload, context):
    """One forward + backward + EM per step on a plain (non-LowRank) circuit;
    `value` = the sum layers' algorithmic TFLOP/s over the step's wall time."""
    import torch
    import log_space_sum_amd as L
    circ, B = cfg["circuit"], cfg["B"]
    dev = "cuda:0"
    h = L.pc_compile_layout(circ, device=0)
    L.pc_set_precision(h, args.mode)
    L.pc_set_option(h, "layer_tile", args.layer_tile)
    L.pc_set_option(h, "param_tile", args.param_tile)
    L.pc_set_option(h, "split_max", args.split_max)
    L.pc_set_option(h, "fuse", args.fuse)
    L.pc_set_option(h, "param_chunk", args.param_chunk)
    for item in filter(None, args.splits.split(";")):
        kind, planes = item.split("=")
        pa, pb = (int(x) for x in planes.split(","))
        L.pc_set_split(h, args.mode, kind.strip(), pa, pb)
    params = torch.tensor(cfg["params"], device=dev)
    tokens = torch.tensor(cfg["tokens"], device=dev) if cfg.get("tokens") is not None else None
    vals = torch.empty((circ.num_nodes, B), device=dev)
    flows = torch.empty((circ.num_nodes, B), device=dev)
    flags = 0
    ext = [l for l in circ.layers if type(l).__name__ == "InputExternal"]
    if ext:      # external child values (the dense layer), set once: the passes never write them
        rows = torch.cat([torch.arange(l.node_start, l.node_start + l.num_nodes) for l in ext]).to(dev)
        vals[rows] = torch.tensor(cfg["external"], device=dev)
    if cfg.get("seed_flows") is not None:   # incoming flows of the output nodes, set once
        flows[torch.tensor(circ.output_nodes(), device=dev)] = torch.tensor(cfg["seed_flows"], device=dev)
        flags = L.PC_BWD_SEEDED
    pflows = torch.zeros(circ.num_params, device=dev)
    ll = torch.empty(B, device=dev) if circ.root >= 0 else None
    ws = L.workspace(h, B, dev)
    stream = torch.cuda.current_stream()

    def step():
        pflows.zero_()
        L.pc_forward(h, B, tokens, params, vals, ll, None, ws, stream.cuda_stream)
        L.pc_backward(h, B, tokens, params, vals, flows, pflows, flags, None, None, ws, stream.cuda_stream)
        L.pc_em_step(h, params, pflows, 1.0, 0.0, stream.cuda_stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    run = step
    if args.graph:
        # the whole step recorded once as a HIP graph, replayed per step
        g = L.StepGraph(h, B, tokens, params, vals, flows, pflows, ll, flags, ws=ws, em=(1.0, 0.0))
        run = g.replay
        run()
        torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        run()
    torch.cuda.synchronize()
    dt = time.perf_counter() - t0
    ms = dt / args.steps * 1e3
    finite = bool(torch.isfinite(ll).all().item()) if ll is not None else bool(torch.isfinite(vals).all().item())

    # second timed pass with per-launch HIP events
    L.pc_set_timing(h, True)
    torch.cuda.synchronize()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    kt = L.pc_kernel_times(h)
    L.pc_set_timing(h, False)

    flops = sum_flops(circ, B)
    value = flops / (ms * 1e-3) / 1e12
    gemm_kinds = ["sum_fwd_gemm", "elem_flow_gemm", "param_flow_gemm"]
    sum_ms = sum(kt[k][1] for k in gemm_kinds) / args.steps
    other_sum_ms = sum(kt[k][1] for k in ("weight_split", "column_max", "exp_children", "scaled_flows")) / args.steps
    per_kind_flops = {"sum_fwd_gemm": flops / 3, "elem_flow_gemm": flops / 3, "param_flow_gemm": flops / 3}
    dom = max(gemm_kinds, key=lambda k: kt[k][1])
    n_launch, tot_ms = kt[dom]
    per_launch_flops = per_kind_flops[dom] * args.steps / max(n_launch, 1)
    avg_ms = tot_ms / max(n_launch, 1)
    achieved = per_launch_flops / (avg_ms * 1e-3) / 1e12
    out = {
        "metric": metric,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if args.mode == "auto" else "bf16x3-split",
        "data": "synthetic",
        "config": {"workload": workload, "precision_mode": args.mode, "global_batch": B, "hip_graph": bool(args.graph),
                   **({"splits": args.splits} if args.splits else {})},
        "frac_of_peak": round(value / PEAK_BF16_TFLOPS, 4),
        "sum_layer_kernels_ms": round(sum_ms, 4),
        "sum_layer_kernels_tflops": round(flops / (sum_ms * 1e-3) / 1e12, 3) if sum_ms > 0 else None,
        "sum_layer_aux_kernels_ms": round(other_sum_ms, 4),
        "kernel_ms_per_step": {k: round(v[1] / args.steps, 4) for k, v in kt.items() if v[0]},
        "kernel_launches_per_step": {k: v[0] // args.steps for k, v in kt.items() if v[0]},
        "roofline": {"kernel": dom, "bound": "mfma", "achieved": round(achieved, 3),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": kernel_traffic(dom) if args.workload == "hmm4096" else None,
                     "per_launch_gflop": round(per_launch_flops / 1e9, 4),
                     "avg_launch_ms": round(avg_ms, 5)},
        "finite": finite,
    }
    if context:
        out["context"] = context
    if not args.no_cpu:
        if args.workload == "hmm4096":
            sample = args.cpu_sample
        elif args.cpu_sample_other is not None:
            sample = args.cpu_sample_other
        else:
            sample = 8 if args.workload == "hclt" else 32 if args.workload == "pd" else B
        sample = min(sample, B)
        out["cpu_baseline"] = cpu_baseline(cfg, sample)
    print(json.dumps(out))


if __name__ == "__main__":
    main()
