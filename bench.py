"""Benchmark of one edge-aware attention layer forward (node + edge outputs) on
one MI355X.

A step is one whole layer call (``edge_attn_layer``: Q/K/V projection, scores
with head-wise FiLM, masked softmax, A and O, residual edge update; large
graphs take both passes of the two-pass scheme) over one synthetic batch
already resident in HBM. Where a batch is small, steps rotate over enough
distinct input/output buffer sets that the working set exceeds the 256 MB
Infinity Cache, so every step streams from HBM.

With no workload named, the JSON line is the large-graph configuration (B=4,
n=1024, two-pass: the largest that the layer is quoted on) and carries the
other four configurations (tiny, planar, tree, SBM) as sub-records in
``configs``, each with its own GPU time, roofline fraction and CPU oracle
legs. ``--workload NAME`` prints that configuration alone.

Every line carries graphs/s (value), edge-tokens/s, the dominant kernel's
roofline record (algorithmic bytes over its HIP-event-timed average
duration), the layer's own algorithmic bytes per step and their rate, and the
CPU oracle timed on the host as a reported baseline (all cores and one
thread, median of three runs where a run is short).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X published HBM3E bandwidth
INFINITY_CACHE_BYTES = 256 << 20
# the layer's kernels and the device headers they are built from
KERNEL_SOURCES = [os.path.join(ROOT, "edge_aware_graph_amd", "csrc", f)
                  for f in ("ea_kernels.hip", "ea_device.h", "ea_internal.h")]
# ablation variants (the EA_VARIANT_* desc flags)
VARIANT_FLAGS = {"none": 0, "light_edge": 0x2, "no_score_mod": 0x4, "unnormalized": 0x8}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="all", choices=["all", "planar", "tree", "sbm", "large", "tiny"],
                    help="all (default): the large configuration as the line, the others as sub-records")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--sub-steps", type=int, default=200,
                    help="timed steps of each sub-record configuration (--workload all)")
    ap.add_argument("--hot", action="store_true", help="also time back-to-back calls on one buffer set")
    ap.add_argument("--variant", default="none", choices=sorted(VARIANT_FLAGS),
                    help="ablation variant of the layer (the default is the full layer)")
    ap.add_argument("--backward", action="store_true",
                    help="time training steps instead: the layer forward plus its backward")
    ap.add_argument("--recompute-a", action="store_true",
                    help="with --backward on two-pass shapes: pass no A (the backward recomputes it)")
    ap.add_argument("--block", action="store_true",
                    help="time the graph-transformer block around the layer (layer + node, edge and y paths)")
    ap.add_argument("--sampling-layers", type=int, default=0,
                    help="instead of single layers, time denoising steps of this many stacked layers "
                         "(a step is then one pass through all of them; with --block, whole blocks)")
    return ap.parse_args()


def backward_bench(args, cfg, dims, batch):
    """Training step of the layer: edge_attn_layer then edge_attn_backward, on
    buffer sets rotated so that every step reads from HBM (two buffer sets:
    at the large shape one set holds several GB). Two-pass shapes pass an A
    buffer, which the layer's second pass fills and the backward reads
    (--recompute-a: no A, the backward recomputes it)."""
    import torch
    from edge_aware_graph_amd.layer import EdgeAttention
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if dims.dtype == "bf16" else torch.float32
    layer = EdgeAttention(dims.B, dims.n, dims.d, dims.de, dims.dy, dims.H, dims.dh, dims.dtype)
    w = {k: torch.from_numpy(v).to(dev, dt) for k, v in batch.items() if k.startswith(("w_", "b_"))}
    B, n, d, de, H, dy = dims.B, dims.n, dims.d, dims.de, dims.H, dims.dy
    rng = np.random.default_rng(0)
    sets = []
    for _ in range(2):
        sets.append(dict(
            X=torch.from_numpy(batch["X"]).to(dev, dt), E=torch.from_numpy(batch["E"]).to(dev, dt),
            y=torch.from_numpy(batch["y"]).to(dev, dt), m=torch.from_numpy(batch["mask"]).to(dev),
            O=torch.empty(B, n, d, dtype=dt, device=dev),
            A=None if (layer.two_pass and args.recompute_a) else torch.empty(B, H, n, n, dtype=dt, device=dev),
            Eo=torch.empty(B, n, n, de, dtype=dt, device=dev),
            dO=torch.from_numpy(rng.standard_normal((B, n, d)).astype(np.float32)).to(dev, dt),
            dEp=torch.from_numpy(rng.standard_normal((B, n, n, de)).astype(np.float32)).to(dev, dt),
            dX=torch.empty(B, n, d, dtype=dt, device=dev), dE=torch.empty(B, n, n, de, dtype=dt, device=dev),
            dy=torch.empty(B, dy, dtype=dt, device=dev),
            g={k: torch.empty(tuple(batch[k].shape), dtype=torch.float32, device=dev)
               for k in batch if k.startswith(("w_", "b_"))},
            ws=torch.empty(layer.workspace_bytes, dtype=torch.uint8, device=dev),
            bws=torch.empty(layer.backward_workspace_bytes, dtype=torch.uint8, device=dev)))

    def step(k):
        s = sets[k % len(sets)]
        layer.layer(w, s["X"], s["E"], s["y"], s["m"], s["O"], s["A"], s["Eo"], s["ws"])
        layer.backward(w, s["X"], s["E"], s["y"], s["m"], s["A"], s["dO"], s["dEp"], s["dX"], s["dE"], s["dy"],
                       s["g"], s["ws"], s["bws"])

    for k in range(args.warmup):
        step(k)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        step(k)
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    layer.profile_begin()
    for k in range(args.steps):
        step(k)
    prof = layer.profile_end()
    kernels = {name: {"avg_us": 1e3 * ms / cnt, "launches": cnt} for name, (ms, cnt) in prof.items() if cnt}
    bwd_name = [k for k in kernels if k.startswith("backward")][0]
    alg = algorithmic_bytes("backward", dims, batch["n_real"], layer.two_pass and args.recompute_a)
    bwd_us = kernels[bwd_name]["avg_us"]
    return {
        "metric": "graphs/s per training step of the layer (forward + backward)",
        "value": B / (ms_per_step * 1e-3), "unit": "graphs/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if dims.dtype == "bf16" else "fp32",
        "data": "synthetic (seeded %s graphs, random Xavier weights, random output gradients)" % cfg.structure,
        "config": {"workload": cfg.name, "B": B, "n": n, "d": d, "de": de, "H": H, "buffer_sets": len(sets),
                   "two_pass": layer.two_pass, "a_stored": sets[0]["A"] is not None},
        # the backward's launches taken together (HIP events around the call)
        "roofline": {"kernel": bwd_name, "bound": "hbm", "achieved": alg / (bwd_us * 1e3), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": alg / (bwd_us * 1e3) / HBM_PEAK_GBS,
                     "traffic": traffic_from_profiles("backward", cfg.name),
                     "alg_bytes_per_launch": alg, "avg_launch_us": bwd_us},
        "kernels": kernels,
    }


def block_bench(args, cfg, dims, batch):
    """Forward of the graph-transformer block around the layer (the layer,
    then the node, edge and global-feature paths), on buffer sets rotated so
    that every step reads from HBM."""
    import torch
    from edge_aware_graph_amd import workloads as W
    from edge_aware_graph_amd.layer import EdgeAttention
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if dims.dtype == "bf16" else torch.float32
    layer = EdgeAttention(dims.B, dims.n, dims.d, dims.de, dims.dy, dims.H, dims.dh, dims.dtype)
    w = {k: torch.from_numpy(v).to(dev, dt) for k, v in batch.items() if k.startswith(("w_", "b_"))}
    bp = {k: torch.from_numpy(v).to(dev, dt) for k, v in W.make_block_params(dims, scale=0.0).items()}
    B, n, d, de, dy = dims.B, dims.n, dims.d, dims.de, dims.dy
    s = 2 if dims.dtype == "bf16" else 4
    set_bytes = (2 * B * n * n * de + 2 * B * n * d + 2 * B * dy) * s + layer.block_workspace_bytes
    nsets = int(max(1, min(16, -(-2 * INFINITY_CACHE_BYTES // set_bytes))))
    calls = []
    for _ in range(nsets):
        X = torch.from_numpy(batch["X"]).to(dev, dt)
        E = torch.from_numpy(batch["E"]).to(dev, dt)
        y = torch.from_numpy(batch["y"]).to(dev, dt)
        m = torch.from_numpy(batch["mask"]).to(dev)
        Xo, Eo, yo = torch.empty_like(X), torch.empty_like(E), torch.empty_like(y)
        ws = torch.empty(layer.block_workspace_bytes, dtype=torch.uint8, device=dev)
        calls.append(layer.bind_block(w, bp, X, E, y, m, Xo, Eo, yo, ws))
    for k in range(args.warmup):
        calls[k % nsets]()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        calls[k % nsets]()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / args.steps
    layer.profile_begin()
    for k in range(args.steps):
        calls[k % nsets]()
    prof = layer.profile_end()
    kernels = {name: {"avg_us": 1e3 * ms / cnt, "launches": cnt} for name, (ms, cnt) in prof.items() if cnt}
    bname = [k for k in kernels if k.startswith("block")][0]
    alg = algorithmic_bytes("block", dims, batch["n_real"], layer.two_pass)
    bus = kernels[bname]["avg_us"]
    return {
        "metric": "graphs/s per graph-transformer block forward (edge-aware attention layer + node, edge "
                  "and global-feature paths)",
        "value": B / (ms_per_step * 1e-3), "unit": "graphs/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if dims.dtype == "bf16" else "fp32",
        "data": "synthetic (seeded %s graphs, random Xavier weights)" % cfg.structure,
        "config": {"workload": cfg.name, "B": B, "n": n, "d": d, "de": de, "dy": dy, "H": dims.H,
                   "two_pass": layer.two_pass, "buffer_sets": nsets},
        # the block's own three launches taken together (HIP events around them)
        "roofline": {"kernel": bname, "bound": "hbm", "achieved": alg / (bus * 1e3), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": alg / (bus * 1e3) / HBM_PEAK_GBS,
                     "traffic": traffic_from_profiles("block", cfg.name),
                     "alg_bytes_per_launch": alg, "avg_launch_us": bus},
        "kernels": kernels,
    }


def sampling_bench(args, cfg, dims, batch):
    """Stacked-layer sampling loop: each timed step runs L layers with their own
    random weights, O and E' of a layer feeding the next (same batch,
    HBM-resident). With --block every layer is a whole graph-transformer
    block (X2, E2 and y2 feed the next one)."""
    import torch
    from edge_aware_graph_amd import workloads as W
    from edge_aware_graph_amd.sampling import SamplingLoop
    dev = torch.device("cuda:0")
    dt = torch.bfloat16 if dims.dtype == "bf16" else torch.float32
    L = args.sampling_layers
    weights = []
    for k in range(L):
        wb = W.make_batch(cfg.name, seed=1000 + k, bias_scale=0.0)
        weights.append({kk: torch.from_numpy(v).to(dev, dt) for kk, v in wb.items() if kk.startswith("w_")})
    bps = None
    if args.block:
        bps = [{kk: torch.from_numpy(v).to(dev, dt) for kk, v in W.make_block_params(dims, seed=2000 + k).items()}
               for k in range(L)]
    loop = SamplingLoop(dims, weights, block_params=bps)
    X0 = torch.from_numpy(batch["X"]).to(dev, dt)
    E0 = torch.from_numpy(batch["E"]).to(dev, dt)
    y0 = torch.from_numpy(batch["y"]).to(dev, dt)
    m0 = torch.from_numpy(batch["mask"]).to(dev)
    loop.run(X0, E0, y0, m0, steps=args.warmup)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    loop.run(X0, E0, y0, m0, steps=args.steps)
    torch.cuda.synchronize()
    dt_s = time.perf_counter() - t0
    ms_per_step = dt_s * 1e3 / args.steps
    B, n = dims.B, dims.n
    return {
        "metric": "graphs/s per denoising step of %d stacked %s" % (
            L, "graph-transformer blocks" if args.block else "edge-aware attention layers"),
        "value": B / (ms_per_step * 1e-3),
        "unit": "graphs/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_per_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16" if dims.dtype == "bf16" else "fp32",
        "data": "synthetic (seeded %s graphs, random Xavier weights per layer)" % cfg.structure,
        "config": {"workload": cfg.name, "B": B, "n": n, "layers": L, "two_pass": loop.layer.two_pass,
                   "blocks": loop.blocks,
                   "note": "a step is the L %s only (the sampler's update rule is not modelled)" % (
                       "blocks" if loop.blocks else "attention layers")},
        "layers_per_s": L / (ms_per_step * 1e-3),
        "ms_per_layer": ms_per_step / L,
    }


def algorithmic_bytes(kernel: str, dims, n_real: np.ndarray, two_pass: bool,
                      recompute: bool = None) -> float:
    """Bytes one launch of `kernel` must move (inputs read once, outputs written once).

    Per edge token (b, i, j): E read (real pairs only), E' written (whole
    padded layout), A written (single pass). Per node row: O written, the
    per-head Q, K, V read from the workspace. Per graph: lse for two-pass.
    `recompute`: the edge update recomputes the logits (two-pass, or the
    unnormalized variant) and reads Q and K instead of A.
    """
    recompute = two_pass if recompute is None else recompute
    s = 2 if dims.dtype == "bf16" else 4
    B, n, d, de, H = dims.B, dims.n, dims.d, dims.de, dims.H
    tokens = B * n * n
    real_tokens = float(np.sum(n_real.astype(np.float64) ** 2))
    rows = B * n
    e_read = real_tokens * de * s
    e_write = tokens * de * s
    a_io = tokens * H * s
    o_write = rows * d * s
    qkv = 3 * rows * d * s
    lse = B * H * n * 4
    if kernel == "attn_kernel(fused)":
        return e_read + e_write + a_io + o_write + qkv
    if kernel == "attn_kernel":
        return e_read + o_write + qkv + (lse if two_pass else a_io)
    if kernel == "update_kernel":
        return e_read + e_write + ((2 * rows * d * s + (lse if two_pass else 0)) if recompute else a_io)
    if kernel == "qkv_kernel":
        return rows * d * s + 3 * d * d * s + qkv
    if kernel == "block":
        # node path: O and X read, X2 written; edge path: E' read, E2 written
        # (real pairs only carry data, but the padded layout is written);
        # parameters read once
        fx, fe, fy = d, 2 * de, dims.dy
        params = (3 * d * d + 2 * de * fe + dims.dy * (2 * dims.dy + d + de)) * s
        return 3 * rows * d * s + e_read + e_write + params
    if kernel == "backward":
        # E and dE' read (real pairs), dE written, A read (two-pass: lse
        # read, A recomputed from E, Q and K); X and dO read, dX written;
        # Q, K, V read back from the workspace; the projection weights read
        # and their float32 gradients written
        return (2 * e_read + e_write + (lse if two_pass else a_io) + 3 * rows * d * s + qkv +
                3 * d * d * (s + 4))
    raise ValueError(kernel)


def source_digest(paths=None) -> str:
    """sha256 prefix of kernel sources, concatenated (default: the layer's)."""
    h = hashlib.sha256()
    for path in (KERNEL_SOURCES if paths is None else paths):
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel: str, workload: str, profiles_dir: str = None):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they
    were taken on the current kernel sources (the record lists the sources it
    was taken on, relative to the repository; the layer's by default); else
    None."""
    profiles_dir = os.path.join(ROOT, "profiles") if profiles_dir is None else profiles_dir
    path = os.path.join(profiles_dir, "traffic_%s_%s.json" % (kernel.split("(")[0].strip(), workload))
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    srcs = rec.get("sources")
    paths = None if srcs is None else [os.path.join(ROOT, p) for p in srcs]
    if paths is not None and not all(os.path.exists(p) for p in paths):
        return None
    if rec.get("kernel_source_sha256_16") != source_digest(paths):
        return None
    return rec.get("hbm_bytes_per_launch")


def layer_algorithmic_bytes(dims, n_real: np.ndarray, two_pass: bool) -> float:
    """Bytes one layer call must move, whatever its kernels keep in between.

    Per edge token (b, i, j): E read on real pairs (twice in two-pass mode:
    the scheme reads it in both passes), E' written over the whole padded
    layout, A written (single pass only). Per node row: X read (real rows),
    O written (all rows). Per graph: y read; two-pass adds the softmax
    statistics (float32, H per row). Plus the weights, read once. At the
    planar shape this is (2 de + H) 2 B = 272 B per edge token and 2 d 2 B =
    1024 B per node, 75.9 MB in all."""
    s = 2 if dims.dtype == "bf16" else 4
    B, n, d, de, dy, H = dims.B, dims.n, dims.d, dims.de, dims.dy, dims.H
    nr = n_real.astype(np.float64)
    tokens, real_tokens = B * n * n, float(np.sum(nr ** 2))
    e_read = real_tokens * de * s * (2 if two_pass else 1)
    e_write = tokens * de * s
    a_write = 0 if two_pass else tokens * H * s
    lse = B * H * n * 4 if two_pass else 0
    x_read, o_write = float(np.sum(nr)) * d * s, B * n * d * s
    weights = (3 * d * d + 2 * H * de + 2 * H * dy + de * H) * s + B * dy * s
    return e_read + e_write + a_write + lse + x_read + o_write + weights


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _sub_batch(batch, graphs: int):
    return {k: (v[:graphs] if k in ("X", "E", "y", "mask", "adj", "n_real") else v) for k, v in batch.items()}


def cpu_legs(batch, dims, budget_s: float = 4.0, oracle_variant: int = 0, runs: int = 3):
    """The oracle (as it stands) timed on the host: all cores (OpenMP over
    query rows) and one thread. Each leg runs the oracle on a sample of the
    batch sized to about `budget_s` (whole graphs when one fits, else the
    first query rows of graph 0: the oracle's cost per row does not depend
    on the row), `runs` times, and reports the median as graphs/s of the
    batch's shape (rows/s divided by the n rows of a graph)."""
    from oracle import oracle as OR
    bf = dims.dtype == "bf16"
    all_threads = OR.num_threads()
    out = {}
    for leg, threads in (("all_cores", all_threads), ("single_thread", 1)):
        prev = OR.set_num_threads(threads)
        try:
            t0 = time.perf_counter()
            OR.forward(_sub_batch(batch, 1), dims.H, bf16=bf, rows=[(0, i) for i in range(min(dims.n, 16))],
                       variant=oracle_variant)
            per_row = max((time.perf_counter() - t0) / min(dims.n, 16), 1e-6)
            rows_fit = budget_s / per_row
            if rows_fit >= dims.n:  # whole graphs
                g = int(max(1, min(dims.B, rows_fit // dims.n)))
                sub, rows, what = _sub_batch(batch, g), None, "the first %d of the %d graphs" % (g, dims.B)
                units = float(g)
            else:
                r = int(max(8, min(dims.n, rows_fit)))
                sub, rows = _sub_batch(batch, 1), [(0, i) for i in range(r)]
                what = "the first %d of the %d query rows of graph 0" % (r, dims.n)
                units = r / float(dims.n)
            times = []
            for _ in range(runs):
                t0 = time.perf_counter()
                OR.forward(sub, dims.H, bf16=bf, rows=rows, variant=oracle_variant)
                times.append(time.perf_counter() - t0)
            med = float(np.median(times))
            out[leg] = {"value": units / med, "unit": "graphs/s", "threads": threads, "runs": runs,
                        "median_s": med, "sample": what}
        finally:
            OR.set_num_threads(prev)
    return out


def cpu_baseline(batch, dims, budget_s: float = 4.0, oracle_variant: int = 0, runs: int = 3):
    """cpu_baseline record: the all-core leg as the value, the one-thread leg beside it."""
    legs = cpu_legs(batch, dims, budget_s, oracle_variant, runs)
    a = legs["all_cores"]
    return {"value": a["value"], "unit": "graphs/s", "cores": a["threads"], "kind": "oracle",
            "sample": "%s, every output of those rows (float64 C loops, OpenMP over query rows), "
                      "median of %d runs; graphs/s of this configuration's shape" % (a["sample"], runs),
            "single_thread": legs["single_thread"], "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(),
            "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS")}


def event_pair_overhead_us(reps: int = 200) -> float:
    """Median elapsed time of two HIP events recorded back to back on the
    current stream: what a per-launch event pair adds to a kernel's time."""
    import torch
    st = torch.cuda.current_stream()
    vals = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        e1.record(st)
        e1.synchronize()
        vals.append(e0.elapsed_time(e1) * 1e3)
    return float(np.median(vals))


def hbm_ceiling(nbytes: int = 1 << 30, reps: int = 10) -> dict:
    """Achievable HBM rate on a plain stream, for context next to the kernels'
    roofline fractions: the library's probe copy (nbytes read + nbytes
    written) and probe read over nbytes, each launched `reps` times after
    three warm-up launches, timed with events on the launch stream (median
    launch)."""
    import torch
    from edge_aware_graph_amd import layer as L
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    src.fill_(1)
    dst = torch.empty_like(src)
    acc = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    st = torch.cuda.current_stream()
    res = {"bytes": nbytes, "launches": reps}
    for kind in ("copy", "read"):
        run = (lambda: L.probe_copy(src, dst, st)) if kind == "copy" else (lambda: L.probe_read(src, acc, st))
        for _ in range(3):
            run()
        times = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            run()
            e1.record(st)
            e1.synchronize()
            times.append(e0.elapsed_time(e1) * 1e-3)
        t = float(np.median(times))
        moved = 2 * nbytes if kind == "copy" else nbytes
        res[kind + "_us"] = t * 1e6
        res[kind + "_GBps"] = moved / t / 1e9
    if not torch.equal(dst[:4096], src[:4096]):
        raise RuntimeError("probe copy gave wrong bytes")
    del src, dst, acc
    torch.cuda.empty_cache()
    return res


def time_layer(name: str, steps: int, warmup: int, variant: str = "none", hot: bool = False):
    """GPU record of one configuration: wall time per layer call over `steps`
    calls (after `warmup`), per-kernel HIP-event durations over the same
    sequence, the dominant kernel's roofline and the layer's algorithmic rate."""
    import torch
    from edge_aware_graph_amd import workloads as W
    from edge_aware_graph_amd.layer import EdgeAttention
    dev = torch.device("cuda:0")
    cfg = W.CONFIGS[name]
    dims = cfg.dims
    print("[bench] workload %s: %s" % (cfg.name, cfg.description), file=sys.stderr, flush=True)
    batch = W.make_batch(cfg.name, bias_scale=0.0)
    n_real = batch["n_real"]
    dt = torch.bfloat16 if dims.dtype == "bf16" else torch.float32
    vflag = VARIANT_FLAGS[variant]
    layer = EdgeAttention(dims.B, dims.n, dims.d, dims.de, dims.dy, dims.H, dims.dh, dims.dtype, variant=vflag)
    two_pass = layer.two_pass
    recompute = layer.recomputes_update
    # biases are all zero in the timed configuration: passed as NULL
    weights = {k: torch.from_numpy(batch[k]).to(dev, dt) for k in batch if k.startswith("w_")}
    X0 = torch.from_numpy(batch["X"]).to(dev, dt)
    E0 = torch.from_numpy(batch["E"]).to(dev, dt)
    y0 = torch.from_numpy(batch["y"]).to(dev, dt)
    m0 = torch.from_numpy(batch["mask"]).to(dev)
    B, n, d, de, H = dims.B, dims.n, dims.d, dims.de, dims.H
    es = 2 if dims.dtype == "bf16" else 4
    set_bytes = (2 * B * n * n * de + B * n * d * 2 + (0 if two_pass else B * H * n * n)) * es + layer.workspace_bytes
    nsets = int(max(1, min(16, -(-2 * INFINITY_CACHE_BYTES // set_bytes))))
    sets = []
    for k in range(nsets):
        sets.append(dict(
            X=X0 if k == 0 else X0.clone(), E=E0 if k == 0 else E0.clone(), y=y0.clone(), mask=m0.clone(),
            O=torch.empty(B, n, d, dtype=dt, device=dev),
            A=None if two_pass else torch.empty(B, H, n, n, dtype=dt, device=dev),
            Eo=torch.empty(B, n, n, de, dtype=dt, device=dev),
            ws=torch.empty(layer.workspace_bytes, dtype=torch.uint8, device=dev)))
    print("[bench] %d buffer sets of %.1f MiB (two_pass=%s)" % (nsets, set_bytes / 2**20, two_pass),
          file=sys.stderr, flush=True)
    calls = [layer.bind_layer(weights, st["X"], st["E"], st["y"], st["mask"], st["O"], st["A"], st["Eo"], st["ws"])
             for st in sets]
    for k in range(warmup):
        calls[k % nsets]()
    torch.cuda.synchronize()
    # timed region: exactly `steps` layer calls
    t0 = time.perf_counter()
    for k in range(steps):
        calls[k % nsets]()
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - t0) * 1e3 / steps
    print("[bench] %s: timed %d steps, %.4f ms/step" % (name, steps, ms_per_step), file=sys.stderr, flush=True)
    # per-kernel durations from HIP events on the launch stream, same step sequence
    layer.profile_begin()
    for k in range(steps):
        calls[k % nsets]()
    prof = layer.profile_end()
    kernels = {kn: {"avg_us": 1e3 * ms / cnt, "launches": cnt} for kn, (ms, cnt) in prof.items() if cnt}
    for kn in kernels:
        b = algorithmic_bytes(kn, dims, n_real, two_pass, recompute)
        kernels[kn]["alg_bytes"] = b
        kernels[kn]["alg_GBps"] = b / (kernels[kn]["avg_us"] * 1e-6) / 1e9
    dominant = max(kernels, key=lambda k: kernels[k]["avg_us"])
    alg = kernels[dominant]["alg_bytes"]
    achieved = kernels[dominant]["alg_GBps"]
    layer_bytes = layer_algorithmic_bytes(dims, n_real, two_pass)
    rec = {
        "graphs_per_s": B / (ms_per_step * 1e-3),
        "ms_per_step": ms_per_step,
        "edge_tokens_per_s": B * n * n / (ms_per_step * 1e-3),
        "real_edge_tokens_per_s": float(np.sum(n_real.astype(np.float64) ** 2)) / (ms_per_step * 1e-3),
        "layer_alg_bytes": layer_bytes,
        "layer_alg_GBps": layer_bytes / (ms_per_step * 1e-3) / 1e9,
        "layer_frac_of_hbm": layer_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS,
        "config": {"workload": cfg.name, "B": B, "n": n, "d": d, "de": de, "dy": dims.dy, "H": H,
                   "dh": dims.dh, "structure": cfg.structure, "two_pass": two_pass, "variant": variant,
                   "edge_tokens_per_step": B * n * n, "real_edge_tokens_per_step": int(np.sum(n_real ** 2)),
                   "buffer_sets": nsets},
        "roofline": {"kernel": dominant, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBS,
                     "traffic": traffic_from_profiles(dominant, cfg.name) if variant == "none" else None,
                     "alg_bytes_per_launch": alg, "avg_launch_us": kernels[dominant]["avg_us"]},
        "kernels": kernels,
        "data": "synthetic (seeded %s graphs, random Xavier weights)" % cfg.structure,
        "dtype": "bf16" if dims.dtype == "bf16" else "fp32",
    }
    if hot:
        for _ in range(warmup):
            calls[0]()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            calls[0]()
        torch.cuda.synchronize()
        rec["hot_ms_per_step"] = (time.perf_counter() - t0) * 1e3 / steps
    del calls, sets, X0, E0
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec, batch, dims


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the layer's batch dimension shards across GPUs "
              "with no communication, so a multi-GPU figure is the one-GPU figure times N; "
              "use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    from edge_aware_graph_amd import workloads as W

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    special = args.sampling_layers > 0 or args.backward or args.block
    if special:
        name = "planar" if args.workload == "all" else args.workload
        cfg = W.CONFIGS[name]
        print("[bench] workload %s: %s" % (cfg.name, cfg.description), file=sys.stderr, flush=True)
        batch = W.make_batch(cfg.name, bias_scale=0.0)
        if args.sampling_layers > 0:
            print(json.dumps(sampling_bench(args, cfg, cfg.dims, batch)), flush=True)
        elif args.backward:
            print(json.dumps(backward_bench(args, cfg, cfg.dims, batch)), flush=True)
        else:
            print(json.dumps(block_bench(args, cfg, cfg.dims, batch)), flush=True)
        return

    oracle_variant = {"none": 0, "light_edge": 1, "no_score_mod": 2, "unnormalized": 4}[args.variant]
    head = "large" if args.workload == "all" else args.workload
    rec, batch, dims = time_layer(head, args.steps, args.warmup, args.variant, args.hot)
    out = {
        "metric": "graphs/s per fused layer forward (edge-aware attention + residual edge update)",
        "value": rec["graphs_per_s"],
        "unit": "graphs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": rec["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": rec["dtype"],
        "data": rec["data"],
        "config": rec["config"],
        "edge_tokens_per_s": rec["edge_tokens_per_s"],
        "real_edge_tokens_per_s": rec["real_edge_tokens_per_s"],
        "layer_alg_bytes": rec["layer_alg_bytes"],
        "layer_alg_GBps": rec["layer_alg_GBps"],
        "layer_frac_of_hbm": rec["layer_frac_of_hbm"],
        "roofline": rec["roofline"],
        "kernels": rec["kernels"],
        "event_pair_overhead_us": event_pair_overhead_us(),
    }
    if "hot_ms_per_step" in rec:
        out["hot_ms_per_step"] = rec["hot_ms_per_step"]
    # plain copy of known size (for scaling rocprofv3 byte counters)
    cp_src = torch.empty(256 << 20, dtype=torch.uint8, device="cuda:0")
    cp_dst = torch.empty_like(cp_src)
    cp_dst.copy_(cp_src)
    torch.cuda.synchronize()
    del cp_src, cp_dst
    out["copy_calibration_bytes"] = 256 << 20
    out["hbm_ceiling"] = hbm_ceiling()
    rl = out["roofline"]
    rl["achieved_over_measured_ceiling"] = rl["achieved"] / out["hbm_ceiling"][
        "copy_GBps" if rl["kernel"] in ("update_kernel", "attn_kernel(fused)") else "read_GBps"]
    if not args.no_cpu_baseline:
        print("[bench] timing the CPU oracle (%s)" % head, file=sys.stderr, flush=True)
        out["cpu_baseline"] = cpu_baseline(batch, dims, budget_s=3.0, oracle_variant=oracle_variant, runs=3)
        out["gpu_over_oracle_all_cores"] = rec["graphs_per_s"] / out["cpu_baseline"]["value"]
    del batch
    if args.workload == "all":
        configs = {}
        for name in ("tiny", "planar", "tree", "sbm"):
            sub, sbatch, sdims = time_layer(name, args.sub_steps, args.warmup, args.variant)
            if not args.no_cpu_baseline:
                print("[bench] timing the CPU oracle (%s)" % name, file=sys.stderr, flush=True)
                legs = cpu_legs(sbatch, sdims, budget_s=3.0, oracle_variant=oracle_variant, runs=3)
                sub["cpu_oracle"] = legs
                sub["gpu_over_oracle_all_cores"] = sub["graphs_per_s"] / legs["all_cores"]["value"]
                sub["gpu_over_oracle_single_thread"] = sub["graphs_per_s"] / legs["single_thread"]["value"]
            del sbatch
            configs[name] = sub
        configs["large"] = {k: rec[k] for k in ("graphs_per_s", "ms_per_step", "edge_tokens_per_s",
                                                "real_edge_tokens_per_s", "layer_alg_bytes", "layer_alg_GBps",
                                                "layer_frac_of_hbm", "roofline")}
        out["configs"] = configs
        # structure changes values, not work: planar and tree should time the same
        out["tree_over_planar_time"] = configs["tree"]["ms_per_step"] / configs["planar"]["ms_per_step"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
