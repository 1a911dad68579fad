"""Host logic of bench.py (CPU only): the one-GPU rule, the algorithmic byte
counts behind the roofline fraction, and the gate that keeps counter traffic
from stale sources out of the JSON line."""
import json
import os
import subprocess
import sys

import numpy as np

import bench
from edge_aware_graph_amd import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_fused_bytes_at_planar():
    """Per edge token E read, E' and A written: (2 de + H) x 2 B = 272 B; per
    node row Q, K, V read and O written: 4 d x 2 B (every node real)."""
    dims = W.CONFIGS["planar"].dims
    n_real = np.full(dims.B, dims.n)
    tokens, rows = dims.B * dims.n * dims.n, dims.B * dims.n
    assert (2 * dims.de + dims.H) * 2 == 272
    want = tokens * 272 + rows * 4 * dims.d * 2
    assert bench.algorithmic_bytes("attn_kernel(fused)", dims, n_real, False) == want


def test_edge_reads_count_real_pairs_only():
    """Padded pairs are not read (E is read on real pairs), but the padded E'
    layout is written whole."""
    dims = W.CONFIGS["sbm"].dims
    full = np.full(dims.B, dims.n)
    ragged = np.arange(dims.B) + 44
    diff = bench.algorithmic_bytes("update_kernel", dims, full, False) - \
        bench.algorithmic_bytes("update_kernel", dims, ragged, False)
    assert diff == float(np.sum(full.astype(np.float64) ** 2 - ragged.astype(np.float64) ** 2)) * dims.de * 2


def test_two_pass_backward_counts_lse_instead_of_a():
    dims = W.CONFIGS["large"].dims
    n_real = np.full(dims.B, dims.n)
    one = bench.algorithmic_bytes("backward", dims, n_real, False)
    two = bench.algorithmic_bytes("backward", dims, n_real, True)
    a_io = dims.B * dims.n * dims.n * dims.H * 2
    lse = dims.B * dims.H * dims.n * 4
    assert one - two == a_io - lse


def test_traffic_gate(tmp_path):
    src = tmp_path / "kernel.hip"
    src.write_text("// kernel source\n")
    rec = {"kernel": "demo", "workload": "planar", "sources": [str(src)],
           "kernel_source_sha256_16": bench.source_digest([str(src)]), "hbm_bytes_per_launch": 123.0}
    (tmp_path / "traffic_demo_planar.json").write_text(json.dumps(rec))
    assert bench.traffic_from_profiles("demo(fused)", "planar", str(tmp_path)) == 123.0
    assert bench.traffic_from_profiles("demo", "sbm", str(tmp_path)) is None  # no record
    src.write_text("// kernel source, changed\n")
    assert bench.traffic_from_profiles("demo", "planar", str(tmp_path)) is None  # stale
    os.remove(src)
    assert bench.traffic_from_profiles("demo", "planar", str(tmp_path)) is None  # source gone



def test_layer_bytes_at_the_configurations():
    """The layer's algorithmic bytes per call: (2 de + H) 2 B = 272 B per edge
    token and 2 d 2 B = 1024 B per node at planar, 75.9 MB with the weights;
    two-pass reads E in both passes (384 B per token), 1.615 GB at the large
    shape; SBM reads E and X on real pairs and rows only, 238 MB."""
    planar = W.CONFIGS["planar"].dims
    full = np.full(planar.B, planar.n)
    b = bench.layer_algorithmic_bytes(planar, full, False)
    assert abs(b - 75.9e6) < 0.05e6
    tokens, rows = planar.B * planar.n ** 2, planar.B * planar.n
    weights = (3 * 256 * 256 + 2 * 8 * 64 * 2 + 64 * 8) * 2 + planar.B * 64 * 2
    assert b == tokens * 272 + rows * 1024 + weights
    large = W.CONFIGS["large"].dims
    bl = bench.layer_algorithmic_bytes(large, np.full(large.B, large.n), True)
    assert abs(bl - 1.615e9) < 0.001e9
    assert bl - large.B * large.n ** 2 * 384 < 5e6
    sbm = W.CONFIGS["sbm"]
    n_real = W.make_batch("sbm")["n_real"]
    assert abs(bench.layer_algorithmic_bytes(sbm.dims, n_real, False) - 238e6) < 1e6


def test_cpu_legs_report_medians_and_both_thread_counts():
    """The oracle's timing legs on a small batch: all cores and one thread,
    graphs/s of the batch's shape, the thread count restored afterwards."""
    from oracle import oracle as OR
    dims = W.CONFIGS["tiny"].dims
    batch = W.make_batch("tiny")
    before = OR.num_threads()
    legs = bench.cpu_legs(batch, dims, budget_s=0.05, runs=3)
    assert OR.num_threads() == before
    assert legs["single_thread"]["threads"] == 1 and legs["all_cores"]["threads"] == before
    for leg in legs.values():
        assert leg["value"] > 0 and leg["runs"] == 3 and leg["unit"] == "graphs/s"
    rec = bench.cpu_baseline(batch, dims, budget_s=0.05)
    assert rec["kind"] == "oracle" and rec["cores"] == before and rec["cpu_model"]
