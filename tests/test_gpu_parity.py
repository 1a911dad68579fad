"""GPU parity: the HIP layer (through the C ABI) against the CPU oracle.

Every expected value comes from ``oracle/`` on the same seeded inputs; the
tolerances are the layer's contract (float32: 1e-4 normwise relative per
tensor; bfloat16: 2e-2 max-abs; masked outputs +0.0 bitwise).
"""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from edge_aware_graph_amd import workloads as W
from oracle import oracle as OR
from tests import _layer_harness as HX

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _need_gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("needs a GPU")
    print("\n[case] %s" % request.node.name, flush=True)
    sys.stdout.flush()


def dims_of(name, **over):
    return dataclasses.replace(W.CONFIGS[name].dims, **over)


def run_case(name, dims, seed=None, bias_scale=0.1, mode="fused", force_two_pass=False, rows=None,
             batch=None):
    if batch is None:
        batch = W.make_batch(name, seed=seed, bias_scale=bias_scale, dims=dims)
    run = HX.Run(batch, dims, force_two_pass=force_two_pass)
    (run.fused() if mode == "fused" else run.separate())
    res = run.results()
    ref = OR.forward(batch, dims.H, bf16=(dims.dtype == "bf16"), rows=rows)
    HX.compare(res, ref, batch["mask"], dims, rows=None if rows is None else ref["rows"])
    return batch, res, ref


FULL_CASES = [
    ("tiny", {}),
    ("tiny", {"dtype": "bf16"}),
    ("planar", {}),
    ("tree", {}),
    ("sbm", {}),
    ("planar", {"dtype": "fp32"}),
    ("sbm", {"dtype": "fp32", "B": 8}),
]


@pytest.mark.parametrize("name,over", FULL_CASES, ids=["%s-%s" % (c, "-".join("%s%s" % kv for kv in o.items()) or "cfg") for c, o in FULL_CASES])
@pytest.mark.parametrize("mode", ["fused", "separate"])
def test_layer_full(name, over, mode):
    """Full-tensor parity of O, A and E' at the configuration shapes."""
    run_case(name, dims_of(name, **over), mode=mode)


def test_bench_configuration_zero_bias():
    """The planar batch exactly as timed (zero biases), full tensors."""
    run_case("planar", dims_of("planar"), bias_scale=0.0)


@pytest.mark.parametrize("name,over", [("tiny", {}), ("planar", {}), ("sbm", {"B": 6})])
def test_logit_stage(name, over):
    """Stage parity: masked logits u from the score stage against the oracle's."""
    dims = dims_of(name, **over)
    batch = W.make_batch(name, bias_scale=0.1, dims=dims)
    run = HX.Run(batch, dims)
    U = run.logits()
    ref = OR.forward(batch, dims.H, bf16=(dims.dtype == "bf16"))["U"]
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(U), ~fin)
    err = np.abs(U[fin] - ref[fin])
    scale = np.abs(ref[fin]).max()
    # logits are float32 in both modes; bf16 mode rounds Q and K on each side
    assert err.max() <= (1e-4 if dims.dtype == "fp32" else 1e-3) * max(scale, 1.0)


def test_large_two_pass_sampled():
    """Large-graph configuration (n = 1024, two-pass): sampled rows against the oracle."""
    dims = dims_of("large")
    batch = W.make_batch("large", bias_scale=0.0)
    rows = HX.sample_rows(batch, 40, seed=1)
    run = HX.Run(batch, dims)
    assert run.layer.two_pass
    run.fused()
    res = run.results()
    # whole-tensor properties at full size: finite, masked entries (none here) zero
    assert np.isfinite(res["O"]).all() and np.isfinite(res["Ep"]).all()
    ref = OR.forward(batch, dims.H, bf16=True, rows=rows)
    HX.compare(res, ref, batch["mask"], dims, rows=ref["rows"])


@pytest.mark.parametrize("n", [12, 64, 192])
def test_forced_two_pass_matches_single(n):
    """The two-pass scheme gives the single-pass result (and the oracle's) at n = 12, 64, 192."""
    name = "sbm" if n == 192 else "planar"
    dims = dims_of(name, n=n, B=4)
    batch = W.make_batch(name, bias_scale=0.1, dims=dims)
    one = HX.Run(batch, dims).fused().results()
    two_run = HX.Run(batch, dims, force_two_pass=True)
    assert two_run.layer.two_pass
    two = two_run.fused().results()
    ref = OR.forward(batch, dims.H, bf16=True)
    for k in ("O", "Ep"):
        HX.assert_close(k, two[k], ref[k], "bf16")
        assert np.abs(two[k] - one[k]).max() <= HX.BF16_ABS_TOL
    HX.assert_masked_zero(two, batch["mask"], dims.H)


@pytest.mark.parametrize("n,dtype", [(37, "bf16"), (100, "bf16"), (250, "bf16"), (100, "fp32"), (1, "fp32"), (17, "fp32")])
def test_ragged_sizes_random_masks(n, dtype):
    """n not a multiple of 16 and arbitrary (non-prefix) node masks."""
    dims = dims_of("planar", n=n, B=3, dtype=dtype)
    batch = W.make_batch("tiny", bias_scale=0.2, dims=dims)  # Erdos-Renyi structure works for any n
    rng = np.random.default_rng(n)
    mask = (rng.random((3, n)) < 0.7).astype(np.uint8)
    mask[0] = 1
    mask[2] = 0 if n > 1 else mask[2]
    batch["mask"] = mask
    run_case("planar", dims, batch=batch)


@pytest.mark.parametrize("n,dtype", [(37, "bf16"), (250, "bf16"), (100, "fp32")])
def test_forced_two_pass_ragged_random_masks(n, dtype):
    """The two-pass scheme with n not a multiple of 16 and non-prefix node masks."""
    dims = dims_of("planar", n=n, B=3, dtype=dtype)
    batch = W.make_batch("tiny", bias_scale=0.2, dims=dims)
    rng = np.random.default_rng(1000 + n)
    mask = (rng.random((3, n)) < 0.7).astype(np.uint8)
    mask[0] = 1
    mask[2] = 0
    batch["mask"] = mask
    run_case("planar", dims, batch=batch, force_two_pass=True)


def test_all_masked_and_single_node_graphs():
    dims = dims_of("planar", n=20, B=3)
    batch = W.make_batch("planar", bias_scale=0.2, dims=dims)
    batch["mask"][:] = 0
    batch["mask"][1, 7] = 1          # one real node in the middle
    batch["mask"][2, :20] = 1
    _, res, _ = run_case("planar", dims, batch=batch)
    assert np.all(res["O"][0] == 0) and np.all(res["A"][0] == 0) and np.all(res["Ep"][0] == 0)
    assert np.all(res["A"][1, :, 7, 7] == 1.0)


def test_mask_enumeration_4096():
    """All 2^12 node subsets of one 12-node graph in a single B = 4096 launch."""
    n = 12
    dims = dims_of("tiny", B=4096)
    base = W.make_batch("tiny", bias_scale=0.2, dims=dims_of("tiny", B=1))
    subsets = np.arange(1 << n)
    mask = ((subsets[:, None] >> np.arange(n)[None, :]) & 1).astype(np.uint8)
    batch = {k: v for k, v in base.items()}
    batch["X"] = np.repeat(base["X"], 4096, 0)
    batch["E"] = np.repeat(base["E"], 4096, 0)
    batch["y"] = np.repeat(base["y"], 4096, 0)
    batch["mask"] = mask
    run_case("tiny", dims, batch=batch)


def test_nan_poisoned_padding_and_inputs_untouched():
    """NaN/Inf in padded X rows and E pairs change no output bit; inputs stay unchanged."""
    dims = dims_of("sbm", B=4)
    batch = W.make_batch("sbm", bias_scale=0.1, dims=dims)
    clean = HX.Run(batch, dims).fused().results()
    pois = dict(batch)
    pm = HX.pair_mask(batch["mask"])
    X = batch["X"].copy(); X[batch["mask"] == 0] = np.nan
    E = batch["E"].copy(); E[~pm] = np.inf; E[~pm, 1] = np.nan
    pois["X"], pois["E"] = X, E
    run = HX.Run(pois, dims)
    x0, e0 = run.dev["X"].clone(), run.dev["E"].clone()
    res = run.fused().results()
    for k in ("O", "A", "Ep"):
        assert np.array_equal(res[k], clean[k]), k
    assert torch.equal(run.dev["X"].isnan(), x0.isnan()) and torch.equal(run.dev["E"].isinf(), e0.isinf())
    assert torch.equal(torch.nan_to_num(run.dev["E"]), torch.nan_to_num(e0))


@pytest.mark.parametrize("mode,two", [("fused", False), ("separate", False), ("fused", True)])
def test_nan_poisoned_padding_one_tile_path(mode, two):
    """The one-tile fused path reads every in-bounds pair (masked ones too) and discards them by
    selects; NaN/Inf there, and in padded X rows, must change no output bit (also separate calls
    and the two-pass scheme)."""
    dims = dims_of("planar", B=4)
    batch = W.make_batch("planar", bias_scale=0.1, dims=dims)
    for g, k in enumerate([64, 50, 33, 1]):
        batch["mask"][g] = 0
        batch["mask"][g, :k] = 1
    run_clean = HX.Run(batch, dims, force_two_pass=two)
    clean = (run_clean.fused() if mode == "fused" else run_clean.separate()).results()
    pois = dict(batch)
    pm = HX.pair_mask(batch["mask"])
    X = batch["X"].copy(); X[batch["mask"] == 0] = np.nan
    E = batch["E"].copy(); E[~pm] = np.nan; E[~pm, 3] = -np.inf
    pois["X"], pois["E"] = X, E
    run = HX.Run(pois, dims, force_two_pass=two)
    res = (run.fused() if mode == "fused" else run.separate()).results()
    for k in clean:
        assert np.array_equal(res[k], clean[k]), k
    ref = OR.forward(batch, dims.H, bf16=True)
    HX.compare(res, ref, batch["mask"], dims)


def test_deterministic_and_in_place():
    """Bitwise run-to-run determinism; E_out aliasing E gives the out-of-place result."""
    dims = dims_of("planar", B=8)
    batch = W.make_batch("planar", bias_scale=0.1, dims=dims)
    r1 = HX.Run(batch, dims).fused().results()
    r2 = HX.Run(batch, dims).fused().results()
    for k in r1:
        assert np.array_equal(r1[k], r2[k]), k
    run = HX.Run(batch, dims)
    d = run.dev
    run.layer.layer(d, d["X"], d["E"], d["y"], d["mask"], run.O, run.A, d["E"], run.ws)
    torch.cuda.synchronize()
    assert np.array_equal(d["E"].float().cpu().numpy(), r1["Ep"])


def test_permutation_equivariance():
    dims = dims_of("planar", B=2)
    batch = W.make_batch("planar", bias_scale=0.1, dims=dims)
    perm = np.random.default_rng(0).permutation(dims.n)
    pb = dict(batch)
    pb["X"] = batch["X"][:, perm]
    pb["E"] = batch["E"][:, perm][:, :, perm]
    a = HX.Run(batch, dims).fused().results()
    p = HX.Run(pb, dims).fused().results()
    assert np.abs(p["O"] - a["O"][:, perm]).max() <= HX.BF16_ABS_TOL
    assert np.abs(p["A"] - a["A"][:, :, perm][:, :, :, perm]).max() <= HX.BF16_ABS_TOL
    assert np.abs(p["Ep"] - a["Ep"][:, perm][:, :, perm]).max() <= HX.BF16_ABS_TOL


@pytest.mark.gpu
@pytest.mark.parametrize("name,over,force", [("tiny", {}, True), ("planar", {"B": 2, "n": 100}, True),
                                             ("planar", {"B": 2, "n": 37}, True), ("planar", {"B": 1, "n": 300}, False)],
                         ids=["tiny-fp32", "n100-bf16", "n37-bf16", "n300-bf16"])
def test_two_pass_layer_writes_a(name, over, force):
    """A two-pass layer call given an A buffer returns the attention map too
    (written by the second pass, +0.0 at masked pairs), with O and E' as
    without it."""
    dims = dataclasses.replace(W.CONFIGS[name].dims, **over)
    batch = W.make_batch(name, bias_scale=0.1, dims=dims)
    if "n" in over:
        rng = np.random.default_rng(over["n"] + 1)
        mask = (rng.random((dims.B, dims.n)) < 0.8).astype(np.uint8)
        mask[0] = 1
        batch["mask"] = mask
    run = HX.Run(batch, dims, force_two_pass=force, keep_a=True)
    assert run.layer.two_pass
    res = run.fused().results()
    assert "A" in res
    ref = OR.forward(batch, dims.H, bf16=(dims.dtype == "bf16"))
    HX.compare(res, ref, batch["mask"], dims)
