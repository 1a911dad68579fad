"""GPU parity of the generic path: shapes the boundary accepts (head width
16, 32 or 64, edge width a multiple of 16, 2H <= 32) that have no tuned
kernels run through the same C ABI on one block per query row. Every case is
checked against the oracle on full tensors under the layer's tolerances
(float32 1e-4 normwise relative, bfloat16 2e-2 absolute, masked outputs
+0.0 bitwise): single pass, the two-pass scheme (forced and natural),
separate forward and edge_update calls, ragged non-prefix masks, the
ablation variants, NaN-poisoned padding, and the two stage exports (logits,
and the softmax from given logits).
"""
import sys

import numpy as np
import pytest
import torch

from edge_aware_graph_amd import layer as L
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


def gdims(H, dh, de, dtype, B=3, n=40, dy=16):
    return W.LayerDims(B=B, n=n, d=H * dh, de=de, dy=dy, H=H, dh=dh, dtype=dtype)


def ragged(batch, n, seed, full_first=True):
    rng = np.random.default_rng(seed)
    B = batch["mask"].shape[0]
    mask = (rng.random((B, n)) < 0.7).astype(np.uint8)
    if full_first:
        mask[0] = 1
    if B > 2:
        mask[2] = 0
    batch["mask"] = mask
    return batch


def check(batch, dims, force_two_pass=False, mode="fused"):
    run = HX.Run(batch, dims, force_two_pass=force_two_pass)
    (run.fused() if mode == "fused" else run.separate())
    res = run.results()
    ref = OR.forward(batch, dims.H, bf16=(dims.dtype == "bf16"))
    HX.compare(res, ref, batch["mask"], dims)
    return run, res


SHAPES = [  # (H, dh, de, dtype, name)
    (8, 64, 64, "bf16", "planar"),   # d = 512
    (4, 32, 32, "fp32", "tiny"),
    (4, 32, 32, "bf16", "tiny"),
    (16, 16, 16, "bf16", "tiny"),    # 2H = 32
    (2, 16, 48, "fp32", "tiny"),     # H not a multiple of 4, de = 48
    (1, 64, 16, "bf16", "tiny"),
    (16, 64, 128, "fp32", "tiny"),   # d = 1024, de = 128
]
SHAPE_IDS = ["H%d-dh%d-de%d-%s" % s[:4] for s in SHAPES]


def test_boundary_takes_the_generic_path():
    for H, dh, de, dtype, _ in SHAPES:
        dims = gdims(H, dh, de, dtype)
        run = HX.Run(W.make_batch("tiny", bias_scale=0.1, dims=dims), dims)
        assert run.layer.workspace_bytes > 0


@pytest.mark.parametrize("shape", SHAPES, ids=SHAPE_IDS)
@pytest.mark.parametrize("mode", ["fused", "separate"])
def test_generic_single_pass(shape, mode):
    H, dh, de, dtype, name = shape
    n = 64 if name == "planar" else 37
    dims = gdims(H, dh, de, dtype, B=4 if name == "planar" else 3, n=n)
    batch = W.make_batch(name if name == "planar" else "tiny", bias_scale=0.1, dims=dims)
    if name != "planar":
        ragged(batch, n, seed=H * 100 + dh + de)
    check(batch, dims, mode=mode)


@pytest.mark.parametrize("shape", SHAPES[:5], ids=SHAPE_IDS[:5])
@pytest.mark.parametrize("mode", ["fused", "separate"])
def test_generic_forced_two_pass(shape, mode):
    H, dh, de, dtype, _ = shape
    dims = gdims(H, dh, de, dtype, B=3, n=70)
    batch = ragged(W.make_batch("tiny", bias_scale=0.2, dims=dims), 70, seed=7 + H)
    run, _ = check(batch, dims, force_two_pass=True, mode=mode)
    assert run.layer.two_pass


def test_generic_natural_two_pass():
    """n = 300 > 256 takes the two-pass scheme; the generic rows walk 2 chunks of keys."""
    dims = gdims(4, 32, 32, "bf16", B=2, n=300, dy=8)
    batch = ragged(W.make_batch("tiny", bias_scale=0.1, dims=dims), 300, seed=3)
    run, _ = check(batch, dims)
    assert run.layer.two_pass


def test_generic_rows_longer_than_a_chunk_single_pass():
    """n = 256 in one pass: the generic rows still walk several chunks of keys? (one of 256)."""
    dims = gdims(8, 64, 64, "bf16", B=1, n=256, dy=8)
    batch = ragged(W.make_batch("tiny", bias_scale=0.1, dims=dims), 256, seed=5)
    check(batch, dims)


VARIANTS = {
    "light_edge": (L.EA_VARIANT_LIGHT_EDGE, OR.LIGHT_EDGE, ("w_emul", "w_eadd", "b_emul", "b_eadd")),
    "no_score_mod": (L.EA_VARIANT_NO_SCORE_MOD, OR.NO_SCORE_MOD,
                     ("w_emul", "w_eadd", "b_emul", "b_eadd", "w_ymul", "w_yadd", "b_ymul", "b_yadd", "y")),
    "unnormalized": (L.EA_VARIANT_UNNORMALIZED, OR.UNNORMALIZED, ()),
}


@pytest.mark.parametrize("variant", list(VARIANTS))
@pytest.mark.parametrize("two", [False, True])
@pytest.mark.parametrize("mode", ["fused", "separate"])
def test_generic_variants(variant, two, mode):
    flag, obits, drop = VARIANTS[variant]
    dims = gdims(2, 32, 16, "fp32", B=3, n=30)
    batch = ragged(W.make_batch("tiny", bias_scale=0.2, dims=dims), 30, seed=11)
    run = HX.Run(batch, dims, force_two_pass=two, variant=flag, drop=drop)
    (run.fused() if mode == "fused" else run.separate())
    res = run.results()
    ref = OR.forward(batch, dims.H, bf16=False, variant=obits)
    HX.compare(res, ref, batch["mask"], dims)


@pytest.mark.parametrize("two", [False, True])
def test_generic_nan_poisoned_padding(two):
    dims = gdims(4, 32, 32, "bf16", B=3, n=33)
    batch = ragged(W.make_batch("tiny", bias_scale=0.1, dims=dims), 33, seed=19)
    clean = HX.Run(batch, dims, force_two_pass=two).fused().results()
    pois = dict(batch)
    pm = HX.pair_mask(batch["mask"])
    X = batch["X"].copy(); X[batch["mask"] == 0] = np.nan
    E = batch["E"].copy(); E[~pm] = np.nan; E[~pm, 2] = np.inf
    pois["X"], pois["E"] = X, E
    res = HX.Run(pois, dims, force_two_pass=two).fused().results()
    for k in clean:
        assert np.array_equal(res[k], clean[k]), k


def test_generic_in_place_update():
    dims = gdims(8, 64, 64, "bf16", B=2, n=48)
    batch = W.make_batch("tiny", bias_scale=0.1, dims=dims)
    ref = HX.Run(batch, dims).fused().results()
    run = HX.Run(batch, dims)
    d = run.dev
    run.layer.layer(d, d["X"], d["E"], d["y"], d["mask"], run.O, run.A, d["E"], run.ws)
    torch.cuda.synchronize()
    assert np.array_equal(d["E"].float().cpu().numpy(), ref["Ep"])


@pytest.mark.parametrize("H,dh,de,dtype,n", [(8, 64, 64, "bf16", 40), (2, 16, 48, "fp32", 300)])
def test_generic_logit_stage(H, dh, de, dtype, n):
    dims = gdims(H, dh, de, dtype, B=2, n=n, dy=8)
    batch = ragged(W.make_batch("tiny", bias_scale=0.1, dims=dims), n, seed=23)
    U = HX.Run(batch, dims).logits()
    ref = OR.forward(batch, dims.H, bf16=(dtype == "bf16"))["U"]
    fin = np.isfinite(ref)
    assert np.array_equal(np.isneginf(U), ~fin)
    err = np.abs(U[fin] - ref[fin]).max()
    assert err <= (1e-4 if dtype == "fp32" else 1e-3) * max(np.abs(ref[fin]).max(), 1.0)


@pytest.mark.parametrize("name,over", [("tiny", {}), ("planar", {"B": 2}), ("sbm", {"B": 2}),
                                        ("gen", {})])
def test_softmax_stage(name, over):
    """ea_debug_softmax: the softmax stage alone, fed the oracle's own logits
    (float32, -inf at masked pairs), against the oracle's A; rows without a
    real key give 0, masked entries +0.0."""
    if name == "gen":
        dims = gdims(16, 16, 16, "bf16", B=2, n=300, dy=8)
        batch = ragged(W.make_batch("tiny", bias_scale=0.1, dims=dims), 300, seed=29)
    else:
        import dataclasses
        dims = dataclasses.replace(W.CONFIGS[name].dims, **over)
        batch = W.make_batch(name, bias_scale=0.1, dims=dims)
    ref = OR.forward(batch, dims.H, bf16=(dims.dtype == "bf16"))
    layer = L.EdgeAttention(dims.B, dims.n, dims.d, dims.de, dims.dy, dims.H, dims.dh, dims.dtype)
    U = torch.from_numpy(ref["U"].astype(np.float32)).cuda()
    A = torch.full(U.shape, float("nan"), dtype=HX.tdtype(dims.dtype), device="cuda")
    layer.debug_softmax(U, A)
    got = A.float().cpu().numpy()
    # the oracle's A is the softmax of its float64 logits; fed their float32
    # rounding, the result moves by at most a few float32 ulps of the logits
    HX.assert_close("A", got, ref["A"], dims.dtype)
    HX.assert_masked_zero({"A": got}, batch["mask"], dims.H)
