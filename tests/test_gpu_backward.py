"""Backward of the layer on the GPU against the backward oracle (autograd of
the definition, pinned by finite differences of the C oracle).

Tolerances, per tensor, relative to the tensor's largest reference value:
float32 1e-4 (the layer's float32 tolerance); bfloat16 2e-2. In bfloat16 both
sides take the softmax Jacobian at the stored (rounded) A (the oracle's
reading, pinned on the CPU against torch's softmax backward handed that A and
against finite differences where the rounding is exact); the GPU also rounds
dO . V-side and FiLM-side intermediates to bfloat16 as MFMA operands and
stores dX, dE and dy in bfloat16: each step is a relative error of about
2^-8, a few of them in a chain. Masked pairs' dE and padded rows' dX are +0.0
bit-exactly.
"""
import dataclasses

import numpy as np
import pytest
import torch

from edge_aware_graph_amd import workloads as W
from oracle import backward as OB
from tests import _layer_harness as HX

pytestmark = pytest.mark.gpu

GRAD_NAMES = ("w_q", "w_k", "w_v", "b_q", "b_k", "b_v", "w_emul", "w_eadd", "b_emul", "b_eadd",
              "w_ymul", "w_yadd", "b_ymul", "b_yadd", "w_e", "b_e")


def dims_of(name, **over):
    return dataclasses.replace(W.CONFIGS[name].dims, **over)


def run_backward(batch, dims, seed=0, force_two_pass=False, keep_a=False):
    dt = HX.tdtype(dims.dtype)
    run = HX.Run(batch, dims, force_two_pass=force_two_pass, keep_a=keep_a)
    run.fused()
    B, n, d, de, H, dy = dims.B, dims.n, dims.d, dims.de, dims.H, dims.dy
    rng = np.random.default_rng(seed)
    dO = rng.standard_normal((B, n, d)).astype(np.float32)
    dEp = rng.standard_normal((B, n, n, de)).astype(np.float32)
    if dims.dtype == "bf16":
        dO, dEp = W.bf16_round_array(dO), W.bf16_round_array(dEp)
    dev = run.dev
    t_dO = torch.from_numpy(dO).to("cuda", dt)
    t_dEp = torch.from_numpy(dEp).to("cuda", dt)
    dX = torch.full((B, n, d), float("nan"), dtype=dt, device="cuda")
    dE = torch.full((B, n, n, de), float("nan"), dtype=dt, device="cuda")
    dyv = torch.full((B, dy), float("nan"), dtype=dt, device="cuda")
    grads = {k: torch.full(tuple(batch[k].shape), float("nan"), dtype=torch.float32, device="cuda") for k in GRAD_NAMES}
    bws = torch.empty(run.layer.backward_workspace_bytes, dtype=torch.uint8, device="cuda")
    run.layer.backward(dev, dev["X"], dev["E"], dev["y"], dev["mask"], run.A, t_dO, t_dEp, dX, dE, dyv,
                       grads, run.ws, bws)
    torch.cuda.synchronize()
    got = {"X": dX.float().cpu().numpy(), "E": dE.float().cpu().numpy(), "y": dyv.float().cpu().numpy()}
    got.update({k: v.cpu().numpy() for k, v in grads.items()})
    ref = OB.backward(batch, dO.astype(np.float64), dEp.astype(np.float64), dims.H, bf16=(dims.dtype == "bf16"))
    return got, ref


# Gradients that vanish identically in float32: beta_e and beta_y add a
# constant to each softmax row (their bias and global weights get
# sum_j du = 0), so the GPU returns rounding noise of sums whose terms are as
# large as those of their gamma siblings; their scale is the sibling's. (In
# bfloat16 the stored A does not sum to exactly 1 and they are small but not
# zero, the same on both sides.)
ZERO_SIBLING = {"b_eadd": "b_emul", "b_yadd": "b_ymul", "w_yadd": "w_ymul"}


def check(got, ref, batch, dims):
    tol = 1e-4 if dims.dtype == "fp32" else 2e-2
    for k in ref:
        g = got[k].astype(np.float64)
        assert g.shape == ref[k].shape, k
        assert np.isfinite(g).all(), "%s has non-finite values" % k
        scale = max(np.abs(ref[k]).max(), 1e-6)
        if k in ZERO_SIBLING:
            if dims.dtype == "fp32":
                assert np.abs(ref[k]).max() < 1e-9, k
            scale = max(scale, np.abs(ref[ZERO_SIBLING[k]]).max())
        err = np.abs(g - ref[k]).max()
        assert err <= tol * scale, "%s: max err %.3e > %.0e * %.3e" % (k, err, tol, scale)
    m = batch["mask"].astype(bool)
    pm = m[:, :, None] & m[:, None, :]
    assert np.all(got["E"][~pm] == 0) and not np.any(np.signbit(got["E"][~pm]))
    assert np.all(got["X"][~m] == 0) and not np.any(np.signbit(got["X"][~m]))


@pytest.mark.parametrize("name,over", [("tiny", {}), ("tiny", {"dtype": "bf16"}), ("planar", {"B": 4})],
                         ids=["tiny-fp32", "tiny-bf16", "planar-bf16"])
def test_backward_matches_autograd_oracle(name, over):
    dims = dims_of(name, **over)
    batch = W.make_batch(name, bias_scale=0.1, dims=dims)
    got, ref = run_backward(batch, dims)
    check(got, ref, batch, dims)


@pytest.mark.parametrize("n,dtype", [(37, "bf16"), (50, "bf16"), (17, "fp32")])
def test_backward_ragged_random_masks(n, dtype):
    over = {"n": n, "B": 3, "dtype": dtype}
    if dtype == "fp32":
        dims = dims_of("tiny", **over)
    else:
        dims = dims_of("planar", **over)
    batch = W.make_batch("tiny", bias_scale=0.2, dims=dims)
    rng = np.random.default_rng(n)
    mask = (rng.random((3, n)) < 0.7).astype(np.uint8)
    mask[0] = 1
    mask[2] = 0
    batch["mask"] = mask
    got, ref = run_backward(batch, dims, seed=n)
    check(got, ref, batch, dims)


@pytest.mark.parametrize("n,dtype,B", [(100, "bf16", 2), (192, "bf16", 2), (256, "bf16", 1), (100, "fp32", 2)])
def test_backward_several_key_blocks(n, dtype, B):
    """64 < n <= 256 (single pass): the pair kernel runs over key blocks of 64,
    the row sums D_i in a first pass; dQ, dK, dV over contraction chunks.
    Ragged random masks with one graph fully real."""
    over = {"n": n, "B": B, "dtype": dtype}
    dims = dims_of("tiny" if dtype == "fp32" else "planar", **over)
    batch = W.make_batch("tiny", bias_scale=0.2, dims=dims)
    rng = np.random.default_rng(1000 + n)
    mask = (rng.random((B, n)) < 0.75).astype(np.uint8)
    mask[0] = 1
    batch["mask"] = mask
    got, ref = run_backward(batch, dims, seed=n)
    check(got, ref, batch, dims)


@pytest.mark.parametrize("n,dtype,n_real,two_pass", [
    (192, "bf16", (44, 100, 187), False), (40, "fp32", (5, 20, 40), False), (100, "bf16", (9, 70), True)],
    ids=["sbm-like-bf16", "n40-fp32", "n100-two-pass-bf16"])
def test_backward_prefix_masks_padded_tiles(n, dtype, n_real, two_pass):
    """SBM-style padding: graphs of n_real nodes padded to n with prefix masks,
    so that whole 16 x 16 pair tiles hold no real pair (zeros only) next to
    partial and full ones."""
    B = len(n_real)
    over = {"n": n, "B": B, "dtype": dtype}
    dims = dims_of("tiny" if dtype == "fp32" else "planar", **over)
    batch = W.make_batch("tiny", bias_scale=0.2, dims=dims)
    mask = np.zeros((B, n), np.uint8)
    for b, k in enumerate(n_real):
        mask[b, :k] = 1
    batch["mask"] = mask
    got, ref = run_backward(batch, dims, seed=n + 1, force_two_pass=two_pass)
    check(got, ref, batch, dims)


@pytest.mark.parametrize("name,over", [("tiny", {}), ("tiny", {"dtype": "bf16"}), ("planar", {"B": 2, "n": 100}),
                                       ("planar", {"B": 2, "n": 37})],
                         ids=["tiny-fp32", "tiny-bf16", "n100-bf16", "n37-bf16"])
def test_backward_forced_two_pass(name, over):
    """Two-pass contexts keep no A: the backward recomputes it as exp(u - lse)
    from the forward's row statistics (forced two-pass at small n). With n =
    37 the rows of the n x n map are not multiples of four keys, so A is
    stored and read back one key at a time."""
    dims = dims_of(name, **over)
    batch = W.make_batch(name, bias_scale=0.1, dims=dims)
    if "n" in over:
        rng = np.random.default_rng(7)
        mask = (rng.random((dims.B, dims.n)) < 0.8).astype(np.uint8)
        mask[0] = 1
        batch["mask"] = mask
    got, ref = run_backward(batch, dims, force_two_pass=True)
    check(got, ref, batch, dims)


@pytest.mark.parametrize("name,over,force", [("tiny", {}, True), ("planar", {"B": 2, "n": 100}, True),
                                             ("planar", {"B": 2, "n": 37}, True), ("planar", {"B": 1, "n": 300}, False)],
                         ids=["tiny-fp32", "n100-bf16", "n37-bf16", "n300-bf16"])
def test_backward_two_pass_with_stored_a(name, over, force):
    """Two-pass contexts given an A buffer: the layer's second pass writes A,
    and the backward, handed that buffer, uses it instead of recomputing it."""
    dims = dims_of(name, **over)
    batch = W.make_batch(name, bias_scale=0.1, dims=dims)
    if "n" in over:
        rng = np.random.default_rng(over["n"])
        mask = (rng.random((dims.B, dims.n)) < 0.8).astype(np.uint8)
        mask[0] = 1
        batch["mask"] = mask
    got, ref = run_backward(batch, dims, seed=5, force_two_pass=force, keep_a=True)
    check(got, ref, batch, dims)


def test_backward_natural_two_pass_n300():
    """n = 300 > 256: the layer runs two passes, the backward recomputes A."""
    dims = dims_of("planar", B=1, n=300)
    batch = W.make_batch("planar", bias_scale=0.1, dims=dims)
    rng = np.random.default_rng(300)
    batch["mask"] = (rng.random((1, 300)) < 0.85).astype(np.uint8)
    got, ref = run_backward(batch, dims, seed=3)
    check(got, ref, batch, dims)


def test_backward_large_full_size_sampled_rows():
    """The large configuration at its full size (B = 4, n = 1024, bfloat16; the
    layer runs two passes and the backward recomputes A), as the training
    benchmark launches it: dE on sampled query rows of every graph against
    the row-restricted oracle (each row's edge gradient depends on that row
    alone), 2e-2 of the largest reference value over the samples; every
    gradient finite."""
    dims = dims_of("large")
    batch = W.make_batch("large", bias_scale=0.1)
    sampled_rows_check(batch, dims)


def test_backward_more_than_16_key_blocks_sampled_rows():
    """n = 1040 (17 key blocks of 64): the second pair pass sums the key
    blocks' parts of D in its loop form rather than from the parts requested
    ahead of the tiles (at most 16); checked like the large configuration on
    sampled rows of one graph with a ragged mask."""
    dims = dims_of("large", B=1, n=1040)
    batch = W.make_batch("large", bias_scale=0.1, dims=dims)
    rng = np.random.default_rng(1040)
    batch["mask"] = (rng.random((1, 1040)) < 0.9).astype(np.uint8)
    batch["mask"][0, [0, 1039]] = 1
    sampled_rows_check(batch, dims)


def sampled_rows_check(batch, dims):
    run = HX.Run(batch, dims)
    assert run.layer.two_pass
    run.fused()
    B, n, d, de, dy = dims.B, dims.n, dims.d, dims.de, dims.dy
    rng = np.random.default_rng(11)
    dO = W.bf16_round_array(rng.standard_normal((B, n, d), dtype=np.float32))
    dEp = W.bf16_round_array(rng.standard_normal((B, n, n, de), dtype=np.float32))
    dt = HX.tdtype(dims.dtype)
    t_dO = torch.from_numpy(dO).to("cuda", dt)
    t_dEp = torch.from_numpy(dEp).to("cuda", dt)
    dX = torch.full((B, n, d), float("nan"), dtype=dt, device="cuda")
    dE = torch.full((B, n, n, de), float("nan"), dtype=dt, device="cuda")
    dyv = torch.full((B, dy), float("nan"), dtype=dt, device="cuda")
    grads = {k: torch.full(tuple(batch[k].shape), float("nan"), dtype=torch.float32, device="cuda")
             for k in GRAD_NAMES}
    bws = torch.empty(run.layer.backward_workspace_bytes, dtype=torch.uint8, device="cuda")
    dev = run.dev
    run.layer.backward(dev, dev["X"], dev["E"], dev["y"], dev["mask"], None, t_dO, t_dEp, dX, dE, dyv,
                       grads, run.ws, bws)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(dE).all()) and bool(torch.isfinite(dX).all()) and bool(torch.isfinite(dyv).all())
    for k, v in grads.items():
        assert bool(torch.isfinite(v).all()), k
    for b in range(B):
        rows = [0, int(rng.integers(1, n - 1)), n - 1]
        ref = OB.edge_grad_rows(batch, dO, dEp, dims.H, True, b, rows)
        got = dE[b, rows].float().cpu().numpy().astype(np.float64)
        scale = max(np.abs(ref).max(), 1e-6)
        err = np.abs(got - ref).max()
        assert err <= 2e-2 * scale, "graph %d rows %s: max err %.3e > 2e-2 * %.3e" % (b, rows, err, scale)


@pytest.mark.parametrize("name,over,two_pass", [("planar", {"B": 4}, False), ("tiny", {"dtype": "fp32"}, False),
                                               ("sbm", {"B": 2}, False), ("planar", {"B": 2}, True)],
                         ids=["planar-bf16", "tiny-fp32", "sbm-bf16", "planar-two-pass"])
def test_backward_bitwise_repeatable(name, over, two_pass):
    """Three identical backward calls give the same bits in every gradient:
    nothing is summed with atomics (each block writes its partial sums to a
    slot of its own, and the slots are added in a fixed order)."""
    dims = dims_of(name, **over)
    batch = W.make_batch(name, bias_scale=0.1, dims=dims)
    runs = [run_backward(batch, dims, seed=3, force_two_pass=two_pass)[0] for _ in range(3)]
    for k in runs[0]:
        for r in runs[1:]:
            assert np.array_equal(runs[0][k], r[k], equal_nan=False), k
