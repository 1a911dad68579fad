"""Stacked layers (the sampling-loop benchmark's path) against the oracle
composed the same way: layer l + 1 takes layer l's O as X and E' as E;
stacked blocks: block l + 1 takes block l's X2, E2 and y2."""
import dataclasses

import numpy as np
import pytest
import torch

from edge_aware_graph_amd import workloads as W
from edge_aware_graph_amd.sampling import SamplingLoop
from oracle import block as OBK
from oracle import oracle as OR
from tests import _layer_harness as HX

pytestmark = pytest.mark.gpu


def layer_weights(dims, seeds):
    out = []
    for s in seeds:
        b = W.make_batch("tiny", seed=s, bias_scale=0.1, dims=dims)
        out.append({k: v for k, v in b.items() if k.startswith(("w_", "b_"))})
    return out


@pytest.mark.parametrize("name,over,L,T", [("tiny", {}, 2, 2), ("planar", {"B": 4, "n": 24, "dtype": "fp32"}, 3, 1)])
def test_stacked_layers_match_composed_oracle(name, over, L, T):
    dims = dataclasses.replace(W.CONFIGS[name].dims, **over)
    batch = W.make_batch(name, bias_scale=0.1, dims=dims)
    ws = layer_weights(dims, seeds=[100 + k for k in range(L)])
    dt = HX.tdtype(dims.dtype)
    dev_w = [{k: torch.from_numpy(v).to("cuda", dt) for k, v in w.items()} for w in ws]
    loop = SamplingLoop(dims, dev_w)
    up = HX.upload(batch, dims.dtype)
    Xg, Eg, _ = loop.run(up["X"], up["E"], up["y"], up["mask"], steps=T)
    torch.cuda.synchronize()
    # the oracle composed the same way, from the same inputs (float32 between layers)
    cur = dict(batch)
    for _ in range(T):
        for w in ws:
            step = dict(cur)
            step.update(w)
            ref = OR.forward(step, dims.H, bf16=False)
            cur = dict(cur)
            cur["X"] = ref["O"].astype(np.float32)
            cur["E"] = ref["Ep"].astype(np.float32)
    # float32 tolerance of one layer, per applied layer (errors add up)
    nl = L * T
    for got, want in ((Xg, cur["X"]), (Eg, cur["E"])):
        g = got.float().cpu().numpy().astype(np.float64)
        scale = max(np.abs(want).max(), 1e-30)
        assert np.abs(g - want).max() <= nl * HX.FP32_REL_TOL * scale
    HX.assert_masked_zero({"O": Xg.float().cpu().numpy(), "Ep": Eg.float().cpu().numpy()}, batch["mask"], dims.H)


@pytest.mark.parametrize("over,L,T", [({}, 2, 2), ({"B": 3, "n": 40}, 3, 1)], ids=["tiny", "n40-ragged"])
def test_stacked_blocks_match_composed_oracle(over, L, T):
    """Whole graph-transformer blocks stacked (float32, d = 64, de = dy = 16),
    ragged non-prefix masks in the second case."""
    dims = dataclasses.replace(W.CONFIGS["tiny"].dims, **over)
    batch = W.make_batch("tiny", bias_scale=0.1, dims=dims)
    if over:
        mask = (np.random.default_rng(40).random((dims.B, dims.n)) < 0.75).astype(np.uint8)
        mask[0] = 1
        batch["mask"] = mask
    ws = layer_weights(dims, seeds=[200 + k for k in range(L)])
    bps = [W.make_block_params(dims, seed=300 + k) for k in range(L)]
    dt = HX.tdtype(dims.dtype)
    dev_w = [{k: torch.from_numpy(v).to("cuda", dt) for k, v in w.items()} for w in ws]
    dev_bp = [{k: torch.from_numpy(np.ascontiguousarray(v)).to("cuda", dt) for k, v in bp.items()} for bp in bps]
    loop = SamplingLoop(dims, dev_w, block_params=dev_bp)
    up = HX.upload(batch, dims.dtype)
    Xg, Eg, yg = loop.run(up["X"], up["E"], up["y"], up["mask"], steps=T)
    torch.cuda.synchronize()
    cur = dict(batch)
    for _ in range(T):
        for w, bp in zip(ws, bps):
            step = dict(cur)
            step.update(w)
            ref = OBK.block(step, bp, dims.H, False)
            cur = dict(cur)
            cur["X"] = ref["X2"].astype(np.float32)
            cur["E"] = ref["E2"].astype(np.float32)
            cur["y"] = ref["y2"].astype(np.float32)
    nl = L * T
    for got, want in ((Xg, cur["X"]), (Eg, cur["E"]), (yg, cur["y"])):
        g = got.float().cpu().numpy().astype(np.float64)
        assert np.isfinite(g).all()
        scale = max(np.abs(want).max(), 1e-30)
        assert np.abs(g - want).max() <= nl * HX.FP32_REL_TOL * scale
    m = batch["mask"].astype(bool)
    pm = m[:, :, None] & m[:, None, :]
    X2, E2 = Xg.float().cpu().numpy(), Eg.float().cpu().numpy()
    assert np.all(X2[~m] == 0) and not np.any(np.signbit(X2[~m]))
    assert np.all(E2[~pm] == 0) and not np.any(np.signbit(E2[~pm]))
