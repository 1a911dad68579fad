"""The allocation-free entry point (edge_attn_layer_noalloc) against
edge_attn_layer on the same inputs: the same kernels run with the library's
own device array as their workspace, so every output must be bitwise equal.
Two calls in a row on different contexts, the second with a smaller input
(the array keeps the first call's contents), single pass and two-pass; a
context whose workspace exceeds the array is refused before any launch."""
import dataclasses
import sys

import numpy as np
import pytest
import torch

from edge_aware_graph_amd import layer as L
from edge_aware_graph_amd import workloads as W
from tests import _layer_harness as HX

pytestmark = pytest.mark.gpu


def _noalloc(run):
    d = run.dev
    dt = HX.tdtype(run.dims.dtype)
    B, n, dd, de, H = run.dims.B, run.dims.n, run.dims.d, run.dims.de, run.dims.H
    O = torch.full((B, n, dd), float("nan"), dtype=dt, device="cuda")
    A = None if run.layer.two_pass else torch.full((B, H, n, n), float("nan"), dtype=dt, device="cuda")
    Eo = torch.full((B, n, n, de), float("nan"), dtype=dt, device="cuda")
    run.layer.layer_noalloc(d, d["X"], d["E"], d["y"], d["mask"], O, A, Eo)
    torch.cuda.synchronize()
    out = {"O": O.float().cpu().numpy(), "Ep": Eo.float().cpu().numpy()}
    if A is not None:
        out["A"] = A.float().cpu().numpy()
    return out


def _case(name, **over):
    dims = dataclasses.replace(W.CONFIGS[name].dims, **over)
    batch = W.make_batch(name, bias_scale=0.1, dims=dims)
    return batch, dims


@pytest.mark.parametrize("first,second", [
    (("sbm", {"B": 8}), ("planar", {"B": 2})),                     # single pass, then a smaller batch
    (("planar", {"B": 8, "n": 300}), ("tiny", {})),                # two-pass, then the tiny float32 batch
    (("planar", {"B": 4, "d": 512, "dh": 64}), ("planar", {"B": 1, "n": 20})),  # generic path, then tuned
])
def test_noalloc_matches_layer_twice(first, second):
    print("\n[case] noalloc %s then %s" % (first, second), flush=True)
    sys.stdout.flush()
    for name, over in (first, second):
        batch, dims = _case(name, **over)
        if over.get("n") == 300:
            batch = W.make_batch("tiny", bias_scale=0.1, dims=dims)
        ref_run = HX.Run(batch, dims).fused()
        ref = ref_run.results()
        got = _noalloc(HX.Run(batch, dims))
        assert set(got) == set(ref)
        for k in ref:
            assert np.array_equal(got[k], ref[k]), (name, over, k)


def test_noalloc_refuses_a_workspace_beyond_the_array():
    lib = L.load_library()
    cap = int(lib.ea_noalloc_max_workspace_bytes())
    assert cap == 16 << 20
    dims = dataclasses.replace(W.CONFIGS["planar"].dims, B=512, n=64)  # workspace ~ 48 MiB
    layer = L.EdgeAttention(dims.B, dims.n, dims.d, dims.de, dims.dy, dims.H, dims.dh, dims.dtype)
    assert layer.workspace_bytes > cap
    dt = torch.bfloat16
    w = {k: torch.zeros(tuple(v), dtype=dt, device="cuda") for k, v in
         (("w_q", (256, 256)), ("w_k", (256, 256)), ("w_v", (256, 256)), ("w_emul", (8, 64)), ("w_eadd", (8, 64)),
          ("w_ymul", (8, 64)), ("w_yadd", (8, 64)), ("w_e", (64, 8)))}
    small = {"X": (dims.B, 64, 256), "E": (dims.B, 64, 64, 64), "y": (dims.B, 64), "O": (dims.B, 64, 256),
             "A": (dims.B, 8, 64, 64), "Eo": (dims.B, 64, 64, 64)}
    t = {k: torch.zeros(v, dtype=dt, device="cuda") for k, v in small.items()}
    m = torch.ones(dims.B, 64, dtype=torch.uint8, device="cuda")
    with pytest.raises(L.EaError) as ei:
        layer.layer_noalloc(w, t["X"], t["E"], t["y"], m, t["O"], t["A"], t["Eo"])
    assert ei.value.status == L.EA_E_WORKSPACE and "at most" in str(ei.value)
