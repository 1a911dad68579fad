"""Pins of the block oracle (oracle/block.py) against library routines,
closed forms and invariants (CPU only).

The block's structure is a reading (the pages keep the graph transformer's
block around the new attention without writing it out); these tests pin the
oracle to that reading: torch's layer_norm, linear and bfloat16 conversion
for its helpers, the stages composed through torch calls, and properties
that any correct implementation has (mask and permutation invariance, the
final normalization, closed forms when parts are switched off).
"""
import dataclasses

import numpy as np
import pytest
import torch

from edge_aware_graph_amd import workloads as W
from oracle import block as OBK
from oracle import oracle as OR

pytestmark = pytest.mark.filterwarnings("ignore")


def _tiny(seed=3, mask=None):
    cfg = W.CONFIGS["tiny"]
    batch = W.make_batch("tiny", seed=seed, bias_scale=0.2)
    if mask is not None:
        batch["mask"] = mask.astype(np.uint8)
        pm = (batch["mask"][:, :, None] & batch["mask"][:, None, :]).astype(bool)
        batch["E"] = np.where(pm[..., None], batch["E"], 0.0).astype(np.float32)
        batch["X"] = np.where(batch["mask"][..., None] > 0, batch["X"], 0.0).astype(np.float32)
    return cfg, batch


def _params(cfg, scale=0.1, seed=7):
    return W.make_block_params(cfg.dims, seed=seed, scale=scale)


def test_layer_norm_matches_torch():
    rng = np.random.default_rng(0)
    z = rng.standard_normal((5, 7, 33)) * 3 + 1
    g, b = rng.standard_normal(33), rng.standard_normal(33)
    ref = torch.nn.functional.layer_norm(torch.tensor(z), (33,), torch.tensor(g), torch.tensor(b), eps=1e-5)
    np.testing.assert_allclose(OBK.layer_norm(z, g, b), ref.numpy(), rtol=1e-12, atol=1e-12)


def test_linear_orientation_matches_torch():
    rng = np.random.default_rng(1)
    x, w, b = rng.standard_normal((4, 6)), rng.standard_normal((3, 6)), rng.standard_normal(3)
    ref = torch.nn.functional.linear(torch.tensor(x), torch.tensor(w), torch.tensor(b))
    np.testing.assert_allclose(OBK.linear(x, w, b), ref.numpy(), rtol=1e-13)


def test_bf16_matches_torch():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(10000) * 10.0 ** rng.integers(-3, 4, 10000)).astype(np.float32)
    ref = torch.tensor(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(OBK.bf16(x), ref)


@pytest.mark.parametrize("bf16", [False, True])
def test_stages_compose_through_torch(bf16):
    """Each stage of the block recomputed from the oracle's own intermediates
    with torch.nn.functional calls (pins operand orientation and order)."""
    cfg, batch = _tiny()
    bp = _params(cfg)
    out = OBK.block(batch, bp, cfg.dims.H, bf16)
    F = torch.nn.functional
    t = lambda a: torch.tensor(np.asarray(a, np.float64))
    r = (lambda a: t(a).to(torch.bfloat16).to(torch.float64)) if bf16 else t
    ln = lambda z, k: F.layer_norm(z, (z.shape[-1],), t(bp["ln_%s_g" % k]), t(bp["ln_%s_b" % k]), eps=1e-5)
    m = t(batch["mask"]).bool()
    pm = m[:, :, None] & m[:, None, :]
    lay = OR.forward(batch, cfg.dims.H, bf16)
    np.testing.assert_allclose(out["O"], r(lay["O"]).numpy(), rtol=0, atol=0)
    X1 = ln(t(batch["X"]) + F.linear(t(out["O"]), t(bp["w_o"]), t(bp["b_o"])), "x1")
    Hx = F.relu(F.linear(r(X1), t(bp["w_x1"]), t(bp["b_x1"])))
    X2 = ln(X1 + F.linear(r(Hx), t(bp["w_x2"]), t(bp["b_x2"])), "x2") * m[..., None]
    E1 = ln(t(out["Ep"]), "e1")
    He = F.relu(F.linear(r(E1), t(bp["w_e1"]), t(bp["b_e1"])))
    E2 = ln(E1 + F.linear(r(He), t(bp["w_e2"]), t(bp["b_e2"])), "e2") * pm[..., None]
    nr = m.sum(1).double()
    xbar = X2.sum(1) / nr[:, None]
    ebar = E2.sum((1, 2)) / (nr * nr)[:, None]
    yv = t(batch["y"])
    y1 = ln(yv + F.linear(yv, t(bp["w_yy"])) + F.linear(xbar, t(bp["w_yx"])) +
            F.linear(ebar, t(bp["w_ye"]), t(bp["b_yo"])), "y1")
    y2 = ln(y1 + F.linear(F.relu(F.linear(y1, t(bp["w_y1"]), t(bp["b_y1"]))), t(bp["w_y2"]), t(bp["b_y2"])), "y2")
    for k, v in (("X1", X1), ("X2", X2), ("E1", E1), ("E2", E2), ("xbar", xbar), ("ebar", ebar),
                 ("y1", y1), ("y2", y2)):
        np.testing.assert_allclose(out[k], v.numpy(), rtol=1e-10, atol=1e-10, err_msg=k)


def test_masked_graph_equals_induced_subgraph():
    """A graph with masked (non-prefix) nodes gives, on its real nodes, the
    block of the subgraph induced by them: the means divide by the real count
    and masked rows and pairs contribute nothing."""
    cfg = W.CONFIGS["tiny"]
    n = cfg.dims.n
    mask = np.zeros((cfg.dims.B, n), np.uint8)
    keep = np.array([0, 2, 3, 5, 8, 9, 11])
    mask[:, keep] = 1
    _, batch = _tiny(seed=5, mask=mask)
    bp = _params(cfg)
    full = OBK.block(batch, bp, cfg.dims.H)
    k = len(keep)
    sub = {kk: v for kk, v in batch.items()}
    sub["X"] = batch["X"][:, keep]
    sub["E"] = batch["E"][:, keep][:, :, keep]
    sub["mask"] = np.ones((cfg.dims.B, k), np.uint8)
    sub["adj"] = batch["adj"][:, keep][:, :, keep]
    part = OBK.block(sub, bp, cfg.dims.H)
    np.testing.assert_allclose(full["X2"][:, keep], part["X2"], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(full["E2"][:, keep][:, :, keep], part["E2"], rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(full["y2"], part["y2"], rtol=1e-10, atol=1e-10)
    off = np.setdiff1d(np.arange(n), keep)
    assert np.all(full["X2"][:, off] == 0) and np.all(full["E2"][:, off] == 0) and np.all(full["E2"][:, :, off] == 0)


def test_permutation_equivariance():
    cfg, batch = _tiny(seed=9)
    bp = _params(cfg)
    base = OBK.block(batch, bp, cfg.dims.H)
    perm = np.random.default_rng(4).permutation(cfg.dims.n)
    pb = dict(batch)
    pb["X"] = batch["X"][:, perm]
    pb["E"] = batch["E"][:, perm][:, :, perm]
    pb["mask"] = batch["mask"][:, perm]
    pb["adj"] = batch["adj"][:, perm][:, :, perm]
    out = OBK.block(pb, bp, cfg.dims.H)
    np.testing.assert_allclose(out["X2"], base["X2"][:, perm], rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(out["E2"], base["E2"][:, perm][:, :, perm], rtol=1e-9, atol=1e-9)
    np.testing.assert_allclose(out["y2"], base["y2"], rtol=1e-9, atol=1e-9)


def test_outputs_are_normalized():
    """Unit gains and zero shifts: every real row of X2, real pair of E2 and
    every y2 has mean 0 and variance var / (var + eps), i.e. within 1e-3 of 1."""
    cfg, batch = _tiny(seed=11)
    bp = _params(cfg, scale=0.0)
    out = OBK.block(batch, bp, cfg.dims.H)
    m = batch["mask"].astype(bool)
    pm = m[:, :, None] & m[:, None, :]
    for v in (out["X2"][m], out["E2"][pm], out["y2"]):
        np.testing.assert_allclose(v.mean(-1), 0.0, atol=1e-12)
        np.testing.assert_allclose(v.var(-1), 1.0, atol=1e-3)


def test_closed_forms_with_parts_switched_off():
    cfg, batch = _tiny(seed=13)
    bp = _params(cfg)
    # node hidden layer killed by a large negative bias: X2 = LN(X1 + b_x2)
    q = dict(bp, b_x1=np.full_like(bp["b_x1"], -1e6))
    out = OBK.block(batch, q, cfg.dims.H)
    m = batch["mask"].astype(bool)
    assert np.all(out["Hx"] == 0)
    ref = OBK.layer_norm(out["X1"] + bp["b_x2"], bp["ln_x2_g"], bp["ln_x2_b"])
    np.testing.assert_allclose(out["X2"][m], ref[m], rtol=1e-12, atol=1e-12)
    # no edge feed-forward output: E2 = LN_e2(LN_e1(E'))
    q = dict(bp, w_e2=np.zeros_like(bp["w_e2"]), b_e2=np.zeros_like(bp["b_e2"]))
    out = OBK.block(batch, q, cfg.dims.H)
    pm = m[:, :, None] & m[:, None, :]
    ref = OBK.layer_norm(OBK.layer_norm(out["Ep"], bp["ln_e1_g"], bp["ln_e1_b"]), bp["ln_e2_g"], bp["ln_e2_b"])
    np.testing.assert_allclose(out["E2"][pm], ref[pm], rtol=1e-12, atol=1e-12)
    # y decoupled from X and E: with W_yx = W_ye = 0, y2 does not move when X changes,
    # and with W_yy = 0 and b_yo = 0 as well, y1 = LN(y)
    q = dict(bp, w_yx=np.zeros_like(bp["w_yx"]), w_ye=np.zeros_like(bp["w_ye"]))
    a = OBK.block(batch, q, cfg.dims.H)
    b2 = dict(batch, X=(batch["X"] * 1.7 + 0.3).astype(np.float32))
    b = OBK.block(b2, q, cfg.dims.H)
    assert not np.allclose(a["X2"], b["X2"])
    np.testing.assert_allclose(a["y2"], b["y2"], rtol=1e-12, atol=1e-12)
    q.update(w_yy=np.zeros_like(bp["w_yy"]), b_yo=np.zeros_like(bp["b_yo"]))
    a = OBK.block(batch, q, cfg.dims.H)
    np.testing.assert_allclose(a["y1"], OBK.layer_norm(batch["y"], bp["ln_y1_g"], bp["ln_y1_b"]), rtol=1e-12, atol=1e-12)


def test_widths():
    for name in ("tiny", "planar"):
        dims = W.CONFIGS[name].dims
        bp = W.make_block_params(dims)
        assert bp["w_x1"].shape == (dims.d, dims.d)
        assert bp["w_e1"].shape == (2 * dims.de, dims.de) and bp["w_e2"].shape == (dims.de, 2 * dims.de)
        assert bp["w_y1"].shape == (dims.dy, dims.dy)


@pytest.mark.parametrize("bf16", [False, True])
def test_block_rows_match_the_whole_block(bf16):
    """The row-restricted block (node path of the row, edge path of the row's
    tokens) equals those rows of the whole block, masked rows included."""
    cfg = W.CONFIGS["tiny"]
    mask = np.ones((cfg.dims.B, cfg.dims.n), np.uint8)
    mask[1, 9:] = 0
    _, batch = _tiny(seed=17, mask=mask)
    if bf16:
        for k in list(batch):
            if k not in ("mask", "adj", "n_real"):
                batch[k] = W.bf16_round_array(batch[k])
    bp = _params(cfg)
    full = OBK.block(batch, bp, cfg.dims.H, bf16)
    rows = [(0, 0), (0, 7), (1, 3), (1, 10), (1, 11)]
    part = OBK.block_rows(batch, bp, cfg.dims.H, bf16, rows)
    rb = np.array([r[0] for r in part["rows"]])
    ri = np.array([r[1] for r in part["rows"]])
    np.testing.assert_allclose(part["X2"], full["X2"][rb, ri], rtol=0, atol=1e-12)
    np.testing.assert_allclose(part["E2"], full["E2"][rb, ri], rtol=0, atol=1e-12)
