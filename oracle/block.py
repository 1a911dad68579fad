"""Oracle of the graph-transformer block around the edge-aware attention layer
(test infrastructure only: the test suite, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may use it; the product library never
does).

The method's page ("Efficient Edge-aware Attention Network for Graph
Generation", full-text summary) replaces the attention inside a graph
transformer and keeps the rest of the block; the block itself is not written
out there. The reading taken here is the usual graph-transformer layer of
the denoising graph generators it builds on (node, edge and global-feature
streams, each with residual connections, layer normalization and a
two-layer ReLU feed-forward network):

  (O, A, E') = edge-aware attention layer (X, E, y, mask)     [the C oracle]
  X1 = LN(X + O W_o^T + b_o)
  X2 = LN(X1 + W_x2 relu(W_x1 X1 + b_x1) + b_x2)               rows of real nodes; else 0
  E1 = LN(E')                                                   (E' already holds E + W_e A + b_e)
  E2 = LN(E1 + W_e2 relu(W_e1 E1 + b_e1) + b_e2)               real pairs; else 0
  xbar = mean of X2 over real nodes, ebar = mean of E2 over real pairs (0 if none)
  y1 = LN(y + W_yy y + W_yx xbar + W_ye ebar + b_yo)
  y2 = LN(y1 + W_y2 relu(W_y1 y1 + b_y1) + b_y2)

LN is layer normalization over the feature axis with the population
variance, eps = 1e-5, and a per-feature gain and shift. Widths: W_x1 is
[d, d], W_e1 is [2 de, de], W_y1 is [dy, dy].

Precision: float64. bfloat16 mode applies the rounding points of the GPU
path: O and E' are stored in bfloat16 by the layer; X1, the node hidden
layer, E1 and the edge hidden layer are rounded to bfloat16 where they enter
a matrix product (the residual adds use the unrounded values); the
global-feature path takes its float32 sums as they are. Outputs are not
rounded.
"""
from __future__ import annotations

from typing import Dict

import numpy as np

from . import oracle as _layer

EPS = 1e-5


def bf16(x: np.ndarray) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even), elementwise, in float64."""
    a = np.ascontiguousarray(x, dtype=np.float32)
    u = a.view(np.uint32).astype(np.uint64)
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16
    return r.astype(np.uint32).view(np.float32).astype(np.float64)


def layer_norm(z: np.ndarray, g: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Normalization over the last axis: (z - mean) / sqrt(var + eps) * g + b."""
    z = np.asarray(z, dtype=np.float64)
    mu = z.sum(-1, keepdims=True) / z.shape[-1]
    c = z - mu
    var = (c * c).sum(-1, keepdims=True) / z.shape[-1]
    return c / np.sqrt(var + EPS) * np.asarray(g, np.float64) + np.asarray(b, np.float64)


def linear(x: np.ndarray, w: np.ndarray, b=None) -> np.ndarray:
    """x W^T (+ b) with W in the [out, in] layout."""
    out = np.asarray(x, np.float64) @ np.asarray(w, np.float64).T
    return out if b is None else out + np.asarray(b, np.float64)


def relu(x: np.ndarray) -> np.ndarray:
    return np.where(x > 0, x, 0.0)


def _rounder(bf16_mode: bool):
    return bf16 if bf16_mode else (lambda v: np.asarray(v, np.float64))


def node_path(X: np.ndarray, O: np.ndarray, bp: Dict[str, np.ndarray], bf16_mode: bool):
    """X1 and X2 (before masking) of node rows, any leading shape; O as stored."""
    r = _rounder(bf16_mode)
    ln = lambda z, k: layer_norm(z, bp["ln_%s_g" % k], bp["ln_%s_b" % k])
    X1 = ln(np.asarray(X, np.float64) + linear(O, bp["w_o"], bp["b_o"]), "x1")
    Hx = relu(linear(r(X1), bp["w_x1"], bp["b_x1"]))
    X2 = ln(X1 + linear(r(Hx), bp["w_x2"], bp["b_x2"]), "x2")
    return X1, Hx, X2


def edge_path(Ep: np.ndarray, bp: Dict[str, np.ndarray], bf16_mode: bool):
    """E1 and E2 (before masking) of edge tokens, any leading shape; E' as stored."""
    r = _rounder(bf16_mode)
    ln = lambda z, k: layer_norm(z, bp["ln_%s_g" % k], bp["ln_%s_b" % k])
    E1 = ln(Ep, "e1")
    He = relu(linear(r(E1), bp["w_e1"], bp["b_e1"]))
    E2 = ln(E1 + linear(r(He), bp["w_e2"], bp["b_e2"]), "e2")
    return E1, He, E2


def block(batch: Dict[str, np.ndarray], bp: Dict[str, np.ndarray], H: int, bf16_mode: bool = False,
          layer_out: Dict[str, np.ndarray] = None) -> Dict[str, np.ndarray]:
    """The block on a batch; returns X2 [B,n,d], E2 [B,n,n,de], y2 [B,dy] and
    the intermediates (O, Ep, X1, Hx, E1, He, xbar, ebar, y1)."""
    f = layer_out if layer_out is not None else _layer.forward(batch, H, bf16_mode)
    r = _rounder(bf16_mode)
    O, Ep = r(f["O"]), r(f["Ep"])
    m = batch["mask"].astype(bool)
    pm = m[:, :, None] & m[:, None, :]
    y = np.asarray(batch["y"], np.float64)
    ln = lambda z, k: layer_norm(z, bp["ln_%s_g" % k], bp["ln_%s_b" % k])

    X1, Hx, X2 = node_path(batch["X"], O, bp, bf16_mode)
    X2 = np.where(m[..., None], X2, 0.0)

    E1, He, E2 = edge_path(Ep, bp, bf16_mode)
    E2 = np.where(pm[..., None], E2, 0.0)

    nr = m.sum(1).astype(np.float64)
    xbar = X2.sum(1) / np.maximum(nr, 1.0)[:, None]
    ebar = E2.sum((1, 2)) / np.maximum(nr * nr, 1.0)[:, None]
    y1 = ln(y + linear(y, bp["w_yy"]) + linear(xbar, bp["w_yx"]) + linear(ebar, bp["w_ye"], bp["b_yo"]), "y1")
    Hy = relu(linear(y1, bp["w_y1"], bp["b_y1"]))
    y2 = ln(y1 + linear(Hy, bp["w_y2"], bp["b_y2"]), "y2")
    return {"X2": X2, "E2": E2, "y2": y2, "O": O, "Ep": Ep, "X1": X1, "Hx": Hx, "E1": E1, "He": He,
            "xbar": xbar, "ebar": ebar, "y1": y1}


def block_rows(batch: Dict[str, np.ndarray], bp: Dict[str, np.ndarray], H: int, bf16_mode: bool,
               rows) -> Dict[str, np.ndarray]:
    """X2 [R,d] and E2 [R,n,de] of the given (b, i) rows: node row i depends
    on its own O row and X row, edge token (i, j) on E'_ij alone, so only the
    layer's rows are needed (for checks at sizes the whole block cannot be
    computed); y2 needs every row and is not returned."""
    f = _layer.forward(batch, H, bf16_mode, rows=rows)
    r = _rounder(bf16_mode)
    rb = np.array([q[0] for q in f["rows"]])
    ri = np.array([q[1] for q in f["rows"]])
    m = batch["mask"].astype(bool)
    mi = m[rb, ri]
    pm = mi[:, None] & m[rb]
    _, _, X2 = node_path(np.asarray(batch["X"])[rb, ri], r(f["O"]), bp, bf16_mode)
    _, _, E2 = edge_path(r(f["Ep"]), bp, bf16_mode)
    return {"rows": f["rows"], "X2": np.where(mi[:, None], X2, 0.0), "E2": np.where(pm[..., None], E2, 0.0)}

