"""Seeded synthetic inputs for the edge-aware attention layer.

This module only draws inputs: graph structure, node/edge/global features,
masks and weights. It holds none of the layer's arithmetic, so the GPU path
and the CPU oracle can both consume the same batch without sharing any code
that computes the method.

Workloads stand in for the Planar, Tree and SBM graph-generation benchmarks
the method is evaluated on ("Efficient Edge-aware Attention Network for Graph
Generation", spec card: Planar/Tree/SBM datasets), plus a tiny check and a
large-graph stress case. No dataset item is reproduced: every graph is drawn
from a seeded random model with the shape of its stand-in.

Draw order (fixed, one ``numpy.random.default_rng(seed)`` per batch):
structure -> edge embedding table -> edge noise -> X -> y ->
W_q, W_k, W_v, W_emul, W_eadd, W_ymul, W_yadd, W_e -> biases (only when
``bias_scale`` is non-zero).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

__all__ = [
    "LayerDims", "CONFIGS", "make_batch", "bf16_round_array",
    "er_adjacency", "delaunay_adjacency", "prufer_tree_adjacency",
    "sbm_adjacency", "rgg_adjacency", "rgg_radius",
]


@dataclasses.dataclass(frozen=True)
class LayerDims:
    """Shape of one layer call: B graphs padded to n nodes."""
    B: int
    n: int
    d: int
    de: int
    dy: int
    H: int
    dh: int
    dtype: str  # "fp32" or "bf16"

    @property
    def edge_tokens(self) -> int:
        return self.B * self.n * self.n


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    dims: LayerDims
    structure: str
    seed: int
    description: str


CONFIGS: Dict[str, Config] = {
    "tiny": Config(
        "tiny", LayerDims(B=2, n=12, d=64, de=16, dy=16, H=4, dh=16, dtype="fp32"),
        "er", 0,
        "B=2, n=12 (graph 1 has 9 real nodes), Erdos-Renyi p=0.3, fp32"),
    "planar": Config(
        "planar", LayerDims(B=64, n=64, d=256, de=64, dy=64, H=8, dh=32, dtype="bf16"),
        "delaunay", 1,
        "B=64, n=64, Delaunay triangulation of 64 uniform points, bf16"),
    "tree": Config(
        "tree", LayerDims(B=64, n=64, d=256, de=64, dy=64, H=8, dh=32, dtype="bf16"),
        "prufer", 2,
        "B=64, n=64, uniform labelled trees from Pruefer sequences, bf16"),
    "sbm": Config(
        "sbm", LayerDims(B=32, n=192, d=256, de=64, dy=64, H=8, dh=32, dtype="bf16"),
        "sbm", 3,
        "B=32, n_b ~ U{44..187} padded to 192, 2-5 communities, p_in=0.3, p_out=0.005, bf16"),
    "large": Config(
        "large", LayerDims(B=4, n=1024, d=256, de=64, dy=64, H=8, dh=32, dtype="bf16"),
        "rgg", 4,
        "B=4, n=1024, random geometric graphs with mean degree ~8, bf16, two-pass"),
}


# ---------------------------------------------------------------- structure

def er_adjacency(rng: np.random.Generator, nb: int, p: float) -> np.ndarray:
    """Symmetric Erdos-Renyi G(nb, p) adjacency, no self-loops."""
    upper = rng.random((nb, nb)) < p
    adj = np.triu(upper, k=1)
    return (adj | adj.T).astype(np.uint8)


def delaunay_adjacency(rng: np.random.Generator, nb: int) -> np.ndarray:
    """Edges of the Delaunay triangulation of nb uniform points in [0,1]^2."""
    from scipy.spatial import Delaunay
    pts = rng.random((nb, 2))
    tri = Delaunay(pts)
    adj = np.zeros((nb, nb), dtype=np.uint8)
    for simplex in tri.simplices:
        for a in range(3):
            for b in range(a + 1, 3):
                u, v = int(simplex[a]), int(simplex[b])
                adj[u, v] = adj[v, u] = 1
    return adj


def prufer_tree_adjacency(rng: np.random.Generator, nb: int) -> np.ndarray:
    """Uniform labelled tree on nb nodes from a uniform Pruefer sequence.

    Decoding is the textbook leaf-removal procedure: repeatedly join the
    smallest current leaf to the next sequence entry.
    """
    adj = np.zeros((nb, nb), dtype=np.uint8)
    if nb < 2:
        return adj
    seq = rng.integers(0, nb, size=nb - 2)
    degree = np.ones(nb, dtype=np.int64)
    for a in seq:
        degree[a] += 1
    for a in seq:
        leaf = int(np.flatnonzero(degree == 1)[0])
        adj[leaf, a] = adj[a, leaf] = 1
        degree[leaf] -= 1
        degree[a] -= 1
    u, v = np.flatnonzero(degree == 1)
    adj[u, v] = adj[v, u] = 1
    return adj


def sbm_adjacency(rng: np.random.Generator, nb: int, k: int,
                  p_in: float, p_out: float) -> np.ndarray:
    """Stochastic block model with k communities (i.i.d. uniform labels)."""
    labels = rng.integers(0, k, size=nb)
    same = labels[:, None] == labels[None, :]
    prob = np.where(same, p_in, p_out)
    upper = np.triu(rng.random((nb, nb)) < prob, k=1)
    return (upper | upper.T).astype(np.uint8)


def rgg_radius(n: int, mean_degree: float) -> float:
    """Radius r with expected degree (n-1) * P(|U-V| < r) = mean_degree.

    P(|U-V| < r) for two uniform points of the unit square is
    pi r^2 - 8 r^3 / 3 + r^4 / 2 (valid for r <= 1).
    """
    from scipy.optimize import brentq
    f = lambda r: (n - 1) * (math.pi * r * r - 8.0 * r ** 3 / 3.0 + r ** 4 / 2.0) - mean_degree
    return float(brentq(f, 1e-9, 1.0))


def rgg_adjacency(rng: np.random.Generator, nb: int, radius: float) -> np.ndarray:
    """Random geometric graph: nb uniform points, edge when distance < radius."""
    pts = rng.random((nb, 2))
    diff = pts[:, None, :] - pts[None, :, :]
    dist2 = np.einsum("ijk,ijk->ij", diff, diff)
    adj = dist2 < radius * radius
    np.fill_diagonal(adj, False)
    return adj.astype(np.uint8)


# ---------------------------------------------------------------- values

def bf16_round_array(a: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even), as float32.

    Input preparation only: the layer's own rounding points are implemented
    separately on each side.
    """
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def _xavier(rng: np.random.Generator, out_f: int, in_f: int) -> np.ndarray:
    bound = math.sqrt(6.0 / (in_f + out_f))
    return rng.uniform(-bound, bound, size=(out_f, in_f)).astype(np.float32)


def _structure(rng: np.random.Generator, cfg: Config):
    """Per-graph real-node counts and adjacency blocks (prefix of real nodes)."""
    dims = cfg.dims
    counts, adjs = [], []
    for b in range(dims.B):
        if cfg.structure == "er":
            nb = dims.n if b == 0 else 9
            adj = er_adjacency(rng, nb, 0.3)
        elif cfg.structure == "delaunay":
            nb = dims.n
            adj = delaunay_adjacency(rng, nb)
        elif cfg.structure == "prufer":
            nb = dims.n
            adj = prufer_tree_adjacency(rng, nb)
        elif cfg.structure == "sbm":
            nb = int(rng.integers(44, 188))
            k = int(rng.integers(2, 6))
            adj = sbm_adjacency(rng, nb, k, 0.3, 0.005)
        elif cfg.structure == "rgg":
            nb = dims.n
            adj = rgg_adjacency(rng, nb, rgg_radius(nb, 8.0))
        else:
            raise ValueError(cfg.structure)
        counts.append(nb)
        adjs.append(adj)
    return counts, adjs


def make_batch(name_or_cfg, seed: Optional[int] = None, bias_scale: float = 0.0,
               dims: Optional[LayerDims] = None) -> Dict[str, np.ndarray]:
    """Draw one synthetic batch.

    Returns float32 arrays (bf16-representable when the config is bf16):
      X [B,n,d], E [B,n,n,de], y [B,dy], mask [B,n] (uint8 0/1, prefix of
      real nodes), adj [B,n,n] (uint8), n_real [B], and weights in the
      nn.Linear [out, in] layout: w_q/w_k/w_v [d,d], w_emul/w_eadd [H,de],
      w_ymul/w_yadd [H,dy], w_e [de,H], plus biases b_* (zero unless
      ``bias_scale`` > 0, then N(0, bias_scale^2)).

    ``dims`` overrides the config's shape while keeping its structure model
    (used by parity tests at reduced sizes).
    """
    cfg = CONFIGS[name_or_cfg] if isinstance(name_or_cfg, str) else name_or_cfg
    if dims is not None:
        cfg = dataclasses.replace(cfg, dims=dims)
    dims = cfg.dims
    rng = np.random.default_rng(cfg.seed if seed is None else seed)
    B, n, d, de, dy, H = dims.B, dims.n, dims.d, dims.de, dims.dy, dims.H

    counts, adjs = _structure(rng, cfg)
    counts = [min(c, n) for c in counts]
    adj = np.zeros((B, n, n), dtype=np.uint8)
    mask = np.zeros((B, n), dtype=np.uint8)
    for b, (nb, a) in enumerate(zip(counts, adjs)):
        adj[b, :nb, :nb] = a[:nb, :nb]
        mask[b, :nb] = 1

    emb = rng.standard_normal((2, de)).astype(np.float32)
    E = emb[adj.astype(np.int64)]
    E += 0.1 * rng.standard_normal(E.shape, dtype=np.float32)
    pair = (mask[:, :, None] & mask[:, None, :]).astype(bool)
    E[~pair] = 0.0

    X = rng.standard_normal((B, n, d), dtype=np.float32)
    X[mask == 0] = 0.0
    y = rng.standard_normal((B, dy), dtype=np.float32)

    w = {
        "w_q": _xavier(rng, d, d), "w_k": _xavier(rng, d, d), "w_v": _xavier(rng, d, d),
        "w_emul": _xavier(rng, H, de), "w_eadd": _xavier(rng, H, de),
        "w_ymul": _xavier(rng, H, dy), "w_yadd": _xavier(rng, H, dy),
        "w_e": _xavier(rng, de, H),
    }
    bias_shapes = {"b_q": d, "b_k": d, "b_v": d, "b_emul": H, "b_eadd": H,
                   "b_ymul": H, "b_yadd": H, "b_e": de}
    for k, m in bias_shapes.items():
        if bias_scale > 0:
            w[k] = (bias_scale * rng.standard_normal(m)).astype(np.float32)
        else:
            w[k] = np.zeros(m, dtype=np.float32)

    out = {"X": X, "E": E, "y": y, **w}
    if dims.dtype == "bf16":
        out = {k: bf16_round_array(v) for k, v in out.items()}
    out["mask"] = mask
    out["adj"] = adj
    out["n_real"] = np.array(counts, dtype=np.int64)
    return out


# Parameters of the graph-transformer block around the layer (node path,
# edge path, global-feature path), nn.Linear [out, in] layout. Widths of the
# feed-forward layers: d for the nodes, 2 de for the edges, dy for y.
BLOCK_WEIGHTS = ("w_o", "w_x1", "w_x2", "w_e1", "w_e2", "w_yy", "w_yx", "w_ye", "w_y1", "w_y2")
BLOCK_VECTORS = ("b_o", "b_x1", "b_x2", "b_e1", "b_e2", "b_yo", "b_y1", "b_y2")
BLOCK_NORMS = ("x1", "x2", "e1", "e2", "y1", "y2")


def block_widths(dims: LayerDims):
    """Feed-forward widths (nodes, edges, y) of the block for a layer shape."""
    return dims.d, 2 * dims.de, dims.dy


def make_block_params(dims: LayerDims, seed: int = 7, scale: float = 0.1) -> Dict[str, np.ndarray]:
    """Seeded block parameters: Xavier-uniform weights, N(0, scale^2) biases,
    LayerNorm gains 1 + N(0, scale^2) and shifts N(0, scale^2) (scale = 0:
    zero biases, unit gains, zero shifts). bfloat16-representable when the
    shape's dtype is bf16."""
    rng = np.random.default_rng(seed)
    d, de, dy = dims.d, dims.de, dims.dy
    fx, fe, fy = block_widths(dims)
    shapes = {"w_o": (d, d), "w_x1": (fx, d), "w_x2": (d, fx), "w_e1": (fe, de), "w_e2": (de, fe),
              "w_yy": (dy, dy), "w_yx": (dy, d), "w_ye": (dy, de), "w_y1": (fy, dy), "w_y2": (dy, fy)}
    vec = {"b_o": d, "b_x1": fx, "b_x2": d, "b_e1": fe, "b_e2": de, "b_yo": dy, "b_y1": fy, "b_y2": dy}
    norm = {"x1": d, "x2": d, "e1": de, "e2": de, "y1": dy, "y2": dy}
    p = {k: _xavier(rng, *s) for k, s in shapes.items()}
    for k, m in vec.items():
        p[k] = (scale * rng.standard_normal(m)).astype(np.float32)
    for k, m in norm.items():
        p["ln_%s_g" % k] = (1.0 + scale * rng.standard_normal(m)).astype(np.float32)
        p["ln_%s_b" % k] = (scale * rng.standard_normal(m)).astype(np.float32)
    if dims.dtype == "bf16":
        p = {k: bf16_round_array(v) for k, v in p.items()}
    return p
