"""Stacked-layer sampling loop (orchestration only; every layer runs in the
HIP kernels through the C ABI).

A synthetic stand-in for the shape of graph-generation sampling with the
edge-aware attention layer ("Efficient Edge-aware Attention Network for Graph
Generation", full-text summary: the layer is the backbone of a DeFoG-style
denoising model and the pages report sampling throughput): L layers with
their own random weights, applied in sequence at each of T denoising steps to
one batch. Layer l + 1 takes layer l's node output O as its X and its edge
output E' as its E; y and the node mask stay fixed. The rest of the graph
transformer block (projections, norms, feed-forward parts) and the denoiser's
sampling rule are not on the pages and are not modelled: a step here is the
layers only.
"""
from __future__ import annotations

from typing import Dict, List

import torch

from .layer import EdgeAttention


class SamplingLoop:
    """L layers of one shape; buffers for two ping-pong (X, E) states."""

    def __init__(self, dims, weights: List[Dict[str, torch.Tensor]], device="cuda"):
        self.dims = dims
        self.weights = weights
        self.layer = EdgeAttention(dims.B, dims.n, dims.d, dims.de, dims.dy, dims.H, dims.dh, dims.dtype)
        dt = torch.bfloat16 if dims.dtype == "bf16" else torch.float32
        B, n, d, de, H = dims.B, dims.n, dims.d, dims.de, dims.H
        self.ws = torch.empty(self.layer.workspace_bytes, dtype=torch.uint8, device=device)
        self.X = [torch.empty(B, n, d, dtype=dt, device=device) for _ in range(2)]
        self.E = [torch.empty(B, n, n, de, dtype=dt, device=device) for _ in range(2)]
        self.A = None if self.layer.two_pass else torch.empty(B, H, n, n, dtype=dt, device=device)

    @property
    def num_layers(self) -> int:
        return len(self.weights)

    def run(self, X0: torch.Tensor, E0: torch.Tensor, y: torch.Tensor, mask: torch.Tensor, steps: int):
        """T denoising steps of L layers from (X0, E0); returns the final (X, E) buffers."""
        self.X[0].copy_(X0)
        self.E[0].copy_(E0)
        cur = 0
        for _ in range(steps):
            for w in self.weights:
                nxt = 1 - cur
                self.layer.layer(w, self.X[cur], self.E[cur], y, mask, self.X[nxt], self.A, self.E[nxt], self.ws)
                cur = nxt
        return self.X[cur], self.E[cur]
