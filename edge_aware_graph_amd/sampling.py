"""Stacked-layer sampling loop (orchestration only; every layer runs in the
HIP kernels through the C ABI).

A synthetic stand-in for the shape of graph-generation sampling with the
edge-aware attention layer ("Efficient Edge-aware Attention Network for Graph
Generation", full-text summary: the layer is the backbone of a DeFoG-style
denoising model and the pages report sampling throughput): L layers with
their own random weights, applied in sequence at each of T denoising steps to
one batch. Two depths of layer:

- attention layers only: layer l + 1 takes layer l's node output O as its X
  and its edge output E' as its E; y and the node mask stay fixed;
- whole graph-transformer blocks (the attention layer, then the node, edge
  and global-feature paths with their norms and feed-forward parts):
  block l + 1 takes block l's X2, E2 and y2; the mask stays fixed.

The denoiser's sampling rule (the noise schedule and the update of the
graph between steps) is not on the pages and is not modelled: a step is the
L layers only.
"""
from __future__ import annotations

from typing import Dict, List, Optional

import torch

from .layer import EdgeAttention


class SamplingLoop:
    """L layers (or blocks) of one shape; buffers for two ping-pong (X, E, y) states.

    `block_params`: one dict of block parameters per layer (the names of
    `layer.BLOCK_PARAM_NAMES`); when given, every layer is a whole block.
    """

    def __init__(self, dims, weights: List[Dict[str, torch.Tensor]], device="cuda",
                 block_params: Optional[List[Dict[str, torch.Tensor]]] = None):
        if block_params is not None and len(block_params) != len(weights):
            raise ValueError("one set of block parameters per layer")
        self.dims = dims
        self.weights = weights
        self.block_params = block_params
        self.layer = EdgeAttention(dims.B, dims.n, dims.d, dims.de, dims.dy, dims.H, dims.dh, dims.dtype)
        dt = torch.bfloat16 if dims.dtype == "bf16" else torch.float32
        B, n, d, de, H = dims.B, dims.n, dims.d, dims.de, dims.H
        nbytes = self.layer.block_workspace_bytes if block_params is not None else self.layer.workspace_bytes
        self.ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
        self.X = [torch.empty(B, n, d, dtype=dt, device=device) for _ in range(2)]
        self.E = [torch.empty(B, n, n, de, dtype=dt, device=device) for _ in range(2)]
        self.y = [torch.empty(B, dims.dy, dtype=dt, device=device) for _ in range(2)]
        self.A = None if (self.layer.two_pass or block_params is not None) else \
            torch.empty(B, H, n, n, dtype=dt, device=device)

    @property
    def num_layers(self) -> int:
        return len(self.weights)

    @property
    def blocks(self) -> bool:
        return self.block_params is not None

    def run(self, X0: torch.Tensor, E0: torch.Tensor, y: torch.Tensor, mask: torch.Tensor, steps: int):
        """T denoising steps of L layers from (X0, E0, y); returns the final
        (X, E, y) buffers (y is the input's copy when only attention layers run)."""
        self.X[0].copy_(X0)
        self.E[0].copy_(E0)
        self.y[0].copy_(y)
        # every (layer, buffer parity) call is checked and marshalled once per
        # run, so the loop itself only launches
        calls = []
        for k, w in enumerate(self.weights):
            per = []
            for cur in (0, 1):
                nxt = 1 - cur
                if self.blocks:
                    per.append(self.layer.bind_block(w, self.block_params[k], self.X[cur], self.E[cur], self.y[cur],
                                                     mask, self.X[nxt], self.E[nxt], self.y[nxt], self.ws))
                else:
                    per.append(self.layer.bind_layer(w, self.X[cur], self.E[cur], self.y[0], mask, self.X[nxt],
                                                     self.A, self.E[nxt], self.ws))
            calls.append(per)
        cur = 0
        for _ in range(steps):
            for per in calls:
                per[cur]()
                cur = 1 - cur
        return self.X[cur], self.E[cur], (self.y[cur] if self.blocks else self.y[0])
