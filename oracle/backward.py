"""Backward oracle of the edge-aware attention layer (test infrastructure only).

Only the test suite imports this module; the product library never does.

The forward definition ("Efficient Edge-aware Attention Network for Graph
Generation", full-text summary: scaled dot-product scores, head-wise FiLM of
the score from the edge and the global feature, graph mask, normalized
softmax, A [V | I], residual edge update E' = E + W_e A + b_e) is restated
here with float64 torch tensor operations, and its gradients are taken by
torch autograd: the backward is exactly the derivative of the definition.
The restatement is pinned against the C oracle's forward, and the gradients
against central finite differences of the C oracle (tests/test_oracle_pins.py).

bf16 mode keeps the forward's rounding points (Q, K, V after the projection,
A after the softmax) with straight-through gradients (the rounding counts as
the identity in the backward), and takes the softmax Jacobian in terms of
its stored output, diag(A) - A A^T at the rounded A: what a backward built on
the stored bfloat16 forward values computes. (Taking it at the unrounded
softmax instead differs by about 2^-8 relative per term; on gradients that
nearly cancel, such as a key bias, that is a few percent of the result.)

Masking follows the forward: rows of padded nodes give zero projections, a
query row with no real key gives A = 0, masked pairs give E' = +0.0 (so their
E gets no gradient through the residual either).
"""
from __future__ import annotations

import math
from typing import Dict, Sequence

import numpy as np
import torch

WEIGHTS = ("w_q", "w_k", "w_v", "b_q", "b_k", "b_v", "w_emul", "w_eadd", "b_emul", "b_eadd",
           "w_ymul", "w_yadd", "b_ymul", "b_yadd", "w_e", "b_e")
INPUTS = ("X", "E", "y")


def _st_round(x: torch.Tensor, on: bool) -> torch.Tensor:
    """bfloat16 rounding (round to nearest even) with a straight-through gradient."""
    if not on:
        return x
    return x + (x.to(torch.bfloat16).to(torch.float64) - x).detach()


class _RoundedSoftmax(torch.autograd.Function):
    """bfloat16-rounded masked softmax whose backward uses the stored (rounded) output."""

    @staticmethod
    def forward(ctx, u, pmh):
        A = torch.where(pmh, torch.softmax(u, -1), torch.zeros((), dtype=torch.float64))
        A = A.to(torch.bfloat16).to(torch.float64)
        ctx.save_for_backward(A)
        return A

    @staticmethod
    def backward(ctx, g):
        (A,) = ctx.saved_tensors
        return A * (g - (A * g).sum(-1, keepdim=True)), None


def layer(t: Dict[str, torch.Tensor], mask: np.ndarray, H: int, bf16: bool, rows=None):
    """Forward of the layer on float64 tensors; returns O [B,n,d], A [B,H,n,n], E' [B,n,n,de].

    `rows` (a list of query indices): only those query rows, with t["E"]
    holding just their edge rows [B, R, n, de]; the outputs are then O
    [B,R,d], A [B,H,R,n], E' [B,R,n,de]. Query row i reads E only in row i,
    so these are exactly the full layer's rows.
    """
    X, E, y = t["X"], t["E"], t["y"]
    B, n, d = X.shape
    dh = d // H
    m = torch.tensor(mask.astype(bool))
    mq = m if rows is None else m[:, list(rows)]
    pm = mq[:, :, None] & m[:, None, :]
    R = mq.shape[1]

    def lin(x, w, b):
        out = x @ t[w].transpose(0, 1)
        return out + t[b] if t.get(b) is not None else out

    def proj(w, b):
        P = torch.where(m[..., None], lin(X, w, b), torch.zeros((), dtype=torch.float64))
        return _st_round(P, bf16).view(B, n, H, dh).transpose(1, 2)  # [B,H,n,dh]

    q, k, v = proj("w_q", "b_q"), proj("w_k", "b_k"), proj("w_v", "b_v")
    if rows is not None:
        q = q[:, :, list(rows)]
    gy = 1.0 + lin(y, "w_ymul", "b_ymul")  # [B,H]
    by = lin(y, "w_yadd", "b_yadd")
    ge = (1.0 + lin(E, "w_emul", "b_emul")).permute(0, 3, 1, 2)  # [B,H,n,n]
    be = lin(E, "w_eadd", "b_eadd").permute(0, 3, 1, 2)
    r = 1.0 / math.sqrt(dh)
    s = (q @ k.transpose(-1, -2)) * r
    u = (s * ge + be) * gy[:, :, None, None] + by[:, :, None, None]
    pmh = pm[:, None].expand(B, H, R, n)
    has = pmh.any(-1, keepdim=True)
    u = torch.where(pmh, u, torch.tensor(float("-inf"), dtype=torch.float64))
    u = torch.where(has, u, torch.zeros((), dtype=torch.float64))  # rows without a real key
    if bf16:
        A = _RoundedSoftmax.apply(u, pmh)
    else:
        A = torch.where(pmh, torch.softmax(u, -1), torch.zeros((), dtype=torch.float64))
    O = (A @ v).transpose(1, 2).reshape(B, R, d)
    O = torch.where(mq[..., None], O, torch.zeros((), dtype=torch.float64))
    Ep = E + lin(A.permute(0, 2, 3, 1), "w_e", "b_e")
    Ep = torch.where(pm[..., None], Ep, torch.zeros((), dtype=torch.float64))
    return O, A, Ep


def backward(batch: Dict[str, np.ndarray], dO: np.ndarray, dEp: np.ndarray, H: int,
             bf16: bool = False, wrt: Sequence[str] = INPUTS + WEIGHTS) -> Dict[str, np.ndarray]:
    """Gradients of sum(O * dO) + sum(E' * dEp) with respect to `wrt` (float64).

    Absent biases count as zero and get no gradient entry.
    """
    t = {}
    for k in INPUTS + WEIGHTS:
        v = batch.get(k)
        if v is None:
            t[k] = None
            continue
        t[k] = torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=k in wrt)
    O, _, Ep = layer(t, batch["mask"], H, bf16)
    loss = (O * torch.tensor(dO, dtype=torch.float64)).sum() + (Ep * torch.tensor(dEp, dtype=torch.float64)).sum()
    keys = [k for k in wrt if t.get(k) is not None]
    grads = torch.autograd.grad(loss, [t[k] for k in keys], allow_unused=True)
    out = {}
    for k, g in zip(keys, grads):
        out[k] = np.zeros(t[k].shape) if g is None else g.detach().numpy()
    return out


def edge_grad_rows(batch: Dict[str, np.ndarray], dO: np.ndarray, dEp: np.ndarray, H: int, bf16: bool,
                   b: int, rows: Sequence[int]) -> np.ndarray:
    """dL/dE[b, rows, :, :] for L = sum(O * dO) + sum(E' * dEp), from the
    layer restricted to graph b and those query rows: E[b, i] reaches L only
    through row i's scores, softmax, O_i and E'_i, so the restricted
    derivative is the full one. For checks at sizes the full backward cannot
    handle; returns [len(rows), n, de]."""
    rows = list(rows)
    t = {}
    for k in INPUTS + WEIGHTS:
        v = batch.get(k)
        if v is None:
            t[k] = None
            continue
        if k == "E":
            v = np.asarray(v)[b:b + 1][:, rows]
        elif k in ("X", "y"):
            v = np.asarray(v)[b:b + 1]
        t[k] = torch.tensor(np.asarray(v, dtype=np.float64), requires_grad=k == "E")
    O, _, Ep = layer(t, batch["mask"][b:b + 1], H, bf16, rows=rows)
    loss = (O * torch.tensor(np.asarray(dO)[b:b + 1][:, rows].astype(np.float64))).sum() + \
        (Ep * torch.tensor(np.asarray(dEp)[b:b + 1][:, rows].astype(np.float64))).sum()
    (g,) = torch.autograd.grad(loss, [t["E"]])
    return g.detach().numpy()[0]


def forward(batch: Dict[str, np.ndarray], H: int, bf16: bool = False) -> Dict[str, np.ndarray]:
    """The restated forward (for its pin against the C oracle)."""
    t = {k: (None if batch.get(k) is None else torch.tensor(np.asarray(batch[k], dtype=np.float64)))
         for k in INPUTS + WEIGHTS}
    O, A, Ep = layer(t, batch["mask"], H, bf16)
    return {"O": O.numpy(), "A": A.numpy(), "Ep": Ep.numpy()}
