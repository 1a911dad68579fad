"""ctypes binding of the CPU oracle (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` import this module. The product library never does.

The oracle computes the plain definition of the edge-aware attention layer
("Efficient Edge-aware Attention Network for Graph Generation", full-text
summary: scaled dot-product scores, head-wise FiLM from edge and global
features in score_mod, graph mask, normalized softmax, A*[V | I], residual
edge update) in double precision; see ``edge_attn_oracle.c`` for the readings.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "edge_attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_f32p = ctypes.POINTER(ctypes.c_float)
_f64p = ctypes.POINTER(ctypes.c_double)
_u8p = ctypes.POINTER(ctypes.c_uint8)
_i32p = ctypes.POINTER(ctypes.c_int32)


class _Dims(ctypes.Structure):
    _fields_ = [(k, ctypes.c_int32) for k in ("B", "n", "d", "de", "dy", "H", "dh", "bf16", "variant")]


# Ablation variants (bits of ``variant``; the C file states the readings).
LIGHT_EDGE, NO_SCORE_MOD, UNNORMALIZED = 1, 2, 4


_PARAM_NAMES = ("w_q", "w_k", "w_v", "b_q", "b_k", "b_v",
                "w_emul", "w_eadd", "b_emul", "b_eadd",
                "w_ymul", "w_yadd", "b_ymul", "b_yadd",
                "w_e", "b_e")


class _Params(ctypes.Structure):
    _fields_ = [(k, _f32p) for k in _PARAM_NAMES]


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (plain IEEE double arithmetic, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp",
                               "-shared", "-fPIC", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is None:
        lib = ctypes.CDLL(build())
        lib.eao_forward_rows.restype = ctypes.c_int
        lib.eao_forward_rows.argtypes = [ctypes.POINTER(_Dims), _f32p, _f32p, _f32p, _u8p,
                                         ctypes.POINTER(_Params), ctypes.c_int, _i32p, _i32p,
                                         _f64p, _f64p, _f64p, _f64p, _f64p]
        lib.eao_project.restype = None
        lib.eao_project.argtypes = [ctypes.POINTER(_Dims), _f32p, _u8p, _f32p, _f32p, _f64p]
        lib.eao_vi_product.restype = None
        lib.eao_vi_product.argtypes = [ctypes.POINTER(_Dims), _f64p, _f64p, _f64p]
        lib.eao_num_threads.restype = ctypes.c_int
        lib.eao_num_threads.argtypes = []
        lib.eao_set_num_threads.restype = ctypes.c_int
        lib.eao_set_num_threads.argtypes = [ctypes.c_int]
        lib.eao_bf16_round.restype = ctypes.c_double
        lib.eao_bf16_round.argtypes = [ctypes.c_double]
        _lib = lib
    return _lib


def _f32(a) -> np.ndarray:
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a: Optional[np.ndarray], typ):
    if a is None:
        return ctypes.cast(None, typ)
    return a.ctypes.data_as(typ)


def dims_of(batch: Dict[str, np.ndarray], H: int, bf16: bool) -> Tuple[int, ...]:
    B, n, d = batch["X"].shape
    de = batch["E"].shape[-1]
    dy = batch["y"].shape[-1]
    return B, n, d, de, dy, H, d // H, int(bool(bf16))


def forward(batch: Dict[str, np.ndarray], H: int, bf16: bool = False,
            rows: Optional[Sequence[Tuple[int, int]]] = None,
            zero_bias_names: Sequence[str] = (), variant: int = 0) -> Dict[str, np.ndarray]:
    """Run the layer definition.

    ``batch`` holds X, E, y, mask and the weights (as drawn by the workload
    generator). With ``rows=None`` every (b, i) row is computed and the result
    has full shapes: O [B,n,d], A [B,H,n,n], Ep [B,n,n,de], U [B,H,n,n],
    lse [B,H,n]. With a list of (b, i) rows the result is compact:
    O [R,d], A [R,H,n], Ep [R,n,de], U [R,H,n], lse [R,H]. ``variant`` is a
    combination of LIGHT_EDGE, NO_SCORE_MOD and UNNORMALIZED.
    """
    lib = _load()
    B, n, d, de, dy, Hh, dh, bf = dims_of(batch, H, bf16)
    dims = _Dims(B, n, d, de, dy, Hh, dh, bf, int(variant))
    X, E, y = _f32(batch["X"]), _f32(batch["E"]), _f32(batch["y"])
    mask = np.ascontiguousarray(batch["mask"], dtype=np.uint8)
    keep = {}
    for k in _PARAM_NAMES:
        v = batch.get(k)
        keep[k] = None if (v is None or k in zero_bias_names) else _f32(v)
    params = _Params(*[_ptr(keep[k], _f32p) for k in _PARAM_NAMES])

    full = rows is None
    if full:
        rows = [(b, i) for b in range(B) for i in range(n)]
    rows = sorted(rows, key=lambda r: r[0]) if not full else rows
    R = len(rows)
    rb = np.array([r[0] for r in rows], dtype=np.int32)
    ri = np.array([r[1] for r in rows], dtype=np.int32)
    O = np.zeros((R, d))
    A = np.zeros((R, Hh, n))
    Ep = np.zeros((R, n, de))
    U = np.zeros((R, Hh, n))
    L = np.zeros((R, Hh))
    rc = lib.eao_forward_rows(ctypes.byref(dims), _ptr(X, _f32p), _ptr(E, _f32p), _ptr(y, _f32p),
                              mask.ctypes.data_as(_u8p), ctypes.byref(params), R,
                              rb.ctypes.data_as(_i32p), ri.ctypes.data_as(_i32p),
                              _ptr(O, _f64p), _ptr(A, _f64p), _ptr(Ep, _f64p), _ptr(U, _f64p),
                              _ptr(L, _f64p))
    if rc != 0:
        raise ValueError("oracle rejected its arguments")
    out = {"rows": rows}
    if full:
        out["O"] = O.reshape(B, n, d)
        out["A"] = A.reshape(B, n, Hh, n).transpose(0, 2, 1, 3).copy()
        out["Ep"] = Ep.reshape(B, n, n, de)
        out["U"] = U.reshape(B, n, Hh, n).transpose(0, 2, 1, 3).copy()
        out["lse"] = L.reshape(B, n, Hh).transpose(0, 2, 1).copy()
    else:
        out.update(O=O, A=A, Ep=Ep, U=U, lse=L)
    return out


def project(batch: Dict[str, np.ndarray], which: str, H: int, bf16: bool = False) -> np.ndarray:
    """One node projection (which in q/k/v) for all graphs: [B,n,d] double."""
    lib = _load()
    B, n, d, de, dy, Hh, dh, bf = dims_of(batch, H, bf16)
    dims = _Dims(B, n, d, de, dy, Hh, dh, bf)
    X = _f32(batch["X"])
    mask = np.ascontiguousarray(batch["mask"], dtype=np.uint8)
    W = _f32(batch["w_" + which])
    bias = batch.get("b_" + which)
    bias = None if bias is None else _f32(bias)
    out = np.zeros((B, n, d))
    lib.eao_project(ctypes.byref(dims), _ptr(X, _f32p), mask.ctypes.data_as(_u8p),
                    _ptr(W, _f32p), _ptr(bias, _f32p), _ptr(out, _f64p))
    return out


def vi_product(A_row: np.ndarray, V: np.ndarray, dh: int) -> np.ndarray:
    """Literal A * [V | I] for one query row: A_row [H,n], V [n,d] -> [H, dh+n]."""
    lib = _load()
    Hh, n = A_row.shape
    d = V.shape[1]
    dims = _Dims(1, n, d, 1, 1, Hh, dh, 0)
    A_row = np.ascontiguousarray(A_row, dtype=np.float64)
    V = np.ascontiguousarray(V, dtype=np.float64)
    out = np.zeros((Hh, dh + n))
    lib.eao_vi_product(ctypes.byref(dims), _ptr(A_row, _f64p), _ptr(V, _f64p), _ptr(out, _f64p))
    return out


def bf16_round(x: float) -> float:
    """The oracle's own round-to-nearest-even bfloat16 routine."""
    return float(_load().eao_bf16_round(float(x)))


def num_threads() -> int:
    """Threads the oracle's row loop runs on."""
    return int(_load().eao_num_threads())


def set_num_threads(t: int) -> int:
    """Threads of the row loop from now on; returns the previous count."""
    return int(_load().eao_set_num_threads(int(t)))
