"""Python binding of the C-ABI library (argument marshalling only).

Every step of the layer runs in the HIP kernels of ``libedge_attn.so``; this
module only turns torch tensors into device pointers and the current torch
stream into a ``hipStream_t``. There is no fallback: if the library is not
built, importing it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Dict, Optional

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libedge_attn.so")

EA_OK, EA_E_NULLPTR, EA_E_SHAPE, EA_E_UNSUPPORTED, EA_E_ALIGN, EA_E_WORKSPACE, EA_E_STATE, EA_E_HIP = range(8)
EA_FP32, EA_BF16 = 0, 1
EA_FORCE_TWO_PASS = 0x1
# Ablation variants (desc.flags): no per-edge FiLM; no FiLM at all; the edge
# update takes the masked logits instead of A.
EA_VARIANT_LIGHT_EDGE = 0x2
EA_VARIANT_NO_SCORE_MOD = 0x4
EA_VARIANT_UNNORMALIZED = 0x8
VARIANTS = {"light_edge": EA_VARIANT_LIGHT_EDGE, "no_score_mod": EA_VARIANT_NO_SCORE_MOD,
            "unnormalized": EA_VARIANT_UNNORMALIZED}
EA_SINGLE_PASS_MAX_N = 256
KERNELS = ("qkv_kernel", "attn_kernel", "update_kernel", "attn_kernel(fused)", "backward (all kernels)",
           "block (node, edge, y kernels)")

# Symbols declared in include/edge_attn.h.
EXPORTS = ("ea_ctx_create", "ea_ctx_destroy", "ea_workspace_bytes", "ea_is_two_pass",
           "edge_attn_forward", "edge_update", "edge_attn_layer", "ea_status_str",
           "ea_last_error", "ea_debug_logits", "ea_profile_begin", "ea_profile_end",
           "ea_backward_workspace_bytes", "edge_attn_backward",
           "ea_block_workspace_bytes", "edge_attn_block",
           "ea_kernel_name")

# Parameters of the graph-transformer block, in the order of ea_block_params.
BLOCK_PARAM_NAMES = ("w_o", "b_o", "ln_x1_g", "ln_x1_b", "w_x1", "b_x1", "w_x2", "b_x2", "ln_x2_g", "ln_x2_b",
                     "ln_e1_g", "ln_e1_b", "w_e1", "b_e1", "w_e2", "b_e2", "ln_e2_g", "ln_e2_b",
                     "w_yy", "w_yx", "w_ye", "b_yo", "ln_y1_g", "ln_y1_b", "w_y1", "b_y1", "w_y2", "b_y2",
                     "ln_y2_g", "ln_y2_b")


class EaError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__("%s (status %d)" % (msg, status))
        self.status = status


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("n", ctypes.c_int32), ("d", ctypes.c_int32),
                ("de", ctypes.c_int32), ("dy", ctypes.c_int32), ("H", ctypes.c_int32),
                ("dh", ctypes.c_int32), ("dtype", ctypes.c_int32), ("flags", ctypes.c_uint32)]


ATTN_PARAM_NAMES = ("w_q", "w_k", "w_v", "b_q", "b_k", "b_v", "w_emul", "w_eadd", "b_emul",
                    "b_eadd", "w_ymul", "w_yadd", "b_ymul", "b_yadd")
UPDATE_PARAM_NAMES = ("w_e", "b_e")


class AttnParams(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in ATTN_PARAM_NAMES]


class UpdateParams(ctypes.Structure):
    _fields_ = [(k, ctypes.c_void_p) for k in UPDATE_PARAM_NAMES]


GRAD_NAMES = ATTN_PARAM_NAMES + UPDATE_PARAM_NAMES


class BlockParams(ctypes.Structure):
    """ea_block_params: device pointers to the block's parameters."""
    _fields_ = [(k, ctypes.c_void_p) for k in BLOCK_PARAM_NAMES]


class Grads(ctypes.Structure):
    """ea_grads: float32 weight-gradient buffers."""
    _fields_ = [(k, ctypes.c_void_p) for k in ("w_q", "w_k", "w_v", "b_q", "b_k", "b_v", "w_emul", "w_eadd",
                                               "b_emul", "b_eadd", "w_ymul", "w_yadd", "b_ymul", "b_yadd",
                                               "w_e", "b_e")]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError("HIP library %s is missing: run __graft_entry__.build() first" % path)
    lib = ctypes.CDLL(path)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    lib.ea_ctx_create.restype = ctypes.c_int
    lib.ea_ctx_create.argtypes = [ctypes.POINTER(Desc), ctypes.POINTER(vp)]
    lib.ea_ctx_destroy.restype = None
    lib.ea_ctx_destroy.argtypes = [vp]
    lib.ea_workspace_bytes.restype = sz
    lib.ea_workspace_bytes.argtypes = [vp]
    lib.ea_is_two_pass.restype = ctypes.c_int
    lib.ea_is_two_pass.argtypes = [vp]
    ap, up = ctypes.POINTER(AttnParams), ctypes.POINTER(UpdateParams)
    lib.edge_attn_forward.restype = ctypes.c_int
    lib.edge_attn_forward.argtypes = [vp, ap, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.edge_update.restype = ctypes.c_int
    lib.edge_update.argtypes = [vp, ap, up, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.edge_attn_layer.restype = ctypes.c_int
    lib.edge_attn_layer.argtypes = [vp, ap, up, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ea_debug_logits.restype = ctypes.c_int
    lib.ea_debug_logits.argtypes = [vp, ap, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.ea_status_str.restype = ctypes.c_char_p
    lib.ea_status_str.argtypes = [ctypes.c_int]
    lib.ea_last_error.restype = ctypes.c_char_p
    lib.ea_last_error.argtypes = []
    lib.ea_profile_begin.restype = ctypes.c_int
    lib.ea_profile_begin.argtypes = [vp]
    lib.ea_profile_end.restype = ctypes.c_int
    lib.ea_profile_end.argtypes = [vp, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.ea_kernel_name.restype = ctypes.c_char_p
    lib.ea_kernel_name.argtypes = [ctypes.c_int]
    lib.ea_backward_workspace_bytes.restype = sz
    lib.ea_backward_workspace_bytes.argtypes = [vp]
    lib.edge_attn_backward.restype = ctypes.c_int
    lib.edge_attn_backward.argtypes = [vp, ap, up, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       ctypes.POINTER(Grads), vp, sz, vp, sz, vp]
    lib.ea_block_workspace_bytes.restype = sz
    lib.ea_block_workspace_bytes.argtypes = [vp]
    lib.edge_attn_block.restype = ctypes.c_int
    lib.edge_attn_block.argtypes = [vp, ap, up, ctypes.POINTER(BlockParams), vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    _lib = lib
    return lib


def _check(lib, status: int):
    if status != EA_OK:
        raise EaError(status, "%s: %s" % (lib.ea_status_str(status).decode(), lib.ea_last_error().decode()))


def _ptr(t) -> Optional[int]:
    """Device pointer of a tensor (None -> NULL). Plain ints pass through."""
    if t is None:
        return None
    if isinstance(t, int):
        return t
    if not t.is_contiguous():
        raise ValueError("tensors passed to the layer must be contiguous")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


class EdgeAttention:
    """A layer context: shape, dtype, mode and workspace plan (host only)."""

    def __init__(self, B: int, n: int, d: int, de: int, dy: int, H: int, dh: int,
                 dtype: str = "bf16", force_two_pass: bool = False, variant: int = 0):
        self.lib = load_library()
        self.desc = Desc(B, n, d, de, dy, H, dh, EA_BF16 if dtype == "bf16" else EA_FP32,
                         (EA_FORCE_TWO_PASS if force_two_pass else 0) | int(variant))
        ctx = ctypes.c_void_p()
        _check(self.lib, self.lib.ea_ctx_create(ctypes.byref(self.desc), ctypes.byref(ctx)))
        self.ctx = ctx
        self.dtype = dtype

    def __del__(self):
        ctx = getattr(self, "ctx", None)
        if ctx is not None and ctx.value:
            self.lib.ea_ctx_destroy(ctx)
            self.ctx = None

    @property
    def workspace_bytes(self) -> int:
        return int(self.lib.ea_workspace_bytes(self.ctx))

    @property
    def two_pass(self) -> bool:
        return bool(self.lib.ea_is_two_pass(self.ctx))

    @staticmethod
    def attn_params(w: Dict) -> AttnParams:
        return AttnParams(*[_ptr(w.get(k)) for k in ATTN_PARAM_NAMES])

    @staticmethod
    def update_params(w: Dict) -> UpdateParams:
        return UpdateParams(*[_ptr(w.get(k)) for k in UPDATE_PARAM_NAMES])

    def forward(self, w, X, E, y, mask, O, A, ws, stream=None):
        p = self.attn_params(w)
        _check(self.lib, self.lib.edge_attn_forward(
            self.ctx, ctypes.byref(p), _ptr(X), _ptr(E), _ptr(y), _ptr(mask), _ptr(O), _ptr(A),
            _ptr(ws), self._ws_len(ws), _stream(stream)))

    @property
    def recomputes_update(self) -> bool:
        """edge_update recomputes the logits (two-pass mode or the unnormalized variant)."""
        return self.two_pass or bool(self.desc.flags & EA_VARIANT_UNNORMALIZED)

    def update(self, w, E, y, mask, A, E_out, ws, stream=None):
        p = self.attn_params(w) if w.get("w_q") is not None else None
        u = self.update_params(w)
        _check(self.lib, self.lib.edge_update(
            self.ctx, ctypes.byref(p) if p is not None else None, ctypes.byref(u), _ptr(E), _ptr(y),
            _ptr(mask), _ptr(A), _ptr(E_out), _ptr(ws), self._ws_len(ws), _stream(stream)))

    def layer(self, w, X, E, y, mask, O, A, E_out, ws, stream=None):
        p = self.attn_params(w)
        u = self.update_params(w)
        _check(self.lib, self.lib.edge_attn_layer(
            self.ctx, ctypes.byref(p), ctypes.byref(u), _ptr(X), _ptr(E), _ptr(y), _ptr(mask),
            _ptr(O), _ptr(A), _ptr(E_out), _ptr(ws), self._ws_len(ws), _stream(stream)))

    def bind_layer(self, w, X, E, y, mask, O, A, E_out, ws, stream=None):
        """Marshal the arguments of one layer call once; returns a callable
        that launches it (on `stream`, else the current stream at bind time)."""
        p = self.attn_params(w)
        u = self.update_params(w)
        args = (self.ctx, ctypes.byref(p), ctypes.byref(u), _ptr(X), _ptr(E), _ptr(y), _ptr(mask),
                _ptr(O), _ptr(A), _ptr(E_out), _ptr(ws), self._ws_len(ws), _stream(stream))
        fn, lib = self.lib.edge_attn_layer, self.lib
        keep = (p, u, w, X, E, y, mask, O, A, E_out, ws)  # keep the tensors alive

        def call():
            st = fn(*args)
            if st != EA_OK:
                _check(lib, st)
        call.keep = keep
        return call

    @property
    def backward_workspace_bytes(self) -> int:
        return int(self.lib.ea_backward_workspace_bytes(self.ctx))

    def backward(self, w, X, E, y, mask, A, dO, dEp, dX, dE, dy, grads: Dict, ws, bws, stream=None):
        """Gradients of the layer after a forward on this context (grads: float32 tensors by name)."""
        p = self.attn_params(w)
        u = self.update_params(w)
        g = Grads(*[_ptr(grads[name]) for name, _ in Grads._fields_])
        _check(self.lib, self.lib.edge_attn_backward(
            self.ctx, ctypes.byref(p), ctypes.byref(u), _ptr(X), _ptr(E), _ptr(y), _ptr(mask), _ptr(A),
            _ptr(dO), _ptr(dEp), _ptr(dX), _ptr(dE), _ptr(dy), ctypes.byref(g),
            _ptr(ws), self._ws_len(ws), _ptr(bws), self._ws_len(bws), _stream(stream)))

    @property
    def block_workspace_bytes(self) -> int:
        return int(self.lib.ea_block_workspace_bytes(self.ctx))

    def bind_block(self, w, bp: Dict, X, E, y, mask, X_out, E_out, y_out, ws, stream=None):
        """Marshal the arguments of one block call (layer weights w, block
        parameters bp by name) once; returns a callable that launches it."""
        p = self.attn_params(w)
        u = self.update_params(w)
        b = BlockParams(*[_ptr(bp[name]) for name in BLOCK_PARAM_NAMES])
        args = (self.ctx, ctypes.byref(p), ctypes.byref(u), ctypes.byref(b), _ptr(X), _ptr(E), _ptr(y), _ptr(mask),
                _ptr(X_out), _ptr(E_out), _ptr(y_out), _ptr(ws), self._ws_len(ws), _stream(stream))
        fn, lib = self.lib.edge_attn_block, self.lib
        keep = (p, u, b, w, bp, X, E, y, mask, X_out, E_out, y_out, ws)

        def call():
            st = fn(*args)
            if st != EA_OK:
                _check(lib, st)
        call.keep = keep
        return call

    def block(self, w, bp: Dict, X, E, y, mask, X_out, E_out, y_out, ws, stream=None):
        """One graph-transformer block (the layer, then the node, edge and y paths)."""
        self.bind_block(w, bp, X, E, y, mask, X_out, E_out, y_out, ws, stream)()

    def debug_logits(self, w, X, E, y, mask, U, ws, stream=None):
        p = self.attn_params(w)
        _check(self.lib, self.lib.ea_debug_logits(
            self.ctx, ctypes.byref(p), _ptr(X), _ptr(E), _ptr(y), _ptr(mask), _ptr(U),
            _ptr(ws), self._ws_len(ws), _stream(stream)))

    def profile_begin(self):
        _check(self.lib, self.lib.ea_profile_begin(self.ctx))

    def profile_end(self) -> Dict[str, tuple]:
        ms = (ctypes.c_double * len(KERNELS))()
        cnt = (ctypes.c_int64 * len(KERNELS))()
        _check(self.lib, self.lib.ea_profile_end(self.ctx, ms, cnt))
        return {KERNELS[k]: (ms[k], cnt[k]) for k in range(len(KERNELS))}

    def _ws_len(self, ws) -> int:
        if ws is None:
            return 0
        if isinstance(ws, int):
            return self.workspace_bytes
        return ws.numel() * ws.element_size()
