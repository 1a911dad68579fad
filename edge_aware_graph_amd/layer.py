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
           "ea_kernel_name", "ea_debug_softmax", "ea_noalloc_max_workspace_bytes", "edge_attn_layer_noalloc",
           "ea_probe_copy", "ea_probe_read")

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
    lib.ea_debug_softmax.restype = ctypes.c_int
    lib.ea_debug_softmax.argtypes = [vp, vp, vp, vp]
    lib.ea_noalloc_max_workspace_bytes.restype = sz
    lib.ea_noalloc_max_workspace_bytes.argtypes = []
    lib.edge_attn_layer_noalloc.restype = ctypes.c_int
    lib.edge_attn_layer_noalloc.argtypes = [vp, ap, up, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.ea_probe_copy.restype = ctypes.c_int
    lib.ea_probe_copy.argtypes = [vp, vp, sz, vp]
    lib.ea_probe_read.restype = ctypes.c_int
    lib.ea_probe_read.argtypes = [vp, sz, vp, vp]
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


def _check_tensor(t, name: str, shape, dtype, what: str = ""):
    """Reject a tensor the C ABI cannot check itself: the library sees only a
    pointer, so a wrong element type or a short buffer would make its kernels
    read or write out of bounds. Checks a torch tensor, contiguous, element
    type and exact shape; None passes (NULL)."""
    if t is None:
        return
    import torch
    if not isinstance(t, torch.Tensor):
        raise ValueError("%s must be a torch tensor (got %s)" % (name, type(t).__name__))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise ValueError("%s has dtype %s, expected %s%s" % (name, t.dtype, dtype, what))
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))


class _Args:
    """The tensor arguments of one call. `add` checks each tensor's type,
    contiguity, element type and shape as it comes; `ptrs` then checks that
    every one lives on the current CUDA device (a host tensor would be read
    through a host address) and returns the pointers in order."""

    def __init__(self, ea: "EdgeAttention"):
        self.ea = ea
        self.items = []

    def add(self, name: str, t, kind: str = "layer", key: Optional[str] = None):
        import torch
        shape = None if kind == "bytes" else self.ea._shapes[key or name]
        if kind == "layer":
            _check_tensor(t, name, shape, self.ea._tdtype(), " (the context's dtype is %s)" % self.ea.dtype)
        else:
            _check_tensor(t, name, shape, {"u8": torch.uint8, "f32": torch.float32, "bytes": None}[kind])
        self.items.append((name, t))

    def ptrs(self):
        import torch
        out = []
        for name, t in self.items:
            if t is None:
                out.append(None)
                continue
            if t.device.type != "cuda" or t.device.index != torch.cuda.current_device():
                raise ValueError("%s is on %s, expected the current CUDA device" % (name, t.device))
            out.append(t.data_ptr())
        return out


def _stream(stream) -> Optional[int]:
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _probe_tensor(t, name: str):
    import torch
    if not isinstance(t, torch.Tensor) or not t.is_contiguous():
        raise ValueError("%s must be a contiguous torch tensor" % name)
    if t.device.type != "cuda" or t.device.index != torch.cuda.current_device():
        raise ValueError("%s is on %s, expected the current CUDA device" % (name, t.device))
    return t.numel() * t.element_size()


def probe_copy(src, dst, stream=None) -> None:
    """ea_probe_copy over the whole of src into dst (same byte size)."""
    nb = _probe_tensor(src, "src")
    if _probe_tensor(dst, "dst") != nb:
        raise ValueError("src and dst must hold the same number of bytes")
    lib = load_library()
    _check(lib, lib.ea_probe_copy(src.data_ptr(), dst.data_ptr(), nb, _stream(stream)))


def probe_read(src, xor_out, stream=None) -> None:
    """ea_probe_read over the whole of src; xor_out: an int32 tensor of one element."""
    import torch
    nb = _probe_tensor(src, "src")
    _probe_tensor(xor_out, "xor_out")
    if xor_out.dtype != torch.int32 or xor_out.numel() != 1:
        raise ValueError("xor_out must be one int32 element")
    lib = load_library()
    _check(lib, lib.ea_probe_read(src.data_ptr(), nb, xor_out.data_ptr(), _stream(stream)))


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
        self._shapes = self._arg_shapes()

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

    def _arg_shapes(self) -> Dict[str, tuple]:
        """Shape of every tensor argument, by name, from the context's desc."""
        dsc = self.desc
        B, n, d, de, dy, H = dsc.B, dsc.n, dsc.d, dsc.de, dsc.dy, dsc.H
        sh = {"X": (B, n, d), "E": (B, n, n, de), "y": (B, dy), "mask": (B, n), "O": (B, n, d),
              "A": (B, H, n, n), "E_out": (B, n, n, de), "U": (B, H, n, n),
              "dO": (B, n, d), "dE_out": (B, n, n, de), "dX": (B, n, d), "dE": (B, n, n, de), "dy": (B, dy),
              "X_out": (B, n, d), "y_out": (B, dy),
              "w_q": (d, d), "w_k": (d, d), "w_v": (d, d), "b_q": (d,), "b_k": (d,), "b_v": (d,),
              "w_emul": (H, de), "w_eadd": (H, de), "b_emul": (H,), "b_eadd": (H,),
              "w_ymul": (H, dy), "w_yadd": (H, dy), "b_ymul": (H,), "b_yadd": (H,),
              "w_e": (de, H), "b_e": (de,)}
        blk = {"w_o": (d, d), "b_o": (d,), "ln_x1_g": (d,), "ln_x1_b": (d,), "w_x1": (d, d), "b_x1": (d,),
               "w_x2": (d, d), "b_x2": (d,), "ln_x2_g": (d,), "ln_x2_b": (d,),
               "ln_e1_g": (de,), "ln_e1_b": (de,), "w_e1": (2 * de, de), "b_e1": (2 * de,),
               "w_e2": (de, 2 * de), "b_e2": (de,), "ln_e2_g": (de,), "ln_e2_b": (de,),
               "w_yy": (dy, dy), "w_yx": (dy, d), "w_ye": (dy, de), "b_yo": (dy,), "ln_y1_g": (dy,),
               "ln_y1_b": (dy,), "w_y1": (dy, dy), "b_y1": (dy,), "w_y2": (dy, dy), "b_y2": (dy,),
               "ln_y2_g": (dy,), "ln_y2_b": (dy,)}
        sh.update({"block." + k: v for k, v in blk.items()})
        return sh

    def _tdtype(self):
        import torch
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    def _args(self, w: Optional[Dict] = None, attn: bool = False, update: bool = False) -> _Args:
        """A checked argument list, starting with the attention and/or update
        parameters of `w` (absent names are NULL)."""
        a = _Args(self)
        for k in (ATTN_PARAM_NAMES if attn else ()) + (UPDATE_PARAM_NAMES if update else ()):
            a.add(k, w.get(k))
        return a

    def attn_params(self, w: Dict) -> AttnParams:
        return AttnParams(*self._args(w, attn=True).ptrs())

    def update_params(self, w: Dict) -> UpdateParams:
        return UpdateParams(*self._args(w, update=True).ptrs())

    @staticmethod
    def _split(ptrs, k: int):
        return ptrs[:k], ptrs[k:]

    def forward(self, w, X, E, y, mask, O, A, ws, stream=None):
        a = self._args(w, attn=True)
        for name, t in (("X", X), ("E", E), ("y", y)):
            a.add(name, t)
        a.add("mask", mask, "u8")
        a.add("O", O)
        a.add("A", A)
        a.add("ws", ws, "bytes")
        pp, rest = self._split(a.ptrs(), len(ATTN_PARAM_NAMES))
        p = AttnParams(*pp)
        _check(self.lib, self.lib.edge_attn_forward(self.ctx, ctypes.byref(p), *rest, self._ws_len(ws),
                                                    _stream(stream)))

    @property
    def recomputes_update(self) -> bool:
        """edge_update recomputes the logits (two-pass mode or the unnormalized variant)."""
        return self.two_pass or bool(self.desc.flags & EA_VARIANT_UNNORMALIZED)

    def update(self, w, E, y, mask, A, E_out, ws, stream=None):
        with_p = w.get("w_q") is not None
        a = self._args(w, attn=with_p, update=True)
        a.add("E", E)
        a.add("y", y)
        a.add("mask", mask, "u8")
        a.add("A", A)
        a.add("E_out", E_out)
        a.add("ws", ws, "bytes")
        ptrs = a.ptrs()
        npar = len(ATTN_PARAM_NAMES) if with_p else 0
        p = AttnParams(*ptrs[:npar]) if with_p else None
        u = UpdateParams(*ptrs[npar:npar + len(UPDATE_PARAM_NAMES)])
        rest = ptrs[npar + len(UPDATE_PARAM_NAMES):]
        _check(self.lib, self.lib.edge_update(
            self.ctx, ctypes.byref(p) if p is not None else None, ctypes.byref(u), *rest, self._ws_len(ws),
            _stream(stream)))

    def _layer_args(self, w, X, E, y, mask, O, A, E_out, ws, stream):
        a = self._args(w, attn=True, update=True)
        for name, t in (("X", X), ("E", E), ("y", y)):
            a.add(name, t)
        a.add("mask", mask, "u8")
        for name, t in (("O", O), ("A", A), ("E_out", E_out)):
            a.add(name, t)
        a.add("ws", ws, "bytes")
        ptrs = a.ptrs()
        na, nu = len(ATTN_PARAM_NAMES), len(UPDATE_PARAM_NAMES)
        p, u = AttnParams(*ptrs[:na]), UpdateParams(*ptrs[na:na + nu])
        return p, u, (self.ctx, ctypes.byref(p), ctypes.byref(u), *ptrs[na + nu:], self._ws_len(ws), _stream(stream))

    def layer(self, w, X, E, y, mask, O, A, E_out, ws, stream=None):
        p, u, args = self._layer_args(w, X, E, y, mask, O, A, E_out, ws, stream)
        _check(self.lib, self.lib.edge_attn_layer(*args))

    def layer_noalloc(self, w, X, E, y, mask, O, A, E_out, stream=None):
        """edge_attn_layer without a workspace argument (the library's own device array)."""
        a = self._args(w, attn=True, update=True)
        for name, t in (("X", X), ("E", E), ("y", y)):
            a.add(name, t)
        a.add("mask", mask, "u8")
        for name, t in (("O", O), ("A", A), ("E_out", E_out)):
            a.add(name, t)
        ptrs = a.ptrs()
        na, nu = len(ATTN_PARAM_NAMES), len(UPDATE_PARAM_NAMES)
        p, u = AttnParams(*ptrs[:na]), UpdateParams(*ptrs[na:na + nu])
        _check(self.lib, self.lib.edge_attn_layer_noalloc(self.ctx, ctypes.byref(p), ctypes.byref(u),
                                                          *ptrs[na + nu:], _stream(stream)))

    def bind_layer(self, w, X, E, y, mask, O, A, E_out, ws, stream=None):
        """Marshal the arguments of one layer call once; returns a callable
        that launches it (on `stream`, else the current stream at bind time)."""
        p, u, args = self._layer_args(w, X, E, y, mask, O, A, E_out, ws, stream)
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
        a = self._args(w, attn=True, update=True)
        for name, t in (("X", X), ("E", E), ("y", y)):
            a.add(name, t)
        a.add("mask", mask, "u8")
        for name, t in (("A", A), ("dO", dO), ("dE_out", dEp), ("dX", dX), ("dE", dE), ("dy", dy)):
            a.add(name, t)
        gnames = [name for name, _ in Grads._fields_]
        for name in gnames:
            a.add("grad " + name, grads[name], "f32", key=name)
        a.add("ws", ws, "bytes")
        a.add("bws", bws, "bytes")
        ptrs = a.ptrs()
        na, nu = len(ATTN_PARAM_NAMES), len(UPDATE_PARAM_NAMES)
        p, u = AttnParams(*ptrs[:na]), UpdateParams(*ptrs[na:na + nu])
        io = ptrs[na + nu:na + nu + 10]
        g = Grads(*ptrs[na + nu + 10:na + nu + 10 + len(gnames)])
        pws, pbws = ptrs[-2], ptrs[-1]
        _check(self.lib, self.lib.edge_attn_backward(
            self.ctx, ctypes.byref(p), ctypes.byref(u), *io, ctypes.byref(g),
            pws, self._ws_len(ws), pbws, self._ws_len(bws), _stream(stream)))

    @property
    def block_workspace_bytes(self) -> int:
        return int(self.lib.ea_block_workspace_bytes(self.ctx))

    def bind_block(self, w, bp: Dict, X, E, y, mask, X_out, E_out, y_out, ws, stream=None):
        """Marshal the arguments of one block call (layer weights w, block
        parameters bp by name) once; returns a callable that launches it."""
        a = self._args(w, attn=True, update=True)
        for name in BLOCK_PARAM_NAMES:
            a.add("block." + name, bp[name])
        for name, t in (("X", X), ("E", E), ("y", y)):
            a.add(name, t)
        a.add("mask", mask, "u8")
        for name, t in (("X_out", X_out), ("E_out", E_out), ("y_out", y_out)):
            a.add(name, t)
        a.add("ws", ws, "bytes")
        ptrs = a.ptrs()
        na, nu, nb = len(ATTN_PARAM_NAMES), len(UPDATE_PARAM_NAMES), len(BLOCK_PARAM_NAMES)
        p, u = AttnParams(*ptrs[:na]), UpdateParams(*ptrs[na:na + nu])
        b = BlockParams(*ptrs[na + nu:na + nu + nb])
        args = (self.ctx, ctypes.byref(p), ctypes.byref(u), ctypes.byref(b), *ptrs[na + nu + nb:],
                self._ws_len(ws), _stream(stream))
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
        a = self._args(w, attn=True)
        for name, t in (("X", X), ("E", E), ("y", y)):
            a.add(name, t)
        a.add("mask", mask, "u8")
        a.add("U", U, "f32")
        a.add("ws", ws, "bytes")
        pp, rest = self._split(a.ptrs(), len(ATTN_PARAM_NAMES))
        p = AttnParams(*pp)
        _check(self.lib, self.lib.ea_debug_logits(self.ctx, ctypes.byref(p), *rest, self._ws_len(ws),
                                                  _stream(stream)))

    def debug_softmax(self, U, A, stream=None):
        """Softmax stage alone: A = softmax over keys of float32 logits U [B, H, n, n]."""
        a = _Args(self)
        a.add("U", U, "f32")
        a.add("A", A)
        pU, pA = a.ptrs()
        _check(self.lib, self.lib.ea_debug_softmax(self.ctx, pU, pA, _stream(stream)))

    def profile_begin(self):
        _check(self.lib, self.lib.ea_profile_begin(self.ctx))

    def profile_end(self) -> Dict[str, tuple]:
        ms = (ctypes.c_double * len(KERNELS))()
        cnt = (ctypes.c_int64 * len(KERNELS))()
        _check(self.lib, self.lib.ea_profile_end(self.ctx, ms, cnt))
        return {KERNELS[k]: (ms[k], cnt[k]) for k in range(len(KERNELS))}

    @staticmethod
    def _ws_len(ws) -> int:
        return 0 if ws is None else ws.numel() * ws.element_size()
