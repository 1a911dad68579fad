"""C-ABI boundary on the CPU: the library loads, exports what include/edge_attn.h
declares, and rejects bad arguments before anything is enqueued.

No call here reaches a kernel launch: every call is built to fail validation,
so fake (never dereferenced) pointer values are safe.
"""
import ctypes
import os
import re

import pytest

from edge_aware_graph_amd import layer as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "edge_attn.h")

FAKE = 0x10000  # 64 KiB: 256-byte aligned, never dereferenced
MISALIGNED = 0x10008


@pytest.fixture(scope="module")
def lib():
    return L.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ea_\w+|edge_\w+)\s*\(", text)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(L.EXPORTS), names
    for name in names:
        assert hasattr(lib, name), name


def make_desc(B=2, n=12, d=64, de=16, dy=16, H=4, dh=16, dtype=L.EA_FP32, flags=0):
    return L.Desc(B, n, d, de, dy, H, dh, dtype, flags)


def create(lib, desc):
    ctx = ctypes.c_void_p()
    st = lib.ea_ctx_create(ctypes.byref(desc), ctypes.byref(ctx))
    return st, ctx


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), L.EA_E_SHAPE), (dict(n=0), L.EA_E_SHAPE), (dict(dy=0), L.EA_E_SHAPE),
    (dict(d=60), L.EA_E_SHAPE), (dict(B=70000), L.EA_E_SHAPE),
    (dict(dtype=7), L.EA_E_UNSUPPORTED), (dict(flags=0x10), L.EA_E_UNSUPPORTED),
    (dict(d=96, H=2, dh=48), L.EA_E_UNSUPPORTED), (dict(d=32, H=4, dh=8), L.EA_E_UNSUPPORTED),
    (dict(de=24), L.EA_E_UNSUPPORTED), (dict(de=8), L.EA_E_UNSUPPORTED),
    (dict(d=17 * 16, H=17, dh=16), L.EA_E_UNSUPPORTED),
    (dict(), L.EA_OK), (dict(d=256, de=64, dy=64, H=8, dh=32, dtype=L.EA_BF16), L.EA_OK),
    # shapes without tuned kernels take the generic path
    (dict(d=512, de=64, dy=64, H=8, dh=64, dtype=L.EA_BF16), L.EA_OK),
    (dict(d=128, de=32, H=4, dh=32), L.EA_OK), (dict(d=64, H=2, dh=32), L.EA_OK),
    (dict(d=256, de=16, H=16, dh=16), L.EA_OK), (dict(d=1024, de=128, H=16, dh=64), L.EA_OK),
    (dict(d=64, de=48, H=1, dh=64, dtype=L.EA_BF16), L.EA_OK),
])
def test_ctx_create_validation(lib, kw, status):
    st, ctx = create(lib, make_desc(**kw))
    assert st == status, lib.ea_last_error()
    if st == L.EA_OK:
        assert ctx.value
        lib.ea_ctx_destroy(ctx)
    else:
        assert not ctx.value and lib.ea_last_error()


def test_null_desc(lib):
    ctx = ctypes.c_void_p()
    assert lib.ea_ctx_create(None, ctypes.byref(ctx)) == L.EA_E_NULLPTR


def test_mode_and_workspace_plan(lib):
    for n, flags, two in ((256, 0, 0), (257, 0, 1), (12, L.EA_FORCE_TWO_PASS, 1), (1024, 0, 1)):
        st, ctx = create(lib, make_desc(B=3, n=n, d=256, de=64, dy=64, H=8, dh=32, dtype=L.EA_BF16, flags=flags))
        assert st == L.EA_OK
        assert lib.ea_is_two_pass(ctx) == two
        NP = (n + 15) // 16 * 16
        qkv = -(-3 * 8 * NP * 32 * 2 // 256) * 256
        lse = -(-3 * 8 * NP * 4 // 256) * 256
        gy = -(-3 * 2 * 8 * 4 // 256) * 256
        order = -(-3 * (NP // 16) * 4 // 256) * 256
        assert lib.ea_workspace_bytes(ctx) == 3 * qkv + lse + gy + order
        lib.ea_ctx_destroy(ctx)
    assert lib.ea_is_two_pass(None) == -1
    assert lib.ea_workspace_bytes(None) == 0


def attn_params(**over):
    vals = {k: FAKE for k in L.ATTN_PARAM_NAMES if k.startswith("w_")}
    vals.update(over)
    return L.AttnParams(*[vals.get(k) for k in L.ATTN_PARAM_NAMES])


def fwd(lib, ctx, p=None, X=FAKE, E=FAKE, y=FAKE, mask=FAKE, O=FAKE, A=FAKE, ws=FAKE, ws_bytes=1 << 40):
    p = attn_params() if p is None else p
    return lib.edge_attn_forward(ctx, ctypes.byref(p), X, E, y, mask, O, A, ws, ws_bytes, None)


@pytest.fixture
def ctx1(lib):
    st, ctx = create(lib, make_desc())
    assert st == L.EA_OK
    yield ctx
    lib.ea_ctx_destroy(ctx)


@pytest.fixture
def ctx2(lib):
    st, ctx = create(lib, make_desc(n=300))
    assert st == L.EA_OK and lib.ea_is_two_pass(ctx) == 1
    yield ctx
    lib.ea_ctx_destroy(ctx)


def test_forward_argument_errors(lib, ctx1):
    assert fwd(lib, None) == L.EA_E_NULLPTR
    assert fwd(lib, ctx1, X=None) == L.EA_E_NULLPTR
    assert b"X" in lib.ea_last_error()
    assert fwd(lib, ctx1, E=MISALIGNED) == L.EA_E_ALIGN
    assert fwd(lib, ctx1, O=None) == L.EA_E_NULLPTR
    assert fwd(lib, ctx1, A=None) == L.EA_E_NULLPTR
    assert fwd(lib, ctx1, mask=None) == L.EA_E_NULLPTR
    assert fwd(lib, ctx1, p=attn_params(w_q=None)) == L.EA_E_NULLPTR
    assert fwd(lib, ctx1, p=attn_params(w_emul=MISALIGNED)) == L.EA_E_ALIGN
    assert fwd(lib, ctx1, ws=None) == L.EA_E_WORKSPACE
    assert fwd(lib, ctx1, ws=FAKE + 16) == L.EA_E_ALIGN
    assert fwd(lib, ctx1, ws_bytes=lib.ea_workspace_bytes(ctx1) - 1) == L.EA_E_WORKSPACE
    assert lib.edge_attn_forward(ctx1, None, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 1 << 40, None) == L.EA_E_NULLPTR


def test_two_pass_rules(lib, ctx2):
    # two-pass forward produces no A
    assert fwd(lib, ctx2) == L.EA_E_UNSUPPORTED
    # update before any forward on this context
    p = attn_params()
    u = L.UpdateParams(FAKE, None)
    st = lib.edge_update(ctx2, ctypes.byref(p), ctypes.byref(u), FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 40, None)
    assert st == L.EA_E_STATE
    assert b"edge_attn_forward" in lib.ea_last_error()


def test_update_and_layer_argument_errors(lib, ctx1):
    p = attn_params()
    u = L.UpdateParams(FAKE, None)
    upd = lambda **k: lib.edge_update(ctx1, ctypes.byref(p), k.get("u", ctypes.byref(u)), k.get("E", FAKE), FAKE, k.get("mask", FAKE),
                                      k.get("A", FAKE), k.get("Eo", FAKE), FAKE, 1 << 40, None)
    assert upd(u=None) == L.EA_E_NULLPTR
    assert upd(A=None) == L.EA_E_NULLPTR
    assert upd(Eo=MISALIGNED) == L.EA_E_ALIGN
    assert upd(mask=None) == L.EA_E_NULLPTR
    bad_u = L.UpdateParams(None, None)
    assert upd(u=ctypes.byref(bad_u)) == L.EA_E_NULLPTR
    layer = lambda **k: lib.edge_attn_layer(ctx1, ctypes.byref(p), k.get("u", ctypes.byref(u)), FAKE, FAKE, FAKE, FAKE, FAKE,
                                            FAKE, k.get("Eo", FAKE), FAKE, k.get("wsb", 1 << 40), None)
    assert layer(u=None) == L.EA_E_NULLPTR
    assert layer(Eo=None) == L.EA_E_NULLPTR
    assert layer(wsb=0) == L.EA_E_WORKSPACE


def test_status_strings(lib):
    for s in range(8):
        assert lib.ea_status_str(s)
    assert lib.ea_status_str(99) == b"unknown status"
    assert lib.ea_kernel_name(0) == b"qkv_kernel"


def test_binding_raises_on_bad_shape():
    with pytest.raises(L.EaError) as e:
        L.EdgeAttention(1, 4, 64, 16, 16, 4, 8, "fp32")
    assert e.value.status == L.EA_E_SHAPE


@pytest.mark.parametrize("flags", [L.EA_VARIANT_LIGHT_EDGE, L.EA_VARIANT_NO_SCORE_MOD, L.EA_VARIANT_UNNORMALIZED,
                                   L.EA_VARIANT_LIGHT_EDGE | L.EA_VARIANT_UNNORMALIZED | L.EA_FORCE_TWO_PASS])
def test_variant_flags_accepted(lib, flags):
    st, ctx = create(lib, make_desc(flags=flags))
    assert st == L.EA_OK, lib.ea_last_error()
    lib.ea_ctx_destroy(ctx)


def test_variant_parameters_that_are_not_read_may_be_null(lib):
    """Light edge does not read the edge FiLM, no-score-modulation no FiLM and no y:
    NULL passes the parameter checks (the call then stops at the missing workspace)."""
    no_edge_film = attn_params(w_emul=None, w_eadd=None)
    no_film = attn_params(w_emul=None, w_eadd=None, w_ymul=None, w_yadd=None)
    st, plain = create(lib, make_desc())
    assert fwd(lib, plain, p=no_edge_film, ws=None) == L.EA_E_NULLPTR
    assert fwd(lib, plain, y=None, ws=None) == L.EA_E_NULLPTR
    lib.ea_ctx_destroy(plain)
    st, light = create(lib, make_desc(flags=L.EA_VARIANT_LIGHT_EDGE))
    assert fwd(lib, light, p=no_edge_film, ws=None) == L.EA_E_WORKSPACE
    assert fwd(lib, light, p=no_film, ws=None) == L.EA_E_NULLPTR  # the global FiLM is still read
    lib.ea_ctx_destroy(light)
    st, nomod = create(lib, make_desc(flags=L.EA_VARIANT_NO_SCORE_MOD))
    assert fwd(lib, nomod, p=no_film, y=None, ws=None) == L.EA_E_WORKSPACE
    lib.ea_ctx_destroy(nomod)


def test_unnormalized_update_needs_the_forward(lib):
    """The unnormalized variant's edge_update recomputes the logits: like two-pass mode it
    needs a preceding forward on the context (A is not used)."""
    st, ctx = create(lib, make_desc(flags=L.EA_VARIANT_UNNORMALIZED))
    assert st == L.EA_OK and lib.ea_is_two_pass(ctx) == 0
    p = attn_params()
    u = L.UpdateParams(FAKE, None)
    st = lib.edge_update(ctx, ctypes.byref(p), ctypes.byref(u), FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 40, None)
    assert st == L.EA_E_STATE
    assert b"edge_attn_forward" in lib.ea_last_error()
    lib.ea_ctx_destroy(ctx)


def test_backward_rules(lib):
    """The backward needs a single-pass context, no variant, a preceding forward."""
    g = L.Grads(*([FAKE] * 16))
    p = attn_params()
    u = L.UpdateParams(FAKE, None)

    def bwd(ctx, **k):
        return lib.edge_attn_backward(ctx, ctypes.byref(p), ctypes.byref(u), FAKE, FAKE, FAKE, FAKE, FAKE,
                                      FAKE, FAKE, FAKE, FAKE, FAKE, k.get("g", ctypes.byref(g)), FAKE, 1 << 40,
                                      k.get("bws", FAKE), k.get("bwsb", 1 << 40), None)
    for kw in (dict(flags=L.EA_VARIANT_LIGHT_EDGE),
               dict(d=256, de=64, dy=64, H=8, dh=32, dtype=L.EA_FP32),
               dict(d=128, de=32, H=4, dh=32), dict(d=512, de=64, dy=64, H=8, dh=64, dtype=L.EA_BF16)):
        st, ctx = create(lib, make_desc(**kw))
        assert st == L.EA_OK
        assert bwd(ctx) == L.EA_E_UNSUPPORTED, kw
        lib.ea_ctx_destroy(ctx)
    st, ctx = create(lib, make_desc())
    assert lib.ea_backward_workspace_bytes(ctx) > 0
    assert bwd(ctx, g=None) == L.EA_E_NULLPTR
    assert bwd(ctx, bws=None) == L.EA_E_WORKSPACE
    assert bwd(ctx, bwsb=16) == L.EA_E_WORKSPACE
    assert bwd(ctx) == L.EA_E_STATE  # no forward on this context yet
    lib.ea_ctx_destroy(ctx)
    for kw in (dict(n=200, B=3), dict(n=300), dict(flags=L.EA_FORCE_TWO_PASS)):  # several key blocks / two-pass
        st, ctx = create(lib, make_desc(**kw))
        assert st == L.EA_OK
        assert bwd(ctx) == L.EA_E_STATE, kw
        lib.ea_ctx_destroy(ctx)


def test_block_rules(lib):
    """The block: built shapes, no variant, every parameter present and aligned, a workspace of the block's size."""
    p = attn_params()
    u = L.UpdateParams(FAKE, None)
    bp = L.BlockParams(*([FAKE] * len(L.BLOCK_PARAM_NAMES)))

    def blk(ctx, **k):
        return lib.edge_attn_block(ctx, ctypes.byref(p), ctypes.byref(u), k.get("bp", ctypes.byref(bp)),
                                   FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, k.get("y_out", FAKE),
                                   k.get("ws", FAKE), k.get("wsb", 1 << 40), None)
    assert ctypes.sizeof(L.BlockParams) == 30 * ctypes.sizeof(ctypes.c_void_p)
    for kw in (dict(flags=L.EA_VARIANT_NO_SCORE_MOD), dict(d=256, de=64, dy=64, H=8, dh=32, dtype=L.EA_FP32),
               dict(d=128, de=32, H=4, dh=32), dict(dy=1024)):
        st, ctx = create(lib, make_desc(**kw))
        if st != L.EA_OK:  # a shape the library does not build at all
            continue
        assert blk(ctx) == L.EA_E_UNSUPPORTED, kw
        lib.ea_ctx_destroy(ctx)
    for two_pass in (False, True):
        st, ctx = create(lib, make_desc(n=300 if two_pass else 12))
        assert st == L.EA_OK
        wsb = lib.ea_block_workspace_bytes(ctx)
        assert wsb > lib.ea_workspace_bytes(ctx)
        assert blk(ctx, bp=None) == L.EA_E_NULLPTR
        for q in range(len(L.BLOCK_PARAM_NAMES)):
            vals = [FAKE] * len(L.BLOCK_PARAM_NAMES)
            vals[q] = None
            assert blk(ctx, bp=ctypes.byref(L.BlockParams(*vals))) == L.EA_E_NULLPTR, L.BLOCK_PARAM_NAMES[q]
            vals[q] = MISALIGNED
            assert blk(ctx, bp=ctypes.byref(L.BlockParams(*vals))) == L.EA_E_ALIGN, L.BLOCK_PARAM_NAMES[q]
        assert blk(ctx, y_out=None) == L.EA_E_NULLPTR
        assert blk(ctx, ws=None) == L.EA_E_WORKSPACE
        assert blk(ctx, wsb=wsb - 1) == L.EA_E_WORKSPACE
        assert "block" in lib.ea_kernel_name(L.KERNELS.index("block (node, edge, y kernels)")).decode()
        lib.ea_ctx_destroy(ctx)


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    """No fallback: without the built HIP library the binding raises."""
    monkeypatch.setattr(L, "_lib", None)
    with pytest.raises(RuntimeError, match="missing"):
        L.load_library(str(tmp_path / "libedge_attn.so"))


def test_sampling_loop_checks_block_parameters():
    from edge_aware_graph_amd import workloads as W
    from edge_aware_graph_amd.sampling import SamplingLoop
    dims = W.CONFIGS["tiny"].dims
    with pytest.raises(ValueError, match="one set of block parameters per layer"):
        SamplingLoop(dims, [{}], device="cpu", block_params=[{}, {}])


def test_softmax_stage_export_rules(lib):
    """ea_debug_softmax checks its pointers before launching anything."""
    st, ctx = create(lib, make_desc())
    assert st == L.EA_OK
    assert lib.ea_debug_softmax(ctx, None, FAKE, None) == L.EA_E_NULLPTR
    assert lib.ea_debug_softmax(ctx, FAKE, None, None) == L.EA_E_NULLPTR
    assert lib.ea_debug_softmax(ctx, MISALIGNED, FAKE, None) == L.EA_E_ALIGN
    assert lib.ea_debug_softmax(None, FAKE, FAKE, None) == L.EA_E_NULLPTR
    lib.ea_ctx_destroy(ctx)


def test_generic_logit_export_has_no_row_limit(lib):
    """The tuned logit export stops at n = 256 (checked after the workspace);
    a generic shape has no such rule and fails here only on its workspace."""
    p = attn_params()
    for kw, ws, status in ((dict(n=300), 1 << 40, L.EA_E_UNSUPPORTED),
                           (dict(n=300, d=128, de=32, H=4, dh=32), 16, L.EA_E_WORKSPACE)):
        st, ctx = create(lib, make_desc(**kw))
        assert st == L.EA_OK
        st = lib.ea_debug_logits(ctx, ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, ws, None)
        assert st == status, (kw, lib.ea_last_error())
        lib.ea_ctx_destroy(ctx)


def test_probe_argument_rules(lib):
    """The bandwidth probes check pointers, alignment and size before launching."""
    assert lib.ea_probe_copy(None, FAKE, 4096, None) == L.EA_E_NULLPTR
    assert lib.ea_probe_copy(FAKE, None, 4096, None) == L.EA_E_NULLPTR
    assert lib.ea_probe_copy(MISALIGNED, FAKE, 4096, None) == L.EA_E_ALIGN
    assert lib.ea_probe_copy(FAKE, FAKE, 4100, None) == L.EA_E_ALIGN
    assert lib.ea_probe_copy(None, None, 0, None) == L.EA_OK  # nothing to move
    assert lib.ea_probe_read(None, 4096, FAKE, None) == L.EA_E_NULLPTR
    assert lib.ea_probe_read(FAKE, 4096, None, None) == L.EA_E_NULLPTR
    assert lib.ea_probe_read(FAKE, 4096, FAKE + 2, None) == L.EA_E_ALIGN
    assert lib.ea_probe_read(FAKE, 4100, FAKE, None) == L.EA_E_ALIGN
