"""The Python binding's argument checks, on the CPU.

The C ABI receives bare pointers and cannot see where a buffer lives, what
element type it holds or how long it is; a host tensor, a bfloat16 tensor in
a float32 context or a short edge tensor would make the kernels read or write
out of bounds. The binding therefore checks every tensor before its pointer
is passed: a torch tensor, contiguous, the context's element type (uint8 for
the mask, float32 for gradients and the logit export), the exact shape from
the context, then the current CUDA device. Every call here fails in those
checks, before any foreign call, so no GPU is needed.
"""
import pytest
import torch

from edge_aware_graph_amd import layer as L

B, n, d, de, dy, H, dh = 2, 12, 64, 16, 16, 4, 16


@pytest.fixture(scope="module")
def ctx():
    L.load_library()
    return L.EdgeAttention(B, n, d, de, dy, H, dh, "fp32")


def host_args(dt=torch.float32):
    w = {"w_q": torch.zeros(d, d, dtype=dt), "w_k": torch.zeros(d, d, dtype=dt), "w_v": torch.zeros(d, d, dtype=dt),
         "w_emul": torch.zeros(H, de, dtype=dt), "w_eadd": torch.zeros(H, de, dtype=dt),
         "w_ymul": torch.zeros(H, dy, dtype=dt), "w_yadd": torch.zeros(H, dy, dtype=dt),
         "w_e": torch.zeros(de, H, dtype=dt)}
    t = dict(X=torch.zeros(B, n, d, dtype=dt), E=torch.zeros(B, n, n, de, dtype=dt), y=torch.zeros(B, dy, dtype=dt),
             mask=torch.ones(B, n, dtype=torch.uint8), O=torch.zeros(B, n, d, dtype=dt),
             A=torch.zeros(B, H, n, n, dtype=dt), Eo=torch.zeros(B, n, n, de, dtype=dt),
             ws=torch.zeros(1 << 16, dtype=torch.uint8))
    return w, t


def call_layer(ctx, w, t):
    ctx.layer(w, t["X"], t["E"], t["y"], t["mask"], t["O"], t["A"], t["Eo"], t["ws"])


def test_host_tensors_are_rejected(ctx):
    w, t = host_args()
    with pytest.raises(ValueError, match="current CUDA device"):
        call_layer(ctx, w, t)


@pytest.mark.parametrize("name", ["X", "E", "y", "O", "A", "Eo"])
def test_wrong_element_type_is_rejected(ctx, name):
    w, t = host_args()
    t[name] = t[name].to(torch.bfloat16)
    with pytest.raises(ValueError, match="dtype torch.bfloat16"):
        call_layer(ctx, w, t)


@pytest.mark.parametrize("name", ["w_q", "w_emul", "w_ymul", "w_e"])
def test_weight_of_wrong_type_or_shape_is_rejected(ctx, name):
    w, t = host_args()
    w[name] = w[name].to(torch.bfloat16)
    with pytest.raises(ValueError, match="dtype"):
        call_layer(ctx, w, t)
    w, t = host_args()
    w[name] = torch.zeros(w[name].shape[0] + 1, w[name].shape[1])  # one row too many
    with pytest.raises(ValueError, match="shape"):
        call_layer(ctx, w, t)
    if name != "w_q":  # [in, out] instead of the nn.Linear [out, in] layout
        w, t = host_args()
        w[name] = w[name].t().contiguous()
        with pytest.raises(ValueError, match="shape"):
            call_layer(ctx, w, t)


@pytest.mark.parametrize("name,shape", [("E", (B, n, n - 1, de)), ("E", (B, n * n * de)), ("X", (B, n, d // 2)),
                                        ("A", (B, H, n, n - 4)), ("Eo", (1, n, n, de)), ("y", (B, dy + 1))])
def test_short_or_reshaped_buffers_are_rejected(ctx, name, shape):
    w, t = host_args()
    t[name] = torch.zeros(shape, dtype=torch.float32)
    with pytest.raises(ValueError, match="shape"):
        call_layer(ctx, w, t)


def test_mask_must_be_uint8_of_the_batch_shape(ctx):
    w, t = host_args()
    t["mask"] = torch.ones(B, n, dtype=torch.bool)
    with pytest.raises(ValueError, match="mask has dtype"):
        call_layer(ctx, w, t)
    w, t = host_args()
    t["mask"] = torch.ones(B, n + 1, dtype=torch.uint8)
    with pytest.raises(ValueError, match="mask has shape"):
        call_layer(ctx, w, t)


def test_non_contiguous_and_raw_pointers_are_rejected(ctx):
    w, t = host_args()
    t["X"] = torch.zeros(B, d, n).transpose(1, 2)
    with pytest.raises(ValueError, match="contiguous"):
        call_layer(ctx, w, t)
    w, t = host_args()
    t["E"] = 0x10000
    with pytest.raises(ValueError, match="torch tensor"):
        call_layer(ctx, w, t)


def test_every_entry_point_checks_before_calling(ctx):
    w, t = host_args()
    for fn in (lambda: ctx.forward(w, t["X"], t["E"], t["y"], t["mask"], t["O"], t["A"], t["ws"]),
               lambda: ctx.update(w, t["E"], t["y"], t["mask"], t["A"], t["Eo"], t["ws"]),
               lambda: ctx.bind_layer(w, t["X"], t["E"], t["y"], t["mask"], t["O"], t["A"], t["Eo"], t["ws"]),
               lambda: ctx.debug_logits(w, t["X"], t["E"], t["y"], t["mask"], torch.zeros(B, H, n, n), t["ws"])):
        with pytest.raises(ValueError, match="current CUDA device"):
            fn()
    with pytest.raises(ValueError, match="U has dtype"):
        ctx.debug_logits(w, t["X"], t["E"], t["y"], t["mask"], torch.zeros(B, H, n, n, dtype=torch.float64), t["ws"])


def test_backward_gradients_must_be_float32(ctx):
    w, t = host_args()
    grads = {k: torch.zeros(tuple(v.shape), dtype=torch.float32) for k, v in w.items()}
    for k, shp in (("b_q", (d,)), ("b_k", (d,)), ("b_v", (d,)), ("b_emul", (H,)), ("b_eadd", (H,)),
                   ("b_ymul", (H,)), ("b_yadd", (H,)), ("b_e", (de,))):
        grads[k] = torch.zeros(shp, dtype=torch.float32)
    grads["w_e"] = torch.zeros(de, H, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="grad w_e has dtype"):
        ctx.backward(w, t["X"], t["E"], t["y"], t["mask"], t["A"], t["O"], t["Eo"], t["O"], t["Eo"], t["y"],
                     grads, t["ws"], t["ws"])


def test_block_parameters_are_checked(ctx):
    from edge_aware_graph_amd import workloads as W
    dims = W.LayerDims(B=B, n=n, d=d, de=de, dy=dy, H=H, dh=dh, dtype="fp32")
    bp = {k: torch.from_numpy(v) for k, v in W.make_block_params(dims).items()}
    bp["w_e1"] = bp["w_e1"].t().contiguous()  # [de, 2 de] instead of [2 de, de]
    w, t = host_args()
    with pytest.raises(ValueError, match="block.w_e1 has shape"):
        ctx.bind_block(w, bp, t["X"], t["E"], t["y"], t["mask"], t["O"], t["Eo"], t["y"], t["ws"])
