"""GPU tests of the residual stream and of a multi-layer decode step.

moe_residual_add is checked bitwise against the oracle's residual_stream.
A two-layer decode step (route -> routed FFN -> residual, twice, on
different weights) is captured as one HIP graph; every replay must give the
eager chain's bits, with eager work between replays.
"""
import numpy as np
import pytest
import torch

import moe_synth as S
from oracle import moe_oracle as O
from parity import DeviceLayer, LayerInputs, to_dev
from sparse_moe_expert_route_amd import binding as B

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T", [1, 7, 16])
def test_residual_add_matches_oracle(dtype, T):
    shape = S.LAYERS["olmoe-like"].with_(dtype=dtype)
    say(f"[case] residual {dtype} T={T}")
    desc = B.make_desc(shape.hidden, shape.n_experts, shape.d_ff, shape.top_k, False, dtype,
                       gate_up_layout="packed")
    x = S.tokens(shape, 30 + T, T)
    y = (np.random.default_rng(T).standard_normal((T, shape.hidden)) * 0.3).astype(np.float32)
    want = O.residual_stream(x, y, dtype)
    x_d, y_d = to_dev(x), torch.from_numpy(y).cuda()
    out = torch.empty_like(x_d)
    B.moe_residual_add(desc, T, x_d, y_d, out)
    B.moe_residual_add(desc, T, x_d, y_d, x_d)            # in place
    torch.cuda.synchronize()
    for got in (out, x_d):
        g = got.view(torch.int16).cpu().numpy().view(np.uint16) if dtype == "bf16" else got.cpu().numpy()
        np.testing.assert_array_equal(g.view(np.uint16 if dtype == "bf16" else np.uint32),
                                      want.view(np.uint16 if dtype == "bf16" else np.uint32))


def test_two_layer_decode_step_graph():
    shape = S.LAYERS["olmoe-like"]
    T, k = 16, B.moe_keep_count(0.9, shape.d_ff)
    say("[case] two-layer decode step, graph vs eager")
    layers = [DeviceLayer(LayerInputs(shape, seed=s)) for s in (0, 1)]
    E, K = shape.n_experts, shape.top_k
    x0 = to_dev(S.tokens(shape, 40, T))
    xs = [torch.empty_like(x0) for _ in layers]
    ys = [torch.empty((T, shape.hidden), dtype=torch.float32, device="cuda") for _ in layers]
    rs = [B.Routing.allocate(T, K, E) for _ in layers]
    d = layers[0].desc
    ws_r = torch.empty(B.moe_route_workspace_size(d, T), dtype=torch.uint8, device="cuda")
    ws = torch.empty(B.moe_ffn_workspace_size(d, T, k, B.MOE_PATH_SPARSE), dtype=torch.uint8,
                     device="cuda")

    def step():
        x = x0
        for L, xo, y, R in zip(layers, xs, ys, rs):
            B.moe_route(L.desc, T, x, L.w_router, L.bias, R, ws_r)
            B.moe_expert_ffn_sparse(L.desc, T, k, x, *L.w, R, y, 0, None, ws)
            B.moe_residual_add(L.desc, T, x, y, xo)
            x = xo

    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in xs + ys]
    assert all(torch.isfinite(t.float()).all() for t in ref)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in xs + ys:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(xs + ys, ref):
            assert torch.equal(a, b), f"replay {rep} differs from the eager step"
        step()                                               # eager work between replays
        torch.cuda.synchronize()


RAGGED_SH = dict(hidden=320, n_experts=12, d_ff=192, top_k=3, norm_topk=True, n_shared=1,
                 d_ff_shared=128, zipf_bias=None)


@pytest.mark.parametrize("name,dtype,T,s,over", [
    ("olmoe-like", "bf16", 1, 0.9, {}),       # select inside the down kernel
    ("olmoe-like", "bf16", 4, 0.9, {}),
    ("olmoe-like", "bf16", 16, 0.9, {}),      # mask kernel + row kernel
    ("olmoe-like", "bf16", 40, 0.9, {}),
    ("olmoe-like", "f32", 5, 0.7, RAGGED_SH),  # routed, then the shared group fused
    ("olmoe-like", "bf16", 9, 0.7, RAGGED_SH),
    ("olmoe-like", "bf16", 3, 1.0, RAGGED_SH),  # k = 0: the residual as its own pass
])
def test_fused_residual_matches_separate(name, dtype, T, s, over):
    shape = S.LAYERS[name].with_(dtype=dtype, **over)
    say(f"[case] fused residual {name} {dtype} T={T} s={s} over={bool(over)}")
    L = DeviceLayer(LayerInputs(shape, seed=0))
    k = B.moe_keep_count(s, shape.d_ff)
    E, K = shape.n_experts, shape.top_k
    x = to_dev(S.tokens(shape, 50 + T, T))
    R = B.Routing.allocate(T, K, E)
    ws_r = torch.empty(B.moe_route_workspace_size(L.desc, T), dtype=torch.uint8, device="cuda")
    B.moe_route(L.desc, T, x, L.w_router, L.bias, R, ws_r)
    ws = torch.empty(max(1, B.moe_ffn_workspace_size(L.desc, T, k, B.MOE_PATH_SPARSE)),
                     dtype=torch.uint8, device="cuda")
    shared = L.desc_sh is not None
    if shared:
        k_sh = B.moe_keep_count(s, shape.d_ff_shared)
        ws_sh = torch.empty(max(1, B.moe_ffn_workspace_size(L.desc_sh, T, k_sh, B.MOE_PATH_SPARSE)),
                            dtype=torch.uint8, device="cuda")

    def layer(y, x_in, x_next=None):
        # routed (then shared) FFN; the last call fuses the residual if asked
        if not shared:
            if x_next is None:
                B.moe_expert_ffn_sparse(L.desc, T, k, x_in, *L.w, R, y, 0, None, ws)
            else:
                B.moe_expert_ffn_sparse_residual(L.desc, T, k, x_in, *L.w, R, y, x_in, x_next, 0,
                                                 None, ws)
            return
        B.moe_expert_ffn_sparse(L.desc, T, k, x_in, *L.w, R, y, 0, None, ws)
        if x_next is None:
            B.moe_expert_ffn_sparse(L.desc_sh, T, k_sh, x_in, *L.w_sh, None, y, 1, None, ws_sh)
        else:
            B.moe_expert_ffn_sparse_residual(L.desc_sh, T, k_sh, x_in, *L.w_sh, None, y, x_in,
                                             x_next, 1, None, ws_sh)

    y_sep = torch.empty((T, shape.hidden), dtype=torch.float32, device="cuda")
    x_sep = torch.empty_like(x)
    layer(y_sep, x)
    B.moe_residual_add(L.desc, T, x, y_sep, x_sep)
    y_fus = torch.full_like(y_sep, float("nan"))
    x_fus = torch.empty_like(x)
    layer(y_fus, x, x_fus)
    x_inp = x.clone()                                   # in place: x_next is the layer input
    y_inp = torch.full_like(y_sep, float("nan"))
    layer(y_inp, x_inp, x_inp)
    torch.cuda.synchronize()
    assert torch.isfinite(y_sep).all()
    assert torch.equal(y_fus, y_sep) and torch.equal(y_inp, y_sep)
    assert torch.equal(x_fus, x_sep) and torch.equal(x_inp, x_sep)
    if s < 1.0:
        assert not torch.equal(x_sep, x)


def test_fused_residual_decode_step_graph():
    # the two-layer step with the residual fused into each layer's FFN call,
    # captured as one graph: replays give the unfused eager chain's bits
    shape = S.LAYERS["olmoe-like"]
    T, k = 4, B.moe_keep_count(0.9, shape.d_ff)
    say("[case] two-layer decode step with fused residuals, graph vs eager")
    layers = [DeviceLayer(LayerInputs(shape, seed=s)) for s in (0, 1)]
    E, K = shape.n_experts, shape.top_k
    x0 = to_dev(S.tokens(shape, 41, T))
    xs = [torch.empty_like(x0) for _ in layers]
    ys = [torch.empty((T, shape.hidden), dtype=torch.float32, device="cuda") for _ in layers]
    rs = [B.Routing.allocate(T, K, E) for _ in layers]
    d = layers[0].desc
    ws_r = torch.empty(B.moe_route_workspace_size(d, T), dtype=torch.uint8, device="cuda")
    ws = torch.empty(B.moe_ffn_workspace_size(d, T, k, B.MOE_PATH_SPARSE), dtype=torch.uint8,
                     device="cuda")

    def step(fused):
        x = x0
        for L, xo, y, R in zip(layers, xs, ys, rs):
            B.moe_route(L.desc, T, x, L.w_router, L.bias, R, ws_r)
            if fused:
                B.moe_expert_ffn_sparse_residual(L.desc, T, k, x, *L.w, R, y, x, xo, 0, None, ws)
            else:
                B.moe_expert_ffn_sparse(L.desc, T, k, x, *L.w, R, y, 0, None, ws)
                B.moe_residual_add(L.desc, T, x, y, xo)
            x = xo

    step(False)
    torch.cuda.synchronize()
    ref = [t.clone() for t in xs + ys]
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(True)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(True)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in xs + ys:
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(xs + ys, ref):
            assert torch.equal(a, b), f"replay {rep} differs from the unfused eager step"
        step(False)                                          # eager work between replays
        torch.cuda.synchronize()
