"""GPU tests of moe_layer_sparse: moe_route then moe_expert_ffn_sparse in one
call.  Up to 2 tokens the gate/up kernel repeats the router's selection (one
wave per token) and the select-and-group launch goes away; every output must
equal the two calls' bits (routing outputs, kept ids, y), also when captured
in a graph.  Larger batches run the two calls' kernels through the same
entry point."""
import numpy as np
import pytest
import torch

import moe_synth as S
from parity import DeviceLayer, LayerInputs, to_dev
from sparse_moe_expert_route_amd import binding as B

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


SHAPES = {
    "olmoe": ("olmoe-like", {}),                                     # E = 64: one logit per lane
    "qwen3": ("qwen3-moe-like", {}),                                 # E = 128, normalised, Zipf bias
    "e160": ("olmoe-like", dict(hidden=512, n_experts=160, d_ff=512, top_k=6)),  # 3 logits per lane
    "top1": ("olmoe-like", dict(hidden=512, n_experts=16, d_ff=1024, top_k=1)),
    "f32": ("tiny-f32", {}),
}


def _run(L, shape, T, k, fused, acc=0, y0=None):
    E, K = shape.n_experts, shape.top_k
    x = to_dev(S.tokens(shape, 70 + T, T))
    R = B.Routing.allocate(T, K, E)
    for t in (R.topk_ids, R.expert_offsets, R.pair_by_expert, R.active_experts, R.n_active):
        t.fill_(-7)
    R.topk_w.fill_(float("nan"))
    y = y0.clone() if y0 is not None else torch.full((T, shape.hidden), float("nan"), device="cuda")
    idx = torch.full((T * K, max(1, k)), -1, dtype=torch.int32, device="cuda")
    if fused:
        ws = torch.empty(B.moe_layer_workspace_size(L.desc, T, k), dtype=torch.uint8, device="cuda")
        B.moe_layer_sparse(L.desc, T, k, x, L.w_router, L.bias, *L.w, R, y, acc, idx, ws)
    else:
        ws_r = torch.empty(B.moe_route_workspace_size(L.desc, T), dtype=torch.uint8, device="cuda")
        ws = torch.empty(max(1, B.moe_ffn_workspace_size(L.desc, T, k, B.MOE_PATH_SPARSE)),
                         dtype=torch.uint8, device="cuda")
        B.moe_route(L.desc, T, x, L.w_router, L.bias, R, ws_r)
        B.moe_expert_ffn_sparse(L.desc, T, k, x, *L.w, R, y, acc, idx, ws)
    torch.cuda.synchronize()
    P = T * K
    na = int(R.n_active.cpu()[0])
    return dict(ids=R.topk_ids[:T].cpu(), w=R.topk_w[:T].cpu(), off=R.expert_offsets.cpu(),
                pairs=R.pair_by_expert[:P].cpu(), na=na, act=R.active_experts[:na].cpu(),
                idx=idx.cpu(), y=y.cpu())


@pytest.mark.parametrize("key", list(SHAPES))
@pytest.mark.parametrize("T,s", [(1, 0.9), (1, 0.5), (2, 0.9), (4, 0.9), (5, 0.9), (8, 0.9),
                                 (8, 0.0), (1, 0.0), (16, 0.9)])
def test_layer_matches_route_then_ffn(key, T, s):
    name, over = SHAPES[key]
    shape = S.LAYERS[name].with_(**over) if over else S.LAYERS[name]
    k = B.moe_keep_count(s, shape.d_ff)
    say(f"[case] layer {key} T={T} k={k}")
    L = DeviceLayer(LayerInputs(shape, seed=0))
    a = _run(L, shape, T, k, fused=False)
    b = _run(L, shape, T, k, fused=True)
    assert torch.isfinite(a["y"]).all()
    for f in ("ids", "w", "off", "pairs", "act", "idx", "y"):
        assert torch.equal(a[f], b[f]), f
    assert a["na"] == b["na"]
    # accumulate onto an existing y
    y0 = torch.randn((T, shape.hidden), device="cuda")
    a = _run(L, shape, T, k, fused=False, acc=1, y0=y0)
    b = _run(L, shape, T, k, fused=True, acc=1, y0=y0)
    assert torch.equal(a["y"], b["y"])


def test_layer_graph_replays():
    shape = S.LAYERS["olmoe-like"]
    T, k = 1, B.moe_keep_count(0.9, shape.d_ff)
    say("[case] layer graph T=1")
    L = DeviceLayer(LayerInputs(shape, seed=0))
    E, K = shape.n_experts, shape.top_k
    xs = [to_dev(S.tokens(shape, 90 + i, T)) for i in range(2)]
    R = B.Routing.allocate(T, K, E)
    y = torch.empty((T, shape.hidden), device="cuda")
    ws = torch.empty(B.moe_layer_workspace_size(L.desc, T, k), dtype=torch.uint8, device="cuda")
    refs = []
    for x in xs:
        B.moe_layer_sparse(L.desc, T, k, x, L.w_router, L.bias, *L.w, R, y, 0, None, ws)
        torch.cuda.synchronize()
        refs.append((y.clone(), R.topk_ids.clone()))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        B.moe_layer_sparse(L.desc, T, k, xs[0], L.w_router, L.bias, *L.w, R, y, 0, None, ws)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    xin = xs[0].clone()
    with torch.cuda.graph(g):
        B.moe_layer_sparse(L.desc, T, k, xin, L.w_router, L.bias, *L.w, R, y, 0, None, ws)
    torch.cuda.synchronize()
    for rep in range(4):
        i = rep % 2
        xin.copy_(xs[i])
        y.fill_(float("nan"))
        R.topk_ids.fill_(-1)
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, refs[i][0]) and torch.equal(R.topk_ids, refs[i][1]), rep
        B.moe_layer_sparse(L.desc, T, k, xs[1 - i], L.w_router, L.bias, *L.w, R, y, 0, None, ws)
        torch.cuda.synchronize()


@pytest.mark.parametrize("T", [1, 6, 16])
def test_layer_with_residual(T):
    # x_next = x + y in the down epilogue: equals route, FFN, then moe_residual_add
    shape = S.LAYERS["olmoe-like"]
    k = B.moe_keep_count(0.9, shape.d_ff)
    say(f"[case] layer + residual T={T}")
    L = DeviceLayer(LayerInputs(shape, seed=0))
    E, K = shape.n_experts, shape.top_k
    x = to_dev(S.tokens(shape, 95 + T, T))
    R = B.Routing.allocate(T, K, E)
    y = torch.empty((T, shape.hidden), device="cuda")
    ws_r = torch.empty(B.moe_route_workspace_size(L.desc, T), dtype=torch.uint8, device="cuda")
    ws_f = torch.empty(B.moe_ffn_workspace_size(L.desc, T, k, B.MOE_PATH_SPARSE), dtype=torch.uint8,
                       device="cuda")
    B.moe_route(L.desc, T, x, L.w_router, L.bias, R, ws_r)
    B.moe_expert_ffn_sparse(L.desc, T, k, x, *L.w, R, y, 0, None, ws_f)
    x_ref = torch.empty_like(x)
    B.moe_residual_add(L.desc, T, x, y, x_ref)
    torch.cuda.synchronize()
    y_ref = y.clone()
    ws = torch.empty(B.moe_layer_workspace_size(L.desc, T, k), dtype=torch.uint8, device="cuda")
    x_in = x.clone()                          # in place: the next input overwrites this one
    y.fill_(float("nan"))
    B.moe_layer_sparse(L.desc, T, k, x_in, L.w_router, L.bias, *L.w, R, y, 0, None, ws,
                       x_res=x_in, x_next=x_in)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(x_in, x_ref)
