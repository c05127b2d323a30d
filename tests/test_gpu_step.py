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
    desc = B.make_desc(shape.hidden, shape.n_experts, shape.d_ff, shape.top_k, False, dtype)
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
