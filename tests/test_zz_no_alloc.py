"""moe_layer_sparse_noalloc: the layer entry point that allocates nothing.

Its workspace is the library's static per-device scratch.  Through the C
ABI it must give moe_layer_sparse's outputs bit for bit (the same kernels)
on two calls in a row, the second with fewer tokens (the scratch keeps the
first call's contents), and refuse a call whose workspace would not fit.
"""
import numpy as np
import pytest
import torch

import moe_synth as S
from oracle import moe_oracle as O
from sparse_moe_expert_route_amd import binding as B

from parity import DeviceLayer, LayerInputs, to_dev

pytestmark = pytest.mark.gpu


def _outputs(R, y, idx, T):
    torch.cuda.synchronize()
    return dict(ids=R.topk_ids[:T].cpu().numpy(), w=R.topk_w[:T].cpu().numpy(),
                off=R.expert_offsets.cpu().numpy(), pairs=R.pair_by_expert.cpu().numpy(),
                na=int(R.n_active.cpu()[0]), idx=idx.cpu().numpy(), y=y.cpu().numpy())


def _call(dev, x, k, noalloc):
    sh = dev.inp.shape
    T = x.shape[0]
    R = B.Routing.allocate(T, sh.top_k, sh.n_experts)
    y = torch.full((T, sh.hidden), float("nan"), device="cuda")
    idx = torch.full((T * sh.top_k, k), -1, dtype=torch.int32, device="cuda")
    if noalloc:
        B.moe_layer_sparse_noalloc(dev.desc, T, k, x, dev.w_router, dev.bias, *dev.w, R, y, 0, idx)
    else:
        ws = torch.empty(B.moe_layer_workspace_size(dev.desc, T, k), dtype=torch.uint8,
                         device="cuda")
        B.moe_layer_sparse(dev.desc, T, k, x, dev.w_router, dev.bias, *dev.w, R, y, 0, idx, ws)
    out = _outputs(R, y, idx, T)
    na = out["na"]
    return out, na


@pytest.mark.parametrize("name,Ts", [("olmoe-like", (16, 4)), ("qwen3-moe-like", (8, 1)),
                                     ("tiny-f32", (40, 3))])
def test_noalloc_matches_layer_entry_on_two_calls(name, Ts):
    inp = LayerInputs(S.LAYERS[name], seed=0)
    dev = DeviceLayer(inp)
    k = O.keep_count(0.9, inp.shape.d_ff)
    for i, T in enumerate(Ts):                       # the second call is smaller
        x = to_dev(inp.tokens(T, 60 + i))
        want, _ = _call(dev, x, k, noalloc=False)
        got, _ = _call(dev, x, k, noalloc=True)
        for key in ("ids", "off", "idx"):
            np.testing.assert_array_equal(got[key], want[key], err_msg=f"{name} T={T} {key}")
        P = T * inp.shape.top_k
        np.testing.assert_array_equal(got["pairs"][:P], want["pairs"][:P])
        assert got["na"] == want["na"]
        np.testing.assert_array_equal(got["w"], want["w"])
        np.testing.assert_array_equal(got["y"], want["y"], err_msg=f"{name} T={T} y")
        assert np.all(np.isfinite(got["y"]))


def test_noalloc_refuses_a_call_larger_than_its_scratch():
    inp = LayerInputs(S.LAYERS["tiny-f32"], seed=0)
    dev = DeviceLayer(inp)
    k = O.keep_count(0.9, inp.shape.d_ff)
    T = 8192                                         # 16384 pairs x 512 x 4 B of h alone: 32 MB
    assert B.moe_layer_workspace_size(dev.desc, T, k) > B.NOALLOC_SCRATCH_BYTES
    x = to_dev(inp.tokens(T, 64))
    R = B.Routing.allocate(T, inp.shape.top_k, inp.shape.n_experts)
    y = torch.full((T, inp.shape.hidden), 3.0, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.moe_layer_sparse_noalloc(dev.desc, T, k, x, dev.w_router, dev.bias, *dev.w, R, y)
    assert ei.value.status == 3 and "static scratch" in ei.value.detail
    torch.cuda.synchronize()
    assert torch.all(y == 3.0)                       # nothing was enqueued
