"""GPU tests of the sparse path's packed-rows down projection.

When the experts of a bf16 sparse call hold many tokens each (on average,
P / min(E, P) routed or T for a shared group, at least 8, 32 or 128 as the
active experts' W_d is >= 512 MB, >= 128 MB or smaller), the down
projection gathers each active expert's union of kept W_d rows once and
multiplies it with all of that expert's tokens (the page's fused
projection over the active neurons), instead of streaming every token's
kept rows on its own.
These tests check which calls take that form (and, beside it, which take
the fused FFN launch: 9-16 tokens at d_ff up to 1024), its parity with the
oracle at
the edges of the union (k = 1, union sizes on and off the 64-row stage,
k = d_ff), that rows outside an expert's union are never read, and its
residual epilogue.  The workload parity tests (test_gpu_parity.py) cover it
at full size on every family whose batches reach it.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import moe_synth as S
from oracle import moe_oracle as O
from sparse_moe_expert_route_amd import binding as B

from parity import DeviceLayer, LayerInputs, compare_layer, to_dev

pytestmark = pytest.mark.gpu
SP = B.MOE_PATH_SPARSE


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


RAGGED = dict(hidden=320, n_experts=12, d_ff=192, top_k=3, norm_topk=True, n_shared=1,
              d_ff_shared=128, zipf_bias=None, dtype="bf16")


@functools.lru_cache(maxsize=1)
def _layer_cached(name, over):
    over = dict(over)
    shape = S.LAYERS[name].with_(**over) if over else S.LAYERS[name]
    inp = LayerInputs(shape, seed=0)
    return inp, DeviceLayer(inp)


def _layer(name, **over):
    return _layer_cached(name, tuple(sorted(over.items())))


def _stages_of_ffn(dev, T, k, x_host, routed=True):
    """Stage names the library launches for one sparse FFN call."""
    sh = dev.inp.shape
    x = to_dev(x_host)
    desc = dev.desc if routed else dev.desc_sh
    R = None
    if routed:
        R = B.Routing.allocate(T, sh.top_k, sh.n_experts)
        ws_r = torch.empty(B.moe_route_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
        B.moe_route(desc, T, x, dev.w_router, dev.bias, R, ws_r)
    w = dev.w if routed else dev.w_sh
    y = torch.zeros((T, sh.hidden), device="cuda")
    ws = torch.empty(B.moe_ffn_workspace_size(desc, T, k, SP), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    tm = B.StageTimer(64)
    try:
        with tm:
            B.moe_expert_ffn_sparse(desc, T, k, x, *w, R, y, 1, None, ws)
        names = list(tm.durations())
    finally:
        tm.close()
    return names


@pytest.mark.parametrize("name,T,routed,want", [
    ("olmoe-like", 16, True, False),      # 2 per expert: the fused launch
    ("olmoe-like", 128, True, False),     # 16 per expert, W = 268 MB: needs 32
    ("olmoe-like", 256, True, True),      # 32 per expert
    ("qwen3-moe-like", 256, True, False),  # 16 per expert, W = 403 MB
    ("qwen3-moe-like", 512, True, True),  # 32 per expert
    ("llama4-like", 64, True, False),     # 4 per expert, W = 1.3 GB: needs 8
    ("llama4-like", 128, True, True),     # 8 per expert
    ("llama4-like", 64, False, False),    # a lone 84 MB shared expert: needs 128
    ("llama4-like", 128, False, True),
    ("deepseek-v2-like", 8, False, False),
])
def test_union_taken_where_expected(name, T, routed, want):
    inp, dev = _layer(name)
    sh = inp.shape
    d_ff = sh.d_ff if routed else sh.d_ff_shared
    k = O.keep_count(0.9, d_ff)
    say(f"[case] stages {name} T={T} routed={routed}")
    names = _stages_of_ffn(dev, T, k, inp.tokens(T, 5), routed)
    assert ("down_union" in names) == want, names
    assert ("union_rows" in names) == want, names
    if want:
        assert "down_rows" not in names and "fused_ffn" not in names, names


@pytest.mark.parametrize("name,T,want", [
    ("olmoe-like", 8, False),         # below the fused launch's batches
    ("olmoe-like", 9, True),
    ("olmoe-like", 16, True),
    ("qwen3-moe-like", 9, True),      # d_ff 768
    ("deepseek-v2-like", 8, False),   # d_ff 1536: the separate kernels
    ("deepseek-v2-like", 16, False),
])
def test_fused_launch_taken_where_expected(name, T, want):
    inp, dev = _layer(name)
    k = O.keep_count(0.9, inp.shape.d_ff)
    say(f"[case] fused launch {name} T={T}")
    names = _stages_of_ffn(dev, T, k, inp.tokens(T, 5), True)
    assert ("fused_ffn" in names) == want, names


@pytest.mark.parametrize("k", [1, 5, 63, 64, 65, 128, 191, 192])
def test_union_keep_extremes_ragged(k):
    # H = 320 (5 column blocks), d_ff = 192 (3 row stages), 12 small experts
    # of 520 * 3 / 12 = 130 tokens each (past the 128-token GEMM item): union
    # counts from a few rows to all 192, on and off the 64-row stage; shared
    # group of d_ff 128
    inp, dev = _layer("olmoe-like", **RAGGED)
    x = inp.tokens(520, 3)
    k_sh = min(k, 128)
    say(f"[case] union ragged bf16 k={k} k_sh={k_sh}")
    got = dev.run(x, k, SP, k_sh=k_sh, path_sh=SP)
    err = compare_layer(inp, x, got, k, k_sh=k_sh)
    say(f"   rel_l2={err:.3e}")


def test_union_single_expert_all_tokens():
    # one routed expert takes every pair: one union over all 130 tokens
    # (past the GEMM's 128-token item), k = 40 of d_ff 192
    inp, dev = _layer("olmoe-like", **dict(RAGGED, n_experts=1, top_k=1))
    x = inp.tokens(130, 4)
    say("[case] union one expert, 130 tokens")
    got = dev.run(x, 40, SP, k_sh=100, path_sh=SP)
    compare_layer(inp, x, got, 40, k_sh=100)


@pytest.mark.parametrize("name,T", [("olmoe-like", 256), ("llama4-like", 128)])
def test_union_reads_only_union_rows(name, T):
    # NaN in every W_d row that no token of its expert keeps: the same bits
    # (a row outside the union loaded and multiplied by zero would give NaN)
    inp, dev = _layer(name)
    sh = inp.shape
    x = inp.tokens(T, 11)
    k = O.keep_count(0.9, sh.d_ff)
    say(f"[case] union NaN-poisoned rows {name} T={T}")
    a = dev.run(x, k, SP)
    b = dev.run(x, k, SP)
    np.testing.assert_array_equal(a["y"], b["y"])        # reruns: the same bits
    keep = np.zeros((sh.n_experts, sh.d_ff), dtype=bool)
    for p, e in enumerate(a["ids"].reshape(-1)):
        keep[e, a["idx"][p, :k]] = True
    assert keep.sum(axis=1).max() < sh.d_ff              # some rows are outside every union
    wd = dev.w[2].clone()
    wd[torch.from_numpy(~keep).cuda()] = float("nan")
    c = dev.run(x, k, SP, poison_rows=wd)
    assert np.all(np.isfinite(c["y"]))
    np.testing.assert_array_equal(a["y"], c["y"])


def test_union_layer_residual_in_place():
    # x_next = x + y (rounded to bf16) written by the combine, in place over
    # the layer input; equals route, FFN, then moe_residual_add
    shape = S.LAYERS["olmoe-like"]
    T, k = 256, B.moe_keep_count(0.9, shape.d_ff)
    say(f"[case] union layer + residual T={T}")
    L = DeviceLayer(LayerInputs(shape, seed=0))
    x = to_dev(S.tokens(shape, 131, T))
    R = B.Routing.allocate(T, shape.top_k, shape.n_experts)
    y = torch.empty((T, shape.hidden), device="cuda")
    ws_r = torch.empty(B.moe_route_workspace_size(L.desc, T), dtype=torch.uint8, device="cuda")
    ws_f = torch.empty(B.moe_ffn_workspace_size(L.desc, T, k, SP), dtype=torch.uint8, device="cuda")
    B.moe_route(L.desc, T, x, L.w_router, L.bias, R, ws_r)
    B.moe_expert_ffn_sparse(L.desc, T, k, x, *L.w, R, y, 0, None, ws_f)
    x_ref = torch.empty_like(x)
    B.moe_residual_add(L.desc, T, x, y, x_ref)
    torch.cuda.synchronize()
    y_ref = y.clone()
    ws = torch.empty(B.moe_layer_workspace_size(L.desc, T, k), dtype=torch.uint8, device="cuda")
    x_in = x.clone()
    y.fill_(float("nan"))
    B.moe_layer_sparse(L.desc, T, k, x_in, L.w_router, L.bias, *L.w, R, y, 0, None, ws,
                       x_res=x_in, x_next=x_in)
    torch.cuda.synchronize()
    assert torch.equal(y, y_ref) and torch.equal(x_in, x_ref)


@pytest.mark.parametrize("name,T,over", [
    ("olmoe-like", 100, RAGGED),          # 25 tokens per expert: four token tiles per item
    ("olmoe-like", 256, {}),              # 32 per expert, H = 2048 (8 column blocks)
    ("llama4-like", 128, {}),             # 8 per expert, d_ff 8192, H = 5120
    ("llama4-like", 256, {}),             # 16 per expert
])
@pytest.mark.parametrize("path", [SP, B.MOE_PATH_DENSE])
def test_skinny_items_both_paths(name, T, over, path):
    # the few-tokens-per-expert down GEMM (one or two 16-token tiles per
    # item), over the union on the sparse path and all rows on the dense one
    inp, dev = _layer(name, **over)
    sh = inp.shape
    x = inp.tokens(T, 13)
    k = O.keep_count(0.9, sh.d_ff)
    k_sh = O.keep_count(0.9, sh.d_ff_shared) if sh.n_shared else None
    say(f"[case] skinny {name} T={T} path={path}")
    got = dev.run(x, k, path, k_sh=k_sh, path_sh=path)
    err = compare_layer(inp, x, got, k, k_sh=k_sh)
    say(f"   rel_l2={err:.3e}")


NARROW = dict(n_experts=4, d_ff=128, top_k=2, norm_topk=False, n_shared=1, d_ff_shared=64,
              zipf_bias=None, dtype="bf16")


@pytest.mark.parametrize("H", [64, 192])
@pytest.mark.parametrize("T,path", [(20, B.MOE_PATH_DENSE), (300, B.MOE_PATH_DENSE), (300, SP)])
def test_narrow_hidden_column_blocks(H, T, path):
    # H = 64 and 192: the skinny GEMM's 256-column and the wide GEMM's
    # 128-column blocks end past H (the columns past it read a stand-in and
    # are never stored); d_ff = 128 and 64 (shared): one or two 64-row
    # stages.  T = 20: 10 tokens per expert (skinny); T = 300: 150 (wide, and
    # the packed-rows form on the sparse path)
    inp, dev = _layer("olmoe-like", **dict(NARROW, hidden=H))
    x = inp.tokens(T, 17)
    k, k_sh = 13, 40
    say(f"[case] narrow H={H} T={T} path={path}")
    got = dev.run(x, k, path, k_sh=k_sh, path_sh=path)
    err = compare_layer(inp, x, got, k, k_sh=k_sh)
    say(f"   rel_l2={err:.3e}")


def test_union_at_max_tokens():
    # the ABI's largest token count on a small bf16 layer: 65536 * 3 pairs on
    # 12 experts take the packed-rows form (16384 tokens each, 128 token
    # items, 8192 groups of 8 pairs per expert, 196608 coefficient rows)
    inp, dev = _layer("olmoe-like", **RAGGED)
    x = inp.tokens(65536, 19)
    k = O.keep_count(0.7, 192)
    say("[case] union T=65536")
    got = dev.run(x, k, SP, k_sh=64, path_sh=SP)
    err = compare_layer(inp, x, got, k, k_sh=64)
    say(f"   rel_l2={err:.3e}")
