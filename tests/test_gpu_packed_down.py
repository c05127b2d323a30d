"""GPU tests of the dense call with W_d packed by moe_pack_down.

The dense path's down GEMM can read W_d in the MFMA fragment layout (the
transposed 16-column x 32-row fragments the header describes), streaming the
weights as the gate/up GEMM does instead of staging them through LDS.  These
tests check the packing against a numpy statement of the layout, and the
dense call on the packed copy against the oracle and against the same call
on the row-major W_d (the same masks; sums in another order) on layers whose
hidden sizes take each column-block width (H = 5120 and 2048: 64 columns per
wave; 384: 32; 320: 16), ragged token items and K chunks, the unmasked
one-token case that the row-major call runs on its row kernel, and the
shared experts.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import moe_synth as S
from oracle import moe_oracle as O
from sparse_moe_expert_route_amd import binding as B

from parity import DeviceLayer, LayerInputs, compare_layer, pack_down_reference, rel_l2, to_dev

pytestmark = pytest.mark.gpu
DN = B.MOE_PATH_DENSE


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


@pytest.mark.parametrize("E,d,H", [(3, 64, 128), (2, 192, 320), (5, 1536, 5120)])
def test_pack_down_layout(E, d, H):
    rng = np.random.default_rng(1)
    host = S.round_to_bf16_bits(rng.standard_normal((E, d, H)).astype(np.float32))
    desc = B.make_desc(H, E, d, 1, False, "bf16", gate_up_layout="packed", down_layout="packed")
    w = to_dev(host)
    say(f"[case] pack_down E={E} d_ff={d} H={H}")
    pk = B.moe_pack_down(desc, w)
    back = B.moe_unpack_down(desc, pk)
    torch.cuda.synchronize()
    got = pk.view(torch.int16).cpu().numpy()
    np.testing.assert_array_equal(got, pack_down_reference(host.view(np.int16)))
    assert torch.equal(back.view(torch.int16), w.view(torch.int16))
    with pytest.raises(B.MoeError):
        B.moe_pack_down(desc, w, w)           # in place is refused


def _k(d_ff, s=0.9):
    return O.keep_count(s, d_ff)


# items of 32 / 64 / 128 tokens as routed experts hold <= 16 / <= 40 / more
# on average (always-on: T <= 32 / <= 64 / more); 4 / 2 / 1 column tiles
# per wave as H / 64 divides by 4 / 2 / 1
@pytest.mark.parametrize("name,T,over,tokens", [
    ("olmoe-like", 16, {}, None),                          # 2 per expert: 32-token items, 4 tiles
    ("qwen3-moe-like", 64, {}, None),                      # 4 per expert
    ("olmoe-like", 130, RAGGED, None),                     # 32 per expert: 64-token items, 1 tile
    ("olmoe-like", 300, RAGGED, None),                     # 75: 128-token items, 1 tile; 3 stages
    ("olmoe-like", 150, dict(RAGGED, hidden=384), None),   # 37: 64-token items, 2 tiles
    ("olmoe-like", 520, dict(RAGGED, hidden=384), None),   # 130: 128-token items, 2 tiles
    ("deepseek-v2-like", 32, {}, None),                    # d_ff 1536: K chunks, 2 shared experts
    ("olmoe-like", 256, {}, None),                         # 32 per expert: 64-token items, 4 tiles
    ("olmoe-like", 1024, {}, np.arange(0, 1024, 33)),      # 128 per expert: 128-token items
    ("llama4-like", 256, {}, np.arange(0, 256, 5)),        # 16 per expert, shared 2 full items
    ("llama4-like", 1024, {}, np.arange(3, 1024, 41)),     # 64 per expert; the MFMA-bound shared expert
])
def test_dense_packed_down_parity(name, T, over, tokens):
    inp, dev = _layer(name, **over)
    sh = inp.shape
    x = inp.tokens(T, 23)
    k = _k(sh.d_ff)
    k_sh = _k(sh.d_ff_shared) if sh.n_shared else None
    say(f"[case] dense packed-down {name} T={T} H={sh.hidden}")
    got = dev.run(x, k, DN, k_sh=k_sh, packed_down=True)
    err = compare_layer(inp, x, got, k, k_sh=k_sh, tokens=tokens)
    say(f"   rel_l2 vs oracle={err:.3e}")
    ref = dev.run(x, k, DN, k_sh=k_sh)
    np.testing.assert_array_equal(got["idx"], ref["idx"])   # the same masks
    d = rel_l2(got["y"], ref["y"])
    say(f"   rel_l2 vs row-major W_d={d:.3e}")
    assert d < 1e-5


@pytest.mark.parametrize("k", [1, 64, 191, 192])
def test_dense_packed_down_keep_extremes(k):
    # ragged layer (H = 320, d_ff = 192, shared d_ff 128): from one kept
    # neuron to all of them
    inp, dev = _layer("olmoe-like", **RAGGED)
    x = inp.tokens(130, 29)
    k_sh = min(k, 128)
    say(f"[case] dense packed-down ragged k={k}")
    got = dev.run(x, k, DN, k_sh=k_sh, packed_down=True)
    compare_layer(inp, x, got, k, k_sh=k_sh)


def test_dense_packed_down_unmasked_single_token():
    # k = d_ff at T = 1: the row-major call runs this on its row kernel, the
    # packed one on the GEMM (one token per item)
    inp, dev = _layer("olmoe-like")
    x = inp.tokens(1, 31)
    say("[case] dense packed-down T=1 k=d_ff")
    got = dev.run(x, 1024, DN, packed_down=True)
    compare_layer(inp, x, got, 1024)
    ref = dev.run(x, 1024, DN)
    assert rel_l2(got["y"], ref["y"]) < 1e-5


def test_dense_packed_down_deterministic():
    inp, dev = _layer("deepseek-v2-like")
    x = inp.tokens(24, 37)
    k = _k(1536)
    say("[case] dense packed-down reruns deepseek-v2-like T=24")
    a = dev.run(x, k, DN, k_sh=k, packed_down=True)
    b = dev.run(x, k, DN, k_sh=k, packed_down=True)
    np.testing.assert_array_equal(a["y"], b["y"])


def test_layer_class_pack_down():
    # MoELayer(pack_down=True): its dense calls read the packed copy and give
    # the same bits as the direct calls on it; the sparse calls are unchanged
    from sparse_moe_expert_route_amd.layer import MoELayer
    inp, dev = _layer("llama4-like")
    sh = inp.shape
    T = 256
    x_host = inp.tokens(T, 41)
    k = _k(sh.d_ff)
    m = MoELayer(hidden=sh.hidden, n_experts=sh.n_experts, d_ff=sh.d_ff, top_k=sh.top_k,
                 norm_topk=sh.norm_topk, dtype=sh.dtype, w_router=dev.w_router,
                 w_gate=dev.w[0], w_up=dev.w[1], w_down=dev.w[2], shared=dev.w_sh, packed=True,
                 pack_down=True)
    say("[case] MoELayer pack_down llama4-like T=256")
    x = to_dev(x_host)
    y = m.forward(x, k, k, path=DN, path_shared=DN)
    got = dev.run(x_host, k, DN, k_sh=k, packed_down=True)
    np.testing.assert_array_equal(y.cpu().numpy(), got["y"])
    ys = m.forward(x, k, k, path=B.MOE_PATH_SPARSE, path_shared=DN)
    want = dev.run(x_host, k, B.MOE_PATH_SPARSE, k_sh=k, path_sh=DN, packed_down=True)
    np.testing.assert_array_equal(ys.cpu().numpy(), want["y"])


NARROW = dict(n_experts=4, d_ff=128, top_k=2, norm_topk=False, n_shared=1, d_ff_shared=64,
              zipf_bias=None, dtype="bf16")


@pytest.mark.parametrize("H", [64, 192])
@pytest.mark.parametrize("T", [1, 20, 300])
def test_dense_packed_down_narrow(H, T):
    # one or three 64-column blocks (16 columns per wave), d_ff 128 and 64
    # (two and one 64-row stages), a single token to 150 per expert
    inp, dev = _layer("olmoe-like", **dict(NARROW, hidden=H))
    x = inp.tokens(T, 43)
    say(f"[case] dense packed-down narrow H={H} T={T}")
    got = dev.run(x, 13, DN, k_sh=40, packed_down=True)
    compare_layer(inp, x, got, 13, k_sh=40)
    ref = dev.run(x, 13, DN, k_sh=40)
    assert rel_l2(got["y"], ref["y"]) < 1e-5
