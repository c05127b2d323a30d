"""GPU tests of the exact selects' kept lists.

The selects inside the down kernels write each kept list to LDS without a
branch per value (a dropped value goes to a spare slot) unless the caller
also asked for the kept ids (active_idx_out), which keeps the per-value
branches.  So every case here runs twice, with and without the ids, and
the outputs must agree bit for bit; the run with ids is compared with the
oracle.  Cases: the one-wave select of the down kernel at 1-8 tokens (1-3
at d_ff 1536, also 17-32 at d_ff 768), the fused FFN's down units at 9-16
tokens (12 and 16 activations per lane), the mask kernel's eight-wave
select (one routed
slot per token over experts of d_ff 8192, a shared expert of d_ff 4096:
1-4 tokens, keep fractions 0.5 and 0.01), and an all-zero token there,
whose kept lists must be the lowest indices.
"""
import functools
import sys

import numpy as np
import pytest

import moe_synth as S
from oracle import moe_oracle as O
from sparse_moe_expert_route_amd import binding as B

from parity import DeviceLayer, LayerInputs, compare_layer

pytestmark = pytest.mark.gpu
SP = B.MOE_PATH_SPARSE

# one routed slot per token over experts of d_ff 8192, a shared expert of
# d_ff 4096 (the eight-wave mask select)
WIDE = dict(hidden=256, n_experts=4, d_ff=8192, top_k=1, norm_topk=False, n_shared=1,
             d_ff_shared=4096, zipf_bias=None)


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=2)
def _layer_cached(name, over):
    over = dict(over)
    shape = S.LAYERS[name].with_(**over) if over else S.LAYERS[name]
    inp = LayerInputs(shape, seed=0)
    return inp, DeviceLayer(inp)


def _layer(name, **over):
    return _layer_cached(name, tuple(sorted(over.items())))


def _both(inp, dev, x, s=0.9):
    sh = inp.shape
    k = O.keep_count(s, sh.d_ff)
    k_sh = O.keep_count(s, sh.d_ff_shared) if sh.n_shared else None
    got = dev.run(x, k, SP, k_sh=k_sh, path_sh=SP)
    plain = dev.run(x, k, SP, k_sh=k_sh, path_sh=SP, want_idx=False)
    np.testing.assert_array_equal(plain["y"], got["y"], err_msg="outputs differ without kept ids")
    return got, k, k_sh


@pytest.mark.parametrize("name,T", [("olmoe-like", 1), ("olmoe-like", 3), ("olmoe-like", 4),
                                    ("olmoe-like", 8), ("olmoe-like", 16),
                                    ("qwen3-moe-like", 16), ("deepseek-v2-like", 8)])
def test_outputs_without_kept_ids(name, T):
    inp, dev = _layer(name)
    x = inp.tokens(T, 17)
    say(f"[case] kept lists with and without ids {name} T={T}")
    got, k, k_sh = _both(inp, dev, x)
    err = compare_layer(inp, x, got, k, k_sh=k_sh)
    say(f"   rel_l2={err:.3e}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 2, 3, 4])
def test_wide_select(dtype, T):
    inp, dev = _layer("olmoe-like", dtype=dtype, **WIDE)
    x = inp.tokens(T, 19)
    say(f"[case] wide select {dtype} T={T}")
    got, k, k_sh = _both(inp, dev, x)
    err = compare_layer(inp, x, got, k, k_sh=k_sh)
    say(f"   rel_l2={err:.3e}")


@pytest.mark.parametrize("s", [0.5, 0.99])
def test_wide_select_keep_counts(s):
    inp, dev = _layer("olmoe-like", dtype="bf16", **WIDE)
    x = inp.tokens(2, 23)
    say(f"[case] wide select bf16 T=2 s={s}")
    got, k, k_sh = _both(inp, dev, x, s=s)
    compare_layer(inp, x, got, k, k_sh=k_sh)


def test_wide_select_zero_token():
    # an all-zero token: every logit is 0 (the lowest expert id wins), every
    # h is 0, so the kept lists are the lowest indices and the output row is 0
    inp, dev = _layer("olmoe-like", dtype="bf16", **WIDE)
    x = inp.tokens(3, 29)
    x[1] = 0
    say("[case] wide select zero token")
    got, k, k_sh = _both(inp, dev, x)
    assert got["ids"][1, 0] == 0
    np.testing.assert_array_equal(got["idx"][1, :k], np.arange(k))
    np.testing.assert_array_equal(got["idx_sh"][1, :k_sh], np.arange(k_sh))
    assert np.all(got["y"][1] == 0)
    compare_layer(inp, x, got, k, k_sh=k_sh)
