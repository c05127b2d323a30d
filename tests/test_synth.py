"""The seeded input generator: determinism, per-expert streams, distributions, bf16 rounding."""
import numpy as np
import torch

import moe_synth as S


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 10,
                        np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 0.0, -0.0], np.float32)])
    want = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(S.round_to_bf16_bits(a), want)


def test_expert_streams_are_independent_of_order_and_threads():
    sh = S.LAYERS["olmoe-like"].with_(hidden=128, d_ff=64, n_experts=6)
    g1, u1, d1 = S.expert_weights(sh, seed=0, threads=1)
    g2, u2, d2 = S.expert_weights(sh, seed=0, experts=[5, 3], threads=4)
    np.testing.assert_array_equal(g1[5], g2[0])
    np.testing.assert_array_equal(d1[3], d2[1])
    np.testing.assert_array_equal(S.LazyExperts(sh, 0, "up")[4], u1[4])
    assert not np.array_equal(g1[0], g1[1]) and not np.array_equal(g1[0], u1[0])
    g3, _, _ = S.expert_weights(sh, seed=1, experts=[0], threads=1)
    assert not np.array_equal(g3[0], g1[0])


def test_distributions():
    sh = S.LAYERS["tiny-f32"]
    g, u, d = S.expert_weights(sh, seed=0)
    assert g.dtype == np.float32 and g.shape == (8, 512, 256)
    np.testing.assert_allclose(g.std(), 1 / np.sqrt(256), rtol=0.01)
    np.testing.assert_allclose(d.std(), 1 / np.sqrt(512), rtol=0.01)
    np.testing.assert_allclose(S.router_matrix(sh).std(), 1 / np.sqrt(256), rtol=0.05)
    x = S.tokens(sh, 0, 4)
    assert x.shape == (4, 256) and abs(x.std() - 1) < 0.1
    assert S.router_bias(sh) is None
    q = S.LAYERS["qwen3-moe-like"]
    b = S.router_bias(q)
    assert b[0] == 0 and np.all(np.diff(b) < 0)
    np.testing.assert_allclose(np.exp(b[:4]), [1, 2 ** -1.1, 3 ** -1.1, 4 ** -1.1], rtol=1e-6)
    xb = S.tokens(S.LAYERS["olmoe-like"], 3, 2)
    assert xb.dtype == np.uint16 and xb.shape == (2, 2048)
