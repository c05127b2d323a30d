"""GPU parity of the HIP layer against the CPU oracle, through the C ABI.

Every layer workload is run at its own shapes (full size), on both paths,
plus ragged shapes that leave partial tiles everywhere and the edge cases
of the method (k = 0, k = d_ff, T = 0, one token, all experts selected,
skewed routing).  Every token row is compared with the oracle: its routing
ids, its kept-neuron lists and its output row.  Selection and output
comparison follow tests/parity.py; exact ties are covered in
tests/test_gpu_ties.py.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import moe_synth as S
from oracle import moe_oracle as O
from sparse_moe_expert_route_amd import binding as B

from parity import (DeviceLayer, LayerInputs, check_grouping, check_routing, compare_layer,
                    compare_threshold_layer, pack_reference, rel_l2, to_dev)

pytestmark = pytest.mark.gpu
SP, DN = B.MOE_PATH_SPARSE, B.MOE_PATH_DENSE


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


@functools.lru_cache(maxsize=2)
def _inputs(name: str, **over):
    shape = S.LAYERS[name].with_(**over) if over else S.LAYERS[name]
    return LayerInputs(shape, seed=0)


@functools.lru_cache(maxsize=2)
def layer(name: str, score: str = "swiglu", **over):
    inp = _inputs(name, **over)
    return inp, DeviceLayer(inp, score)


def run_case(name, T, s, path, s_sh=None, path_sh=None, seed=1, score="swiglu", **over):
    inp, dev = layer(name, score, **over)
    sh = inp.shape
    k = O.keep_count(s, sh.d_ff)
    k_sh = O.keep_count(s_sh, sh.d_ff_shared) if (sh.n_shared and s_sh is not None) else None
    x = inp.tokens(T, seed)
    say(f"[case] {sh.name} T={T} s={s} k={k} path={path} s_sh={s_sh} score={score} over={over}")
    got = dev.run(x, k, path, k_sh, path_sh)
    check_grouping(got, sh.n_experts, sh.top_k)
    err = compare_layer(inp, x, got, k, k_sh, score=score)
    say(f"   rel_l2={err:.3e}")
    return got


# ------------------------------------------------------------------ the workloads

@pytest.mark.parametrize("path", [SP, DN])
@pytest.mark.parametrize("s", [0.9, 0.0, 0.5])
def test_tiny_f32_layer(s, path):
    run_case("tiny-f32", 4, s, path)


@pytest.mark.parametrize("T", [1, 4, 16])
@pytest.mark.parametrize("s", [0.9, 0.75, 0.5, 0.0])
def test_olmoe_like_sparse(T, s):
    run_case("olmoe-like", T, s, SP)


@pytest.mark.parametrize("name,T", [("olmoe-like", 8), ("olmoe-like", 9),
                                    ("qwen3-moe-like", 8), ("qwen3-moe-like", 9),
                                    ("qwen3-moe-like", 17), ("qwen3-moe-like", 33),
                                    ("deepseek-v2-like", 3), ("deepseek-v2-like", 4)])
def test_dispatch_boundaries(name, T):
    # the last batch that selects inside the down kernel and the first on
    # the fused FFN launch (d_ff up to 1024), or on the mask and down
    # kernels (d_ff 1536); past 16 tokens at d_ff 768 the down kernel
    # selects again, up to 32
    run_case(name, T, 0.9, SP)


@pytest.mark.parametrize("T", [1, 16])
def test_olmoe_like_dense(T):
    run_case("olmoe-like", T, 0.9, DN)


@pytest.mark.parametrize("T", [1, 2, 16])
def test_olmoe_like_dense_unmasked(T):
    # k = d_ff on the dense path: a token's 8 x 1024 rows exceed one row
    # stage, so every batch takes the grouped GEMM
    run_case("olmoe-like", T, 0.0, DN)


@pytest.mark.parametrize("T", [1, 2, 3])
def test_dense_unmasked_rows(T):
    # k = d_ff on the dense path with a token's rows within one stage (4 x 512)
    # and about one token per expert: every row streamed per pair, weights
    # applied while staging (T = 3 on 64 experts is still under 2 per expert)
    run_case("olmoe-like", T, 0.0, DN, top_k=4, d_ff=512)


@pytest.mark.parametrize("T", [1, 2, 8])
def test_deepseek_v2_like_shared_dense_unmasked(T):
    # the always-on experts at sparsity 0 on the dense path: rows per pair at
    # T <= 2 tokens per expert, the grouped GEMM at T = 8
    run_case("deepseek-v2-like", T, 0.9, SP, s_sh=0.0, path_sh=DN)


@pytest.mark.parametrize("T,path", [(1, SP), (4, SP), (16, SP), (32, SP), (64, SP), (64, DN)])
def test_qwen3_like_zipf(T, path):
    got = run_case("qwen3-moe-like", T, 0.9, path)
    if T == 64:   # the Zipf bias concentrates load on the lowest expert ids
        counts = np.diff(got["offsets"])
        assert counts[0] == counts.max() and counts[0] > 2 * T * 8 / 128


@pytest.mark.parametrize("T,s_sh", [(1, 0.0), (1, 0.5), (8, 0.0), (32, 0.5)])
def test_deepseek_v2_like(T, s_sh):
    run_case("deepseek-v2-like", T, 0.9, SP, s_sh=s_sh, path_sh=SP)


def test_deepseek_v2_like_dense():
    run_case("deepseek-v2-like", 32, 0.9, DN, s_sh=0.5, path_sh=DN)


@pytest.mark.parametrize("path", [SP, DN])
def test_deepseek_v2_like_large_batch(path):
    # 256 tokens: the two shared experts' gate/up on the grouped GEMM with
    # its weight ring (96 blocks), routed experts at ~10 tokens each
    run_case("deepseek-v2-like", 256, 0.9, path, s_sh=0.5, path_sh=DN)


@pytest.mark.parametrize("T", [1, 8, 64, 256, 1024])
@pytest.mark.parametrize("path", [SP, DN])
def test_llama4_like(T, path):
    run_case("llama4-like", T, 0.9, path, s_sh=0.9, path_sh=path)


# ------------------------------------------------------------------ the page's own split

UPDOWN = [("tiny-f32", 4, 0.9, None), ("tiny-f32", 4, 0.0, None), ("olmoe-like", 1, 0.9, None),
          ("olmoe-like", 4, 0.9, None), ("olmoe-like", 16, 0.9, None), ("olmoe-like", 16, 0.5, None),
          ("qwen3-moe-like", 4, 0.9, None), ("qwen3-moe-like", 32, 0.9, None),
          ("deepseek-v2-like", 1, 0.9, 0.5), ("deepseek-v2-like", 8, 0.9, 0.0),
          ("llama4-like", 1, 0.9, 0.9), ("llama4-like", 64, 0.9, 0.9),
          ("llama4-like", 256, 0.9, 0.9)]   # shared gate scores on the GEMM's weight ring


@pytest.mark.parametrize("name,T,s,s_sh", UPDOWN)
def test_updown_split(name, T, s, s_sh):
    # scores from the dense gate alone; up and down gathered on kept rows
    run_case(name, T, s, SP, s_sh=s_sh, path_sh=SP, score="gate")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 17, 37])
def test_updown_ragged(dtype, T):
    run_case("olmoe-like", T, 0.7, SP, s_sh=0.5, path_sh=SP, score="gate", dtype=dtype, **RAGGED)


def test_updown_reads_only_kept_up_and_down_rows_and_is_reproducible():
    # NaN in every W_u and W_d row no pair keeps: same bits
    inp, dev = layer("olmoe-like", "gate")
    x = inp.tokens(4, 7)
    k = O.keep_count(0.9, 1024)
    say("[case] updown NaN-poisoned unkept W_u / W_d rows")
    a = dev.run(x, k, SP)
    b = dev.run(x, k, SP)
    np.testing.assert_array_equal(a["y"], b["y"])
    keep = np.zeros((64, 1024), dtype=bool)
    for p, e in enumerate(a["ids"].reshape(-1)):
        keep[e, a["idx"][p, :k]] = True
    poison = torch.from_numpy(~keep).cuda()
    wu, wd = dev.w[1].clone(), dev.w[2].clone()
    wu[poison] = float("nan")
    wd[poison] = float("nan")
    c = dev.run(x, k, SP, poison_rows=wd, poison_up=wu)
    assert np.all(np.isfinite(c["y"]))
    np.testing.assert_array_equal(a["y"], c["y"])


# ------------------------------------------------------------------ threshold masking

# batches up to 16 run the compare inside the down kernel, larger ones the
# separate mask kernel
THRESH = [("tiny-f32", 8, 4, 0.9), ("olmoe-like", 32, 16, 0.9), ("olmoe-like", 32, 4, 0.5),
          ("qwen3-moe-like", 64, 8, 0.9), ("deepseek-v2-like", 8, 4, 0.9),
          ("llama4-like", 4, 2, 0.9), ("olmoe-like", 32, 33, 0.7), ("qwen3-moe-like", 64, 40, 0.9),
          ("tiny-f32", 8, 24, 0.5)]


@pytest.mark.parametrize("name,T_cal,T,s", THRESH)
def test_threshold_calibration_and_masking(name, T_cal, T, s):
    inp, dev = layer(name)
    sh = inp.shape
    x_cal = inp.tokens(T_cal, 21)
    say(f"[case] threshold {name} T_cal={T_cal} T={T} s={s}")
    tau = dev.calibrate(x_cal, s)
    tau_sh = dev.calibrate(x_cal, s, shared=True) if sh.n_shared else None
    ids_cal = dev.route_ids(x_cal)
    check_routing(inp, x_cal, ids_cal)
    t_or, t_or_sh = O.calibrate_thresholds(x_cal, inp.w_router, inp.bias, inp.wg, inp.wu,
                                           top_k=sh.top_k, norm_topk=sh.norm_topk,
                                           dtype=sh.dtype, sparsity=s, shared=inp.shared,
                                           forced_ids=ids_cal)
    # order statistics move by at most the scores' own rounding
    np.testing.assert_allclose(tau, t_or, rtol=1e-4, atol=1e-7)
    if tau_sh is not None:
        np.testing.assert_allclose(tau_sh, t_or_sh, rtol=1e-4, atol=1e-7)
    x = inp.tokens(T, 22)
    got = dev.run_threshold(x, torch.from_numpy(tau).cuda(),
                            torch.from_numpy(tau_sh).cuda() if tau_sh is not None else None)
    err = compare_threshold_layer(inp, x, got, tau, tau_sh)
    say(f"   rel_l2={err:.3e} mean kept {got['cnt'].mean():.1f}")


# the page's own pipeline: dense gate scores, threshold mask, sparse up + down
THRESH_SPLIT = [("tiny-f32", 8, 4, 0.9), ("olmoe-like", 32, 16, 0.9), ("olmoe-like", 32, 1, 0.5),
                ("olmoe-like", 32, 33, 0.7), ("qwen3-moe-like", 64, 8, 0.9),
                ("deepseek-v2-like", 8, 4, 0.9), ("llama4-like", 4, 2, 0.9)]


@pytest.mark.parametrize("name,T_cal,T,s", THRESH_SPLIT)
def test_split_threshold_calibration_and_masking(name, T_cal, T, s):
    inp, dev = layer(name, "gate")
    sh = inp.shape
    x_cal = inp.tokens(T_cal, 25)
    say(f"[case] split threshold {name} T_cal={T_cal} T={T} s={s}")
    tau = dev.calibrate(x_cal, s)
    tau_sh = dev.calibrate(x_cal, s, shared=True) if sh.n_shared else None
    ids_cal = dev.route_ids(x_cal)
    check_routing(inp, x_cal, ids_cal)
    t_or, t_or_sh = O.calibrate_thresholds(x_cal, inp.w_router, inp.bias, inp.wg, inp.wu,
                                           top_k=sh.top_k, norm_topk=sh.norm_topk,
                                           dtype=sh.dtype, sparsity=s, shared=inp.shared,
                                           score="gate", forced_ids=ids_cal)
    np.testing.assert_allclose(tau, t_or, rtol=1e-4, atol=1e-7)
    if tau_sh is not None:
        np.testing.assert_allclose(tau_sh, t_or_sh, rtol=1e-4, atol=1e-7)
    x = inp.tokens(T, 26)
    got = dev.run_threshold(x, torch.from_numpy(tau).cuda(),
                            torch.from_numpy(tau_sh).cuda() if tau_sh is not None else None)
    err = compare_threshold_layer(inp, x, got, tau, tau_sh, score="gate")
    say(f"   rel_l2={err:.3e} mean kept {got['cnt'].mean():.1f}")


def test_split_threshold_reads_only_kept_rows():
    # NaN in every W_u and W_d row no pair keeps under the threshold: same bits
    inp, dev = layer("olmoe-like", "gate")
    x = inp.tokens(4, 27)
    tau = torch.full((64,), 0.02, device="cuda")
    say("[case] split threshold, NaN-poisoned unkept rows")
    a = dev.run_threshold(x, tau)
    keep = np.zeros((64, 1024), dtype=bool)
    for p, e in enumerate(a["ids"].reshape(-1)):
        keep[e, a["idx"][p, :a["cnt"][p]]] = True
    poison = torch.from_numpy(~keep).cuda()
    w_saved = dev.w
    wu, wd = dev.w[1].clone(), dev.w[2].clone()
    wu[poison] = float("nan")
    wd[poison] = float("nan")
    try:
        dev.w = (dev.w[0], wu, wd)
        c = dev.run_threshold(x, tau)
    finally:
        dev.w = w_saved
    assert np.all(np.isfinite(c["y"]))
    np.testing.assert_array_equal(a["y"], c["y"])


def test_threshold_extremes_and_calibration_target():
    inp, dev = layer("olmoe-like")
    x = inp.tokens(16, 23)
    E = inp.shape.n_experts
    say("[case] threshold extremes")
    # tau < 0 keeps everything: the dense SwiGLU MoE, the same as k = d_ff
    allk = dev.run_threshold(x, torch.full((E,), -1.0, device="cuda"))
    assert np.all(allk["cnt"] == inp.shape.d_ff)
    full = dev.run(x, inp.shape.d_ff, SP)
    assert rel_l2(allk["y"], full["y"]) < 1e-5
    # a huge tau keeps nothing: y == 0
    none = dev.run_threshold(x, torch.full((E,), 1e30, device="cuda"))
    assert np.all(none["cnt"] == 0) and np.all(none["y"] == 0)
    # the kept counts and ids are optional outputs; y does not depend on them
    tau_mid = torch.full((E,), 0.05, device="cuda")
    for T in (16, 40):
        xt = inp.tokens(T, 24)
        a = dev.run_threshold(xt, tau_mid)
        b = dev.run_threshold(xt, tau_mid, outputs=False)
        np.testing.assert_array_equal(a["y"], b["y"])
    # calibrated on these very tokens, each expert keeps its target count
    for s in (0.5, 0.9):
        tau = dev.calibrate(x, s)
        got = dev.run_threshold(x, torch.from_numpy(tau).cuda())
        ids = got["ids"].reshape(-1)
        for e in np.unique(ids):
            n = int(got["cnt"][ids == e].sum())
            m = int((ids == e).sum()) * inp.shape.d_ff
            assert n == O.keep_count(s, m), (e, n, m)


# ------------------------------------------------------------------ ragged shapes and edges

RAGGED = dict(hidden=320, n_experts=12, d_ff=192, top_k=3, norm_topk=True, n_shared=1,
              d_ff_shared=128, zipf_bias=None)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("T", [1, 17, 37, 130])
@pytest.mark.parametrize("path", [SP, DN])
def test_ragged_shapes(dtype, T, path):
    run_case("olmoe-like", T, 0.7, path, s_sh=0.5, path_sh=1 - path, dtype=dtype, **RAGGED)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d_ff", [2112, 3584, 4096])
@pytest.mark.parametrize("path", [SP, DN])
def test_large_dff_masks(dtype, d_ff, path):
    # d_ff past the one-wave mask: 8-wave segments with an odd and an even
    # per-lane count (3584, 4096), the LDS fallback (2112), and a shared
    # expert of d_ff 2560
    run_case("olmoe-like", 5, 0.9, path, s_sh=0.5, path_sh=path, dtype=dtype,
             **dict(hidden=128, n_experts=4, d_ff=d_ff, top_k=2, norm_topk=False, n_shared=1,
                    d_ff_shared=2560, zipf_bias=None))


@pytest.mark.parametrize("k", [0, 1, 191, 192])
def test_keep_extremes(k):
    inp, dev = layer("olmoe-like", dtype="f32", **RAGGED)
    x = inp.tokens(9, 3)
    for path in (SP, DN):
        say(f"[case] ragged f32 k={k} path={path}")
        got = dev.run(x, k, path, k_sh=64, path_sh=SP)
        compare_layer(inp, x, got, k, k_sh=64)


def test_all_experts_selected_and_single_expert():
    run_case("olmoe-like", 5, 0.5, SP, s_sh=0.0, dtype="f32", **dict(RAGGED, top_k=12))
    run_case("olmoe-like", 5, 0.5, DN, s_sh=0.0, dtype="f32", **dict(RAGGED, n_experts=1, top_k=1))


@pytest.mark.parametrize("score,path", [("swiglu", SP), ("swiglu", DN), ("gate", SP)])
def test_max_experts_and_top_k(score, path):
    # E = 1024 experts and top-32 routing, the ABI's maxima
    run_case("olmoe-like", 3, 0.75, path, score=score,
             **dict(hidden=128, n_experts=1024, d_ff=64, top_k=32, norm_topk=True))


@pytest.mark.parametrize("score,path", [("swiglu", SP), ("swiglu", DN), ("gate", SP)])
def test_max_hidden(score, path):
    # H = 16384, the ABI's maximum hidden size, on the fp32 layer
    run_case("olmoe-like", 2, 0.75, path, score=score,
             **dict(dtype="f32", hidden=16384, n_experts=2, d_ff=128, top_k=1, norm_topk=False))


def test_many_tokens_max_T():
    # the largest token count the ABI takes, on the small fp32 layer, every row
    run_case("tiny-f32", 65536, 0.9, SP)


# ------------------------------------------------------------------ properties

@pytest.mark.parametrize("dtype,E,d,H", [("bf16", 3, 64, 128), ("f32", 2, 128, 320),
                                         ("bf16", 5, 1536, 5120)])
def test_pack_gate_up_layout(dtype, E, d, H):
    rng = np.random.default_rng(0)
    a = rng.standard_normal((E, d, H)).astype(np.float32)
    host = S.round_to_bf16_bits(a) if dtype == "bf16" else a
    desc = B.make_desc(H, E, d, 1, False, dtype, gate_up_layout="packed")
    w = to_dev(host)
    pk = B.moe_pack_gate_up(desc, w)
    back = B.moe_unpack_gate_up(desc, pk)
    torch.cuda.synchronize()
    view = np.int16 if dtype == "bf16" else np.float32
    got = pk.view(torch.int16 if dtype == "bf16" else torch.float32).cpu().numpy()
    want = pack_reference(host.view(view) if dtype == "bf16" else host, dtype)
    np.testing.assert_array_equal(got, want)
    assert torch.equal(back.view(torch.int16 if dtype == "bf16" else torch.int32),
                       w.view(torch.int16 if dtype == "bf16" else torch.int32))
    with pytest.raises(B.MoeError):
        B.moe_pack_gate_up(desc, w, w)        # in place is refused


def test_deterministic_and_sparse_equals_dense():
    inp, dev = layer("olmoe-like")
    x = inp.tokens(16, 5)
    k = O.keep_count(0.9, 1024)
    say("[case] determinism olmoe-like T=16")
    a = dev.run(x, k, SP)
    b = dev.run(x, k, SP)
    np.testing.assert_array_equal(a["y"], b["y"])
    np.testing.assert_array_equal(a["idx"], b["idx"])
    c = dev.run(x, k, DN)
    np.testing.assert_array_equal(a["idx"], c["idx"])
    assert rel_l2(c["y"], a["y"]) < 1e-2


@pytest.mark.parametrize("nbytes", [16, 4096 * 16 + 48, 3375104, 54001664, 64 << 20, 300 << 20])
def test_stream_read_folds_every_chunk(nbytes):
    # the calibration read touches every 16-byte chunk exactly once: the XOR
    # of all block folds equals the XOR of all chunks
    rng = np.random.default_rng(nbytes)
    host = rng.integers(0, 2**32, size=nbytes // 4, dtype=np.uint32)
    buf = torch.from_numpy(host.view(np.int32)).cuda()
    sink = torch.zeros(B.STREAM_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    B.moe_stream_read(buf, sink)
    got = np.bitwise_xor.reduce(sink.cpu().numpy().view(np.uint32).reshape(-1, 4), axis=0)
    want = np.bitwise_xor.reduce(host.reshape(-1, 4), axis=0)
    np.testing.assert_array_equal(got, want)


def test_unkept_rows_are_never_read():
    # Poison every W_d row no pair keeps with NaN: the sparse path must give
    # the same bits (a load-and-multiply by zero would give NaN).
    inp, dev = layer("olmoe-like")
    x = inp.tokens(4, 7)
    k = O.keep_count(0.9, 1024)
    say("[case] NaN-poisoned W_d rows")
    a = dev.run(x, k, SP)
    wd = dev.w[2].clone()
    keep = np.zeros((64, 1024), dtype=bool)
    ids = a["ids"].reshape(-1)
    for p, e in enumerate(ids):
        keep[e, a["idx"][p, :k]] = True
    poison = torch.from_numpy(~keep).cuda()
    wd[poison] = float("nan")
    b = dev.run(x, k, SP, poison_rows=wd)
    assert np.all(np.isfinite(b["y"]))
    np.testing.assert_array_equal(a["y"], b["y"])


def test_outputs_outside_bounds_untouched_and_accumulate():
    inp, dev = layer("olmoe-like")
    sh = inp.shape
    T = 3
    k = O.keep_count(0.9, 1024)
    x = to_dev(inp.tokens(T, 9))
    R = B.Routing.allocate(T, sh.top_k, sh.n_experts)
    B.moe_route(dev.desc, T, x, dev.w_router, None, R,
                torch.empty(B.moe_route_workspace_size(dev.desc, T), dtype=torch.uint8, device="cuda"))
    for path in (SP, DN):
        buf = torch.full((T + 2, sh.hidden), 12345.0, device="cuda")
        y = buf[1:T + 1]
        ws = torch.empty(B.moe_ffn_workspace_size(dev.desc, T, k, path), dtype=torch.uint8, device="cuda")
        fn = B.moe_expert_ffn_sparse if path == SP else B.moe_expert_ffn_dense
        fn(dev.desc, T, k, x, *dev.w, R, y, 0, None, ws)
        y1 = y.clone()
        y.zero_()
        fn(dev.desc, T, k, x, *dev.w, R, y, 1, None, ws)      # 0 + contribution: same bits
        torch.cuda.synchronize()
        assert torch.all(buf[0] == 12345.0) and torch.all(buf[T + 1] == 12345.0)
        torch.testing.assert_close(y, y1, rtol=0, atol=0)
        fn(dev.desc, T, k, x, *dev.w, R, y, 1, None, ws)      # y1 + contribution
        torch.testing.assert_close(y, 2 * y1, rtol=1e-6, atol=1e-7)
        y2 = y.clone()
        fn(dev.desc, T, 0, x, *dev.w, R, y, 1, None, ws)      # k = 0 adds nothing
        torch.testing.assert_close(y, y2, rtol=0, atol=0)
        fn(dev.desc, T, 0, x, *dev.w, R, y, 0, None, ws)      # ... and overwrites with 0
        torch.cuda.synchronize()
        assert torch.all(y == 0) and torch.all(buf[T + 1] == 12345.0)
        fn(dev.desc, 0, k, x, *dev.w, R, y, 0, None, ws)      # T = 0 is a no-op
        torch.cuda.synchronize()
        assert torch.all(y == 0)


def test_errors_leave_outputs_untouched():
    inp, dev = layer("olmoe-like")
    T = 2
    x = to_dev(inp.tokens(T, 2))
    R = B.Routing.allocate(T, 8, 64)
    y = torch.full((T, 2048), 7.0, device="cuda")
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(B.MoeError) as ei:
        B.moe_expert_ffn_sparse(dev.desc, T, 103, x, *dev.w, R, y, 0, None, ws)
    assert ei.value.status == 3
    with pytest.raises(B.MoeError):
        B.moe_expert_ffn_dense(dev.desc, T, 2000, x, *dev.w, R, y, 0, None, ws)
    torch.cuda.synchronize()
    assert torch.all(y == 7.0)


@pytest.mark.parametrize("T", [1, 2, 4])
def test_layer_class_matches_direct_calls(T):
    # MoELayer runs moe_layer_sparse (the selection inside gate/up at T <= 2)
    from sparse_moe_expert_route_amd.layer import MoELayer
    inp, dev = layer("deepseek-v2-like")
    sh = inp.shape
    x_host = inp.tokens(T, 11)
    k, k_sh = O.keep_count(0.9, sh.d_ff), O.keep_count(0.5, sh.d_ff_shared)
    m = MoELayer(hidden=sh.hidden, n_experts=sh.n_experts, d_ff=sh.d_ff, top_k=sh.top_k,
                 norm_topk=sh.norm_topk, dtype=sh.dtype, w_router=dev.w_router,
                 w_gate=dev.w[0], w_up=dev.w[1], w_down=dev.w[2], shared=dev.w_sh, packed=True)
    say(f"[case] MoELayer deepseek-v2-like T={T}")
    y = m.forward(to_dev(x_host), k, k_sh, path=SP, path_shared=SP)
    got = dev.run(x_host, k, SP, k_sh, SP)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(y.cpu().numpy(), got["y"])


# ------------------------------------------------------------------ canaries

def _pad(dtype):  # 256 bytes of canary before and after every buffer
    return 256 // torch.empty((), dtype=dtype).element_size()


def _canaried(n, dtype, fill):
    pad = _pad(dtype)
    full = torch.full((n + 2 * pad,), fill, dtype=dtype, device="cuda")
    return full, full[pad:pad + n]


def _intact(full, n, fill, what):
    torch.cuda.synchronize()
    pad = _pad(full.dtype)
    head, tail = full[:pad], full[pad + n:]
    assert torch.all(head == fill) and torch.all(tail == fill), f"{what}: canary overwritten"


@pytest.mark.parametrize("T", [1, 4, 16, 40])
def test_no_write_outside_any_buffer(T):
    # every entry point, on buffers sized exactly as the header states, with
    # canaries around each output and workspace
    inp, dev = layer("olmoe-like")
    inp_g, dev_g = layer("olmoe-like", "gate")
    sh = inp.shape
    E, K, H, d = sh.n_experts, sh.top_k, sh.hidden, sh.d_ff
    P, k = T * K, O.keep_count(0.9, d)
    say(f"[case] canaries T={T}")
    x = to_dev(inp.tokens(T, 31))
    bufs = []

    def buf(n, dtype=torch.int32, fill=-7):
        full, view = _canaried(n, dtype, fill)
        bufs.append((full, n, fill, f"buffer {len(bufs)}"))
        return view

    def ws(nbytes):
        return buf(nbytes, torch.uint8, 0x5A)

    R = B.Routing(buf(P).view(T, K), buf(P, torch.float32, -7.0).view(T, K), buf(E + 1), buf(P),
                  buf(E), buf(1))
    B.moe_route(dev.desc, T, x, dev.w_router, None, R, ws(B.moe_route_workspace_size(dev.desc, T)))
    usage = buf(T * E).view(T, E)
    usage.zero_()
    B.moe_route_roster(dev.desc, T, x, dev.w_router, None, usage, None, 8, 0.5, R,
                       ws(B.moe_route_workspace_size(dev.desc, T)))
    for path in (SP, DN):
        fn = B.moe_expert_ffn_sparse if path == SP else B.moe_expert_ffn_dense
        fn(dev.desc, T, k, x, *dev.w, R, buf(T * H, torch.float32, -7.0).view(T, H), 0,
           buf(P * k).view(P, k), ws(B.moe_ffn_workspace_size(dev.desc, T, k, path)))
    B.moe_expert_ffn_sparse_updown(dev_g.desc, T, k, x, *dev_g.w, R,
                                   buf(T * H, torch.float32, -7.0).view(T, H), 0,
                                   buf(P * k).view(P, k),
                                   ws(B.moe_ffn_workspace_size(dev_g.desc, T, k, SP)))
    tau = buf(E, torch.float32, -7.0)
    B.moe_calibrate_thresholds(dev.desc, T, x, dev.w[0], dev.w[1], R, 0.9, tau,
                               ws(B.moe_calibrate_workspace_size(dev.desc, T)))
    B.moe_expert_ffn_sparse_threshold(dev.desc, T, tau, x, *dev.w, R,
                                      buf(T * H, torch.float32, -7.0).view(T, H), 0, buf(P),
                                      buf(P * d).view(P, d),
                                      ws(B.moe_ffn_threshold_workspace_size(dev.desc, T)))
    tau_g = buf(E, torch.float32, -7.0)
    B.moe_calibrate_thresholds_gate(dev_g.desc, T, x, dev_g.w[0], R, 0.9, tau_g,
                                    ws(B.moe_calibrate_workspace_size(dev_g.desc, T)))
    B.moe_expert_ffn_sparse_updown_threshold(dev_g.desc, T, tau_g, x, *dev_g.w, R,
                                             buf(T * H, torch.float32, -7.0).view(T, H), 0,
                                             buf(P), buf(P * d).view(P, d),
                                             ws(B.moe_ffn_threshold_workspace_size(dev_g.desc, T)))
    y = buf(T * H, torch.float32, 0.0).view(T, H)
    xo = buf(T * H // 2, torch.int32, -7).view(torch.bfloat16).view(T, H)
    B.moe_residual_add(dev.desc, T, x, y, xo)
    for full, n, fill, what in bufs:
        _intact(full, n, fill, what)
