"""Pins of the CPU oracle to things other than itself.

Each test checks the oracle against a closed form, a hand-derived worked
example, brute-force enumeration, a library routine or an invariant of the
definition, chosen so that a plausible slip (|h| vs h, largest vs smallest,
a tie going the wrong way, gate and up swapped, a dropped router weight or
renormalisation, a wrong W_d row) fails at least one of them.  CPU only.
"""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle
from oracle import moe_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ keep count

def _golden_keep_rows():
    rows = []
    with open(os.path.join(GOLDEN, "keep_counts.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            s, d, k = line.split()[:3]
            rows.append((s, int(d), int(k)))
    return rows


@pytest.mark.parametrize("s,d_ff,k", _golden_keep_rows())
def test_keep_count_golden(s, d_ff, k):
    # fixture value, and the exact rational ceiling of (1 - s) * d_ff
    exact = math.ceil((1 - Fraction(s)) * d_ff)
    assert exact == k
    assert O.keep_count(float(s), d_ff) == k


def test_keep_count_exact_rational_sweep():
    # every sparsity with up to 3 decimals against exact rationals
    for d_ff in (512, 768, 1000, 1024, 1536, 8192):
        for m in range(0, 1001):
            s = Fraction(m, 1000)
            assert O.keep_count(float(s), d_ff) == math.ceil((1 - s) * d_ff), (m, d_ff)


# ------------------------------------------------------------ selection

def _dominates(score, K, n):
    """Brute-force definition: K holds the |K| best by (score desc, index asc)."""
    Ks = set(K)
    for i in Ks:
        for j in range(n):
            if j in Ks:
                continue
            if not (score[i] > score[j] or (score[i] == score[j] and i < j)):
                return False
    return True


def _tie_heavy(rng, n):
    vals = np.array([-2.0, -1.0, -0.0, 0.0, 1.0, 2.0, 0.5, -0.5])
    return vals[rng.integers(0, len(vals), n)]


@pytest.mark.parametrize("seed", range(40))
def test_kept_neurons_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, 10))
    h = _tie_heavy(rng, n) if seed % 2 else rng.standard_normal(n)
    for k in range(n + 1):
        got = O.kept_neurons(h, k)
        assert list(got) == sorted(got)
        winners = [c for c in itertools.combinations(range(n), k)
                   if _dominates(np.abs(h), c, n)]
        assert len(winners) == 1
        assert tuple(got) == winners[0]


def test_kept_neurons_uses_magnitude_and_zero_signs():
    h = np.array([-3.0, 1.0, 2.0, -0.0, 0.0])
    assert list(O.kept_neurons(h, 1)) == [0]           # |-3| wins: magnitude, not value
    assert list(O.kept_neurons(h, 2)) == [0, 2]
    assert list(O.kept_neurons(h, 4)) == [0, 1, 2, 3]  # -0 == +0, lower index first


@pytest.mark.parametrize("seed", range(30))
def test_top_experts_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    E = int(rng.integers(1, 9))
    l = _tie_heavy(rng, E) if seed % 2 else rng.standard_normal(E)
    for k in range(1, E + 1):
        got = O.top_experts(l, k)
        winners = [c for c in itertools.combinations(range(E), k) if _dominates(l, c, E)]
        assert len(winners) == 1
        assert sorted(got) == list(winners[0])          # signed logits, not |l|
        # slot order: descending logit, ties to the lower id
        keys = [(-l[e], e) for e in got]
        assert keys == sorted(keys)


# ------------------------------------------------------------ softmax / route

def test_softmax_closed_form():
    l = np.array([[math.log(3.0), 0.0, math.log(4.0)]])
    np.testing.assert_allclose(O.softmax(l), [[3 / 8, 1 / 8, 4 / 8]], rtol=1e-15)
    np.testing.assert_allclose(O.softmax(np.array([[1000.0, 1000.0]])), [[0.5, 0.5]])
    # ratio property p_i / p_j = exp(l_i - l_j)
    rng = np.random.default_rng(1)
    l = rng.standard_normal((4, 7)) * 3
    p = O.softmax(l)
    np.testing.assert_allclose(p[:, 1] / p[:, 4], np.exp(l[:, 1] - l[:, 4]), rtol=1e-12)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)


@pytest.mark.parametrize("norm", [False, True])
def test_route_against_torch(norm):
    rng = np.random.default_rng(7)
    T, H, E, k = 6, 32, 12, 3
    x = rng.standard_normal((T, H))
    wr = rng.standard_normal((E, H)) / np.sqrt(H)
    b = rng.standard_normal(E).astype(np.float32)
    ids, w, l, p = O.route(x, wr, b, k, norm)
    lt = F.linear(torch.from_numpy(x), torch.from_numpy(wr)) + torch.from_numpy(b).double()
    pt = torch.softmax(lt, dim=-1)
    tv, ti = torch.topk(pt, k, dim=-1)          # random data: no ties
    if norm:
        tv = tv / tv.sum(dim=-1, keepdim=True)
    np.testing.assert_array_equal(ids, ti.numpy())
    np.testing.assert_allclose(w, tv.numpy(), rtol=1e-13)
    if norm:
        np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)


# ------------------------------------------------------------ activation

def test_silu_library_and_limits():
    z = np.linspace(-30, 30, 1001)
    np.testing.assert_allclose(O.silu(z), z * scipy.special.expit(z), rtol=1e-13, atol=1e-300)
    assert O.silu(np.array([0.0]))[0] == 0.0
    big = O.silu(np.array([-800.0, 800.0]))
    assert np.all(np.isfinite(big)) and big[0] == 0.0 and big[1] == 800.0


def test_expert_activation_against_torch():
    rng = np.random.default_rng(3)
    H, d = 48, 40
    x = rng.standard_normal(H)
    wg, wu = rng.standard_normal((d, H)), rng.standard_normal((d, H))
    want = (F.silu(F.linear(torch.from_numpy(x), torch.from_numpy(wg)))
            * F.linear(torch.from_numpy(x), torch.from_numpy(wu))).numpy()
    np.testing.assert_allclose(O.expert_activation(x, wg, wu), want, rtol=1e-12, atol=1e-14)
    # gate and up are not interchangeable
    assert not np.allclose(O.expert_activation(x, wu, wg), want)


def test_expert_scores_batch_against_torch():
    # several tokens of one expert at once: each row is the per-token
    # definition (SwiGLU product, or the gate-only score of the split)
    rng = np.random.default_rng(4)
    n, H, d = 5, 48, 40
    X = rng.standard_normal((n, H))
    wg, wu = rng.standard_normal((d, H)), rng.standard_normal((d, H))
    g = F.linear(torch.from_numpy(X), torch.from_numpy(wg))
    u = F.linear(torch.from_numpy(X), torch.from_numpy(wu))
    np.testing.assert_allclose(O.expert_scores_batch(X, wg, wu, "swiglu"), (F.silu(g) * u).numpy(),
                               rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(O.expert_scores_batch(X, wg, wu, "gate"), F.silu(g).numpy(),
                               rtol=1e-12, atol=1e-14)
    # row order follows the tokens; gate and up are not interchangeable
    np.testing.assert_allclose(O.expert_scores_batch(X[::-1], wg, wu, "swiglu")[::-1],
                               (F.silu(g) * u).numpy(), rtol=1e-12, atol=1e-14)
    assert not np.allclose(O.expert_scores_batch(X, wu, wg, "swiglu"), (F.silu(g) * u).numpy())


def test_sparse_down_reads_only_kept_rows():
    rng = np.random.default_rng(4)
    d, H = 20, 16
    h = rng.standard_normal(d)
    wd = rng.standard_normal((d, H))
    keep = O.kept_neurons(h, 5)
    poisoned = np.full_like(wd, np.nan)
    poisoned[keep] = wd[keep]
    got = O.sparse_down(h, keep, poisoned)
    hm = np.zeros(d)
    hm[keep] = h[keep]
    assert np.all(np.isfinite(got))
    np.testing.assert_allclose(got, hm @ wd, rtol=1e-13)
    assert np.all(O.sparse_down(h, keep[:0], poisoned) == 0)


# ------------------------------------------------------------ worked examples

def _eval_expr(s):
    return float(eval(s, {"__builtins__": {}}, {"exp": math.exp}))


def _golden_cases():
    with open(os.path.join(GOLDEN, "worked_examples.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden_cases(), ids=lambda c: c["name"])
def test_worked_example(case):
    f32 = lambda a: np.asarray(a, dtype=np.float32)
    bias = None if case["bias"] is None else f32(case["bias"])
    r = oracle.moe_layer(f32(case["x"]), f32(case["w_router"]), bias,
                         f32(case["w_gate"]), f32(case["w_up"]), f32(case["w_down"]),
                         top_k=case["top_k"], norm_topk=case["norm_topk"],
                         k_keep=case["k_keep"], dtype="f32", score=case.get("score", "swiglu"))
    np.testing.assert_array_equal(r.ids, case["expect_ids"])
    want = np.array([[_eval_expr(s) for s in row] for row in case["expect"]])
    np.testing.assert_allclose(r.y, want, rtol=1e-14, atol=1e-15)


# ------------------------------------------------------------ whole layer

def _rand_layer(seed, T=3, H=16, E=6, d=12, dtype="f32"):
    rng = np.random.default_rng(seed)
    f = lambda *s: (rng.standard_normal(s) / np.sqrt(s[-1])).astype(np.float32)
    return dict(x=rng.standard_normal((T, H)).astype(np.float32), wr=f(E, H),
                bias=rng.standard_normal(E).astype(np.float32) * 0.1,
                wg=f(E, d, H), wu=f(E, d, H), wd=(rng.standard_normal((E, d, H)) / np.sqrt(d)).astype(np.float32))


def _run(L, top_k, norm, k, **kw):
    return oracle.moe_layer(L["x"], L["wr"], L["bias"], L["wg"], L["wu"], L["wd"],
                            top_k=top_k, norm_topk=norm, k_keep=k, dtype="f32", **kw)


def _brute_layer(L, top_k, norm, k, score="swiglu", taus=None):
    """Scalar float64 loops; mask by brute-force subset enumeration.  With
    score="gate" neurons are ranked by |silu(g)| alone and u is formed for
    the kept neurons only."""
    x, wr, b, wg, wu, wd = (np.asarray(L[n], dtype=np.float64) for n in ("x", "wr", "bias", "wg", "wu", "wd"))
    T, H = x.shape
    E, d, _ = wg.shape
    y = [[0.0] * H for _ in range(T)]
    for t in range(T):
        logit = [sum(x[t, i] * wr[e, i] for i in range(H)) + b[e] for e in range(E)]
        sel = next(c for c in itertools.combinations(range(E), top_k) if _dominates(logit, c, E))
        m = max(logit)
        z = sum(math.exp(v - m) for v in logit)
        p = {e: math.exp(logit[e] - m) / z for e in sel}
        tot = sum(p.values())
        for e in sel:
            w = p[e] / tot if norm else p[e]
            h, sg = [], []
            for j in range(d):
                g = sum(wg[e, j, i] * x[t, i] for i in range(H))
                u = sum(wu[e, j, i] * x[t, i] for i in range(H))
                sg.append(g / (1 + math.exp(-g)))
                h.append(sg[-1] * u)
            rank = h if score == "swiglu" else sg
            if taus is not None:                  # threshold mask: a compare per neuron
                K = [j for j in range(d) if abs(rank[j]) > taus[e]]
            else:
                K = next(c for c in itertools.combinations(range(d), k)
                         if _dominates([abs(v) for v in rank], c, d))
            for j in K:
                for i in range(H):
                    y[t][i] += w * h[j] * wd[e, j, i]
    return np.array(y)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("top_k,norm,k", [(2, False, 3), (3, True, 1), (1, True, 12), (2, False, 0)])
def test_layer_brute_force(seed, top_k, norm, k):
    L = _rand_layer(seed, T=2, H=8, E=5, d=8 if k != 12 else 12)
    r = _run(L, top_k, norm, k)
    np.testing.assert_allclose(r.y, _brute_layer(L, top_k, norm, k), rtol=1e-11, atol=1e-13)


@pytest.mark.parametrize("seed", range(6))
@pytest.mark.parametrize("top_k,norm,k", [(2, False, 3), (3, True, 1), (1, True, 12), (2, False, 0)])
def test_gate_score_layer_brute_force(seed, top_k, norm, k):
    L = _rand_layer(100 + seed, T=2, H=8, E=5, d=8 if k != 12 else 12)
    r = _run(L, top_k, norm, k, score="gate")
    np.testing.assert_allclose(r.y, _brute_layer(L, top_k, norm, k, score="gate"),
                               rtol=1e-11, atol=1e-13)


def test_gate_score_mask_ignores_up_projection():
    # the gate alone ranks the neurons: a new W_u changes no kept set (while
    # it does change the SwiGLU-scored sets), and y scales with W_u
    L = _rand_layer(21, T=4, H=32, E=4, d=24)
    wu2 = _rand_layer(22, T=4, H=32, E=4, d=24)["wu"]
    a = _run(L, 2, False, 5, score="gate")
    b = _run(dict(L, wu=wu2), 2, False, 5, score="gate")
    assert all(np.array_equal(a.keep[key], b.keep[key]) for key in a.keep)
    sa = _run(L, 2, False, 5)
    sb = _run(dict(L, wu=wu2), 2, False, 5)
    assert any(not np.array_equal(sa.keep[key], sb.keep[key]) for key in sa.keep)
    assert any(not np.array_equal(a.keep[key], sa.keep[key]) for key in a.keep)
    c = _run(dict(L, wu=L["wu"] * 2.0), 2, False, 5, score="gate")
    np.testing.assert_allclose(c.y, 2.0 * a.y, rtol=1e-14)
    # the scores it reports are silu(W_g x)
    for (t, s), sc in a.h.items():
        e = int(a.ids[t, s])
        g = L["wg"][e].astype(np.float64) @ L["x"][t].astype(np.float64)
        np.testing.assert_allclose(sc, scipy.special.expit(g) * g, rtol=1e-13, atol=1e-15)


def test_gate_score_reads_only_kept_up_and_down_rows():
    L = _rand_layer(23, T=4, H=32, E=8, d=40)
    r = _run(L, 2, False, 4, score="gate")
    wu, wd = L["wu"].copy(), L["wd"].copy()
    used = {}
    for (t, s), keep in r.keep.items():
        used.setdefault(int(r.ids[t, s]), set()).update(int(j) for j in keep)
    for e in range(wd.shape[0]):
        for j in range(wd.shape[1]):
            if j not in used.get(e, ()):
                wu[e, j] = np.nan
                wd[e, j] = np.nan
    r2 = _run(dict(L, wu=wu, wd=wd), 2, False, 4, score="gate")
    assert np.all(np.isfinite(r2.y))
    np.testing.assert_array_equal(r2.y, r.y)


@pytest.mark.parametrize("seed", range(3))
def test_gate_score_at_sparsity_zero_is_dense_moe(seed):
    L = _rand_layer(30 + seed, T=4, H=32, E=8, d=24)
    r = _run(L, 2, True, 24, score="gate")
    np.testing.assert_allclose(r.y, _torch_dense_moe(L, 2, True), rtol=1e-12, atol=1e-14)


def _torch_dense_moe(L, top_k, norm):
    """A dense MoE layer from torch library calls (no masking)."""
    td = lambda a: torch.from_numpy(np.asarray(a, dtype=np.float64))
    x = td(L["x"])
    p = torch.softmax(F.linear(x, td(L["wr"])) + td(L["bias"]), dim=-1)
    val, idx = torch.topk(p, top_k, dim=-1)
    if norm:
        val = val / val.sum(-1, keepdim=True)
    y = torch.zeros_like(x)
    for t in range(x.shape[0]):
        for s in range(top_k):
            e = int(idx[t, s])
            act = F.silu(F.linear(x[t], td(L["wg"][e]))) * F.linear(x[t], td(L["wu"][e]))
            y[t] += val[t, s] * F.linear(act, td(L["wd"][e]).T)   # down_proj.weight is W_d^T
    return y.numpy()


@pytest.mark.parametrize("seed", range(4))
def test_sparsity_zero_is_dense_moe(seed):
    L = _rand_layer(seed, T=4, H=32, E=8, d=24)
    for top_k, norm in ((2, False), (3, True)):
        r = _run(L, top_k, norm, O.keep_count(0.0, 24))
        np.testing.assert_allclose(r.y, _torch_dense_moe(L, top_k, norm), rtol=1e-12, atol=1e-14)


def test_single_expert_is_textbook_swiglu_ffn():
    L = _rand_layer(9, T=3, H=32, E=1, d=24)
    r = _run(L, 1, True, 24)
    x = torch.from_numpy(L["x"]).double()
    ffn = F.linear(F.silu(F.linear(x, torch.from_numpy(L["wg"][0]).double()))
                   * F.linear(x, torch.from_numpy(L["wu"][0]).double()),
                   torch.from_numpy(L["wd"][0]).double().T)
    np.testing.assert_allclose(r.y, ffn.numpy(), rtol=1e-12, atol=1e-14)


def test_zeroed_neurons_contribute_nothing():
    L = _rand_layer(11, T=4, H=32, E=8, d=40)
    r = _run(L, 2, False, 4)
    # poison every W_d row that no pair keeps
    wd = L["wd"].copy()
    used = {}
    for (t, s), keep in r.keep.items():
        used.setdefault(int(r.ids[t, s]), set()).update(int(j) for j in keep)
    for e in range(wd.shape[0]):
        for j in range(wd.shape[1]):
            if j not in used.get(e, ()):
                wd[e, j] = np.nan
    r2 = _run(dict(L, wd=wd), 2, False, 4)
    assert np.all(np.isfinite(r2.y))
    np.testing.assert_array_equal(r2.y, r.y)
    # and the kept count is exactly k for every pair
    assert all(len(v) == 4 for v in r.keep.values())


def test_batch_invariance():
    L = _rand_layer(12, T=5, H=32, E=8, d=24)
    full = _run(L, 2, True, 5)
    for t in range(5):
        one = _run(dict(L, x=L["x"][t:t + 1]), 2, True, 5)
        # equal up to BLAS blocking order; the same experts and neurons
        np.testing.assert_allclose(one.y[0], full.y[t], rtol=1e-13, atol=1e-16)
        assert np.array_equal(one.ids[0], full.ids[t])


def test_expert_permutation_invariance():
    L = _rand_layer(13, T=4, H=32, E=8, d=24)
    perm = np.random.default_rng(0).permutation(8)
    P = {n: L[n][perm] for n in ("wr", "bias", "wg", "wu", "wd")}
    a = _run(L, 3, False, 6)
    b = _run(dict(L, **P), 3, False, 6)
    np.testing.assert_allclose(a.y, b.y, rtol=1e-13, atol=1e-15)
    np.testing.assert_array_equal(perm[b.ids], a.ids)


def test_up_scaling_and_sign_flip_keep_mask():
    L = _rand_layer(14, T=3, H=32, E=4, d=24)
    a = _run(L, 1, True, 5)
    wu = L["wu"].copy()
    wu *= 2.0                                    # exact in binary
    b = _run(dict(L, wu=wu), 1, True, 5)
    assert all(np.array_equal(a.keep[key], b.keep[key]) for key in a.keep)
    np.testing.assert_allclose(b.y, 2.0 * a.y, rtol=1e-14)
    wu = L["wu"].copy()
    wu[:, ::2] *= -1                             # flip the sign of every even neuron
    c = _run(dict(L, wu=wu), 1, True, 5)
    assert all(np.array_equal(a.keep[key], c.keep[key]) for key in a.keep)


def test_shared_experts_weight_one_own_mask():
    L = _rand_layer(15, T=3, H=32, E=4, d=24)
    S = _rand_layer(16, T=3, H=32, E=2, d=16)
    r = _run(L, 2, False, 5, shared=(S["wg"], S["wu"], S["wd"]), k_keep_shared=16)
    # shared part at k = d_ff is two dense SwiGLU FFNs summed with weight 1
    x = torch.from_numpy(L["x"]).double()
    want = sum(F.linear(F.silu(F.linear(x, torch.from_numpy(S["wg"][j]).double()))
                        * F.linear(x, torch.from_numpy(S["wu"][j]).double()),
                        torch.from_numpy(S["wd"][j]).double().T) for j in range(2))
    np.testing.assert_allclose(r.y_shared, want.numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(r.y, r.y_routed + r.y_shared, rtol=0, atol=0)
    r2 = _run(L, 2, False, 5, shared=(S["wg"], S["wu"], S["wd"]), k_keep_shared=8)
    assert all(len(v) == 8 for v in r2.keep_shared.values())


def test_forced_mode_reproduces_own_choice():
    L = _rand_layer(17, T=4, H=32, E=8, d=24)
    a = _run(L, 3, True, 5)
    b = _run(L, 3, True, 5, forced_ids=a.ids, forced_keep=a.keep)
    np.testing.assert_array_equal(a.y, b.y)


def test_bf16_inputs_are_exact_bit_patterns():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x3E80], dtype=np.uint16)
    np.testing.assert_array_equal(O.to_f64(bits, "bf16"), [1.0, -1.0, 3.140625, 0.0, -0.0, 0.25])
    with pytest.raises(ValueError):
        oracle.moe_layer(np.array([[np.nan, 0.0]], dtype=np.float32), np.zeros((2, 2), np.float32),
                         None, np.zeros((2, 2, 2), np.float32), np.zeros((2, 2, 2), np.float32),
                         np.zeros((2, 2, 2), np.float32), top_k=1, norm_topk=False, k_keep=1, dtype="f32")


# ------------------------------------------------------------ threshold masking

@pytest.mark.parametrize("seed", range(20))
def test_calibrated_threshold_keeps_the_target_count(seed):
    rng = np.random.default_rng(200 + seed)
    m = int(rng.integers(1, 60))
    v = rng.standard_normal(m)
    for s in (0.0, 0.3, 0.5, 0.9, 0.99, 1.0):
        tau = O.calibrated_threshold(v, s)
        c = math.ceil((1 - s) * m - 1e-9)
        assert sum(1 for x in v if abs(x) > tau) == c
        if c < m:   # tau is the largest score left out
            assert tau == sorted(abs(x) for x in v)[m - c - 1]
    assert O.calibrated_threshold(v, 0.0) == -1.0


def test_threshold_mask_is_one_compare_pass():
    rng = np.random.default_rng(5)
    h = rng.standard_normal(50)
    h[7] = -0.0
    for tau in (-1.0, 0.0, 0.3, 1.1, 10.0):
        want = [j for j in range(50) if abs(h[j]) > tau]
        np.testing.assert_array_equal(O.threshold_neurons(h, tau), want)


def _rand_taus(L, seed):
    E = L["wg"].shape[0]
    return np.random.default_rng(seed).uniform(0.01, 0.2, size=E)


@pytest.mark.parametrize("seed", range(5))
@pytest.mark.parametrize("top_k,norm", [(2, False), (3, True)])
def test_threshold_layer_brute_force(seed, top_k, norm):
    L = _rand_layer(300 + seed, T=2, H=8, E=5, d=8)
    taus = _rand_taus(L, seed)
    for score in ("swiglu", "gate"):
        r = _run(L, top_k, norm, 0, score=score, thresholds=taus)
        np.testing.assert_allclose(r.y, _brute_layer(L, top_k, norm, 0, score=score, taus=taus),
                                   rtol=1e-11, atol=1e-13)


def test_threshold_minus_one_is_dense_moe():
    L = _rand_layer(40, T=4, H=32, E=8, d=24)
    r = _run(L, 2, True, 0, thresholds=np.full(8, -1.0))
    np.testing.assert_allclose(r.y, _torch_dense_moe(L, 2, True), rtol=1e-12, atol=1e-14)


@pytest.mark.parametrize("score", ["swiglu", "gate"])
@pytest.mark.parametrize("k", [1, 5, 23])
def test_threshold_at_pair_midpoint_is_the_top_k_layer(score, k):
    # one token: each routed expert serves one pair, so a tau_e between that
    # pair's k-th and (k+1)-th largest |score| keeps exactly its top k
    L = _rand_layer(44 + k, T=1, H=32, E=6, d=24)
    ref = _run(L, 3, True, k, score=score)
    taus = np.full(6, 1e9)
    for slot in range(3):
        v = np.sort(np.abs(ref.h[(0, slot)]))[::-1]
        taus[int(ref.ids[0, slot])] = 0.5 * (v[k - 1] + v[k])
    r = _run(L, 3, True, 0, score=score, thresholds=taus)
    for slot in range(3):
        np.testing.assert_array_equal(r.keep[(0, slot)], ref.keep[(0, slot)])
    np.testing.assert_allclose(r.y, ref.y, rtol=1e-13, atol=1e-15)


@pytest.mark.parametrize("score", ["swiglu", "gate"])
def test_calibration_hits_its_target_on_its_own_tokens(score):
    # calibrated on a token batch, the thresholds keep exactly c_e of each
    # expert's m_e scores on that batch (the scores are distinct)
    L = _rand_layer(41, T=12, H=32, E=6, d=24)
    S = _rand_layer(42, T=12, H=32, E=1, d=16)
    sh = (S["wg"], S["wu"], S["wd"])
    for s in (0.5, 0.9):
        tau, tau_sh = O.calibrate_thresholds(L["x"], L["wr"], L["bias"], L["wg"], L["wu"],
                                             top_k=2, norm_topk=False, dtype="f32", sparsity=s,
                                             score=score, shared=sh)
        r = _run(L, 2, False, 0, score=score, thresholds=tau, shared=sh, thresholds_shared=tau_sh)
        kept = {}
        for (t, slot), keep in r.keep.items():
            e = int(r.ids[t, slot])
            kept[e] = kept.get(e, 0) + len(keep)
        for e, n in kept.items():
            m = 24 * sum(1 for t in range(12) if e in r.ids[t])
            assert n == math.ceil((1 - s) * m - 1e-9), (e, n, m)
        assert sum(len(v) for v in r.keep_shared.values()) == math.ceil((1 - s) * 12 * 16 - 1e-9)


def test_calibration_expert_without_tokens_takes_layer_value():
    L = _rand_layer(43, T=2, H=32, E=8, d=24)
    tau, _ = O.calibrate_thresholds(L["x"], L["wr"], L["bias"], L["wg"], L["wu"], top_k=1,
                                    norm_topk=False, dtype="f32", sparsity=0.75)
    ids, *_ = O.route(L["x"].astype(np.float64), L["wr"].astype(np.float64), L["bias"], 1, False)
    used = set(int(e) for e in ids.ravel())
    all_scores = np.concatenate([O.expert_activation(L["x"][t].astype(np.float64),
                                                     L["wg"][int(ids[t, 0])].astype(np.float64),
                                                     L["wu"][int(ids[t, 0])].astype(np.float64))
                                 for t in range(2)])
    layer_tau = O.calibrated_threshold(all_scores, 0.75)
    for e in range(8):
        if e not in used:
            assert tau[e] == layer_tau


# ------------------------------------------------------------ roster routing
# Pins of the roster rule (Predatory MoE, technical summary, section 2).

def test_roster_worked_values():
    u = np.array([3, 0, 5, 1, 0, 2])
    np.testing.assert_array_equal(O.roster(u, 3), [0, 2, 5])
    np.testing.assert_array_equal(O.roster(np.array([2, 2, 2, 0]), 2), [0, 1])    # ties: lower id
    # 4 experts used: barrier at m = 3, exploration at m = 5
    np.testing.assert_array_equal(O.roster_bias(u, 3, 0.5, False), [.5, -.5, .5, -.5, -.5, .5])
    np.testing.assert_array_equal(O.roster_bias(u, 5, 0.5, False), np.zeros(6))
    np.testing.assert_array_equal(O.roster_bias(u, 4, 0.5, False), [.5, -.5, .5, .5, -.5, .5])
    pinned = O.roster_bias(u, 2, 0.5, True)
    assert pinned[0] == 0 and pinned[2] == 0 and np.all(np.isneginf(np.delete(pinned, [0, 2])))


def test_roster_eviction_worked_example():
    # E = 4, m = 2, delta = 1, top-1.  Usage (5, 1, 0, 0): barrier, R = {0, 1}.
    # Logits (0, 0, 2.5, 0): expert 2 beats the members by 2.5 > 2 delta and
    # is selected, but with usage 1 it ties member 1 and the lower id stays;
    # a second such step gives it usage 2 and evicts expert 1.
    wr = np.eye(4)
    x = np.array([[0.0, 0.0, 2.5, 0.0]])
    u = np.array([[5, 1, 0, 0]])
    ids, w, lb, u1 = O.route_roster(x, wr, None, u, None, m=2, delta=1.0, top_k=1,
                                    norm_topk=False)
    assert ids[0, 0] == 2
    np.testing.assert_allclose(lb[0], [1.0, 1.0, 1.5, -1.0])
    np.testing.assert_array_equal(u1, [[5, 1, 1, 0]])
    np.testing.assert_array_equal(O.roster(u1[0], 2), [0, 1])
    np.testing.assert_allclose(w[0, 0], math.exp(1.5) / (2 * math.e + math.exp(1.5) + math.exp(-1)))
    ids, _, _, u2 = O.route_roster(x, wr, None, u1, None, m=2, delta=1.0, top_k=1,
                                   norm_topk=False)
    assert ids[0, 0] == 2
    np.testing.assert_array_equal(O.roster(u2[0], 2), [0, 2])
    # a gap below 2 delta does not get through
    ids, *_ = O.route_roster(np.array([[0.0, 0.0, 1.9, 0.0]]), wr, None, u, None, m=2,
                             delta=1.0, top_k=1, norm_topk=False)
    assert ids[0, 0] == 0


@pytest.mark.parametrize("norm", [False, True])
def test_roster_without_bias_is_the_plain_router(norm):
    L = _rand_layer(60, T=5, H=16, E=9, d=4)
    rng = np.random.default_rng(61)
    usage = rng.integers(0, 4, size=(5, 9))
    usage[0] = 0                                        # a fresh sequence
    ids0, w0, _, _ = O.route(L["x"].astype(np.float64), L["wr"].astype(np.float64), L["bias"], 3, norm)
    ids, w, _, new = O.route_roster(L["x"].astype(np.float64), L["wr"].astype(np.float64),
                                    L["bias"], usage, None, m=4, delta=0.0, top_k=3, norm_topk=norm)
    np.testing.assert_array_equal(ids, ids0)
    np.testing.assert_allclose(w, w0, rtol=1e-15)
    for t in range(5):                                  # one count per selection
        d = new[t] - usage[t]
        assert d.sum() == 3 and set(np.nonzero(d)[0]) == set(ids[t])
    # exploration (fewer than m used) ignores delta
    few = np.zeros((5, 9), dtype=np.int64)
    few[:, 0] = 2
    ids, w, _, _ = O.route_roster(L["x"].astype(np.float64), L["wr"].astype(np.float64),
                                  L["bias"], few, None, m=4, delta=5.0, top_k=3, norm_topk=norm)
    np.testing.assert_array_equal(ids, ids0)


def test_roster_selection_brute_force():
    # the top-k set maximises the sum of biased logits over all k-subsets
    L = _rand_layer(62, T=6, H=16, E=7, d=4)
    rng = np.random.default_rng(63)
    usage = rng.integers(0, 5, size=(6, 7))
    ids, _, lb, _ = O.route_roster(L["x"], L["wr"], None, usage, None, m=3, delta=0.3,
                                   top_k=2, norm_topk=False)
    xf, wf = L["x"].astype(np.float64), L["wr"].astype(np.float64)
    for t in range(6):
        bias = [0.0] * 7
        used = sum(1 for e in range(7) if usage[t, e] > 0)
        if used >= 3:
            best3 = sorted(range(7), key=lambda e: (-usage[t, e], e))[:3]
            bias = [0.3 if e in best3 else -0.3 for e in range(7)]
        score = [sum(xf[t, h] * wf[e, h] for h in range(16)) + bias[e] for e in range(7)]
        best = max(itertools.combinations(range(7), 2), key=lambda s: sum(score[e] for e in s))
        assert set(ids[t]) == set(best)


def test_roster_working_set_stays_at_m():
    # once 2 delta exceeds every row's logit range, a sequence in the barrier
    # phase never selects a non-member: its working set stays at m
    rng = np.random.default_rng(64)
    E, H, m, k = 16, 32, 4, 2
    wr = rng.standard_normal((E, H)) / np.sqrt(H)
    usage = np.zeros((3, E), dtype=np.int64)
    free = np.zeros((3, E), dtype=np.int64)
    for step in range(60):
        x = rng.standard_normal((3, H))
        _, _, lb, usage = O.route_roster(x, wr, None, usage, None, m=m, delta=50.0, top_k=k,
                                         norm_topk=True)
        _, _, _, free = O.route_roster(x, wr, None, free, None, m=m, delta=0.0, top_k=k,
                                       norm_topk=True)
    for t in range(3):
        assert np.count_nonzero(usage[t]) <= m + k - 1      # m reached inside one step at most
        assert np.count_nonzero(free[t]) > m + k
    # ... and the experts it keeps using are exactly its roster
    for t in range(3):
        assert set(np.nonzero(usage[t])[0]) >= set(O.roster(usage[t], m))


def test_roster_pinned_rows_stay_inside():
    L = _rand_layer(65, T=4, H=16, E=8, d=4)
    usage = np.array([[9, 0, 4, 0, 1, 0, 0, 0], [0] * 8, [1, 1, 1, 1, 1, 1, 1, 1],
                      [0, 0, 0, 0, 0, 0, 3, 3]])
    pinned = np.array([True, True, True, False])
    ids, w, _, _ = O.route_roster(L["x"], L["wr"], None, usage, pinned, m=3, delta=0.1, top_k=2,
                                  norm_topk=False)
    l = L["x"].astype(np.float64) @ L["wr"].astype(np.float64).T
    for t in range(3):
        R = O.roster(usage[t], 3)
        assert set(ids[t]) <= set(R)
        z = sum(math.exp(l[t, e]) for e in R)          # softmax over the roster only
        for s in range(2):
            assert math.isclose(w[t, s], math.exp(l[t, ids[t, s]]) / z, rel_tol=1e-12)


# ------------------------------------------------------------ residual stream

def _bf16_value(bits):
    return float(np.array([int(bits) << 16], dtype=np.uint32).view(np.float32)[0])


def test_residual_stream_worked_ties():
    one = np.array([0x3F80], dtype=np.uint16)          # 1.0 in bf16; its ulp is 2^-7
    cases = [(2.0 ** -8, 0x3F80),                      # exactly half an ulp: tie, to even (1.0)
             (3 * 2.0 ** -8, 0x3F82),                  # 1.5 ulp: tie, to even (1 + 2^-6)
             (2.0 ** -8 + 2.0 ** -20, 0x3F81),         # just above half: up
             (-2.0 ** -9, 0x3F80),                     # below 1 by a quarter of 1's lower ulp
             (1.0, 0x4000)]
    for y, want in cases:
        got = O.residual_stream(one, np.array([y], dtype=np.float32), "bf16")
        assert got[0] == want, (y, hex(int(got[0])), hex(want))
    f = O.residual_stream(np.array([1.5], np.float32), np.array([2.25], np.float32), "f32")
    assert f[0] == np.float32(3.75)


def test_residual_stream_is_nearest_bf16():
    # brute force: the result is a bf16 value nearest to the float32 sum, and
    # on an exact tie the one with an even last mantissa bit
    rng = np.random.default_rng(70)
    x = (rng.integers(0, 1 << 16, size=4000, dtype=np.uint32) & 0x7F7F).astype(np.uint16)
    x[x == 0] = 0x3F80
    y = rng.standard_normal(4000).astype(np.float32)
    got = O.residual_stream(x, y, "bf16")
    for i in range(4000):
        s = float(np.float32(_bf16_value(x[i])) + np.float32(y[i]))
        g = int(got[i])
        err = abs(_bf16_value(g) - s)
        for nb in (g - 1, g + 1):
            alt = abs(_bf16_value(nb & 0xFFFF) - s)
            assert err < alt or (err == alt and g % 2 == 0), (i, hex(g), s)
