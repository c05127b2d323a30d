"""Exact ties on the GPU, checked for equality with the oracle's tie rules.

The header promises: equal router logits pick the lower expert id (slot
order too), equal |h| keep the lower neuron index, and -0 scores equal +0.
The selection-window rule of tests/parity.py accepts either choice at a
tie, and random normal inputs never produce one, so these cases build exact
ties on purpose and require the GPU's ids and kept lists to equal the
oracle's exactly:

* a token of all zeros: every logit is 0 (no router bias), so its experts
  are 0 .. top_k-1 with weight 1/E each, every h is +-0, so its kept
  neurons are 0 .. k-1, and its output row is 0;
* up rows zeroed for three neurons in four: those h are +0 or -0 (the sign
  of silu(g)), and with k above the nonzero count the boundary falls among
  the zeros;
* gate/up rows duplicated so that five neurons share one |h| straddling
  the k-th place: the two lowest-index copies are kept;
* router rows duplicated so that three experts share the last selected
  logit (the lowest id wins the slot), and two experts share the top one
  (both selected, the lower id in the first slot).

Each duplicated value is checked in the oracle to sit at least 1e-3
relative from every other score, so fp32 rounding cannot reorder it.
"""
import functools
import sys

import numpy as np
import pytest
import torch

import moe_synth as S
import oracle
from oracle import moe_oracle as O
from sparse_moe_expert_route_amd import binding as B

from parity import DeviceLayer, LayerInputs, check_grouping, compare_layer, to_dev

pytestmark = pytest.mark.gpu
SP, DN = B.MOE_PATH_SPARSE, B.MOE_PATH_DENSE
GAP = 1e-3


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def _shape(name):
    return S.LAYERS[name]


@functools.lru_cache(maxsize=2)
def _base(name):
    return LayerInputs(_shape(name), seed=0)


def _copy_inputs(name):
    """A private LayerInputs whose host arrays may be modified."""
    base = _base(name)
    inp = LayerInputs.__new__(LayerInputs)
    inp.shape, inp.seed = base.shape, base.seed
    inp.w_router = base.w_router.copy()
    inp.bias = base.bias
    inp.wg, inp.wu, inp.wd = base.wg.copy(), base.wu.copy(), base.wd.copy()
    inp.shared = None
    return inp


def _f64(a, dtype):
    return oracle.to_f64(a, dtype)


def _run_layer_entry(dev, x_host, k):
    """moe_layer_sparse (the in-kernel expert selection at T <= 2)."""
    sh = dev.inp.shape
    T = x_host.shape[0]
    x = to_dev(x_host)
    R = B.Routing.allocate(T, sh.top_k, sh.n_experts)
    y = torch.full((T, sh.hidden), float("nan"), device="cuda")
    idx = torch.full((T * sh.top_k, k), -1, dtype=torch.int32, device="cuda")
    ws = torch.empty(B.moe_layer_workspace_size(dev.desc, T, k), dtype=torch.uint8, device="cuda")
    B.moe_layer_sparse(dev.desc, T, k, x, dev.w_router, dev.bias, *dev.w, R, y, 0, idx, ws)
    torch.cuda.synchronize()
    return dict(T=T, k=k, ids=R.topk_ids.cpu().numpy()[:T], w=R.topk_w.cpu().numpy()[:T],
                offsets=R.expert_offsets.cpu().numpy(), pairs=R.pair_by_expert.cpu().numpy(),
                active=R.active_experts.cpu().numpy(), n_active=int(R.n_active.cpu()[0]),
                idx=idx.cpu().numpy(), y=y.cpu().numpy())


def _run(dev, x, k, entry):
    if entry == "layer":
        return _run_layer_entry(dev, x, k)
    return dev.run(x, k, DN if entry == "dense" else SP)


def _oracle_forced(inp, x, got, k, score):
    sh = inp.shape
    return oracle.moe_layer(x, inp.w_router, inp.bias, inp.wg, inp.wu, inp.wd, top_k=sh.top_k,
                            norm_topk=sh.norm_topk, k_keep=k, dtype=sh.dtype,
                            forced_ids=got["ids"], score=score)


def _assert_masks_equal(got, ref, pairs, k, what):
    K = got["ids"].shape[1]
    for (t, s) in pairs:
        g = got["idx"][t * K + s, :k]
        np.testing.assert_array_equal(g, ref.keep[(t, s)], err_msg=f"{what}: kept list t={t} s={s}")


# ------------------------------------------------------------------ all-zero tokens

ZERO_CASES = [("olmoe-like", 1, "layer"), ("olmoe-like", 1, "sparse"), ("olmoe-like", 3, "sparse"),
              ("olmoe-like", 8, "sparse"), ("olmoe-like", 8, "dense"), ("olmoe-like", 80, "dense"),
              ("olmoe-like", 3, "gate"), ("olmoe-like", 8, "gate"), ("tiny-f32", 4, "sparse"),
              ("tiny-f32", 8, "dense"), ("tiny-f32", 2, "layer")]


@pytest.mark.parametrize("name,T,entry", ZERO_CASES)
def test_zero_token(name, T, entry):
    inp = _base(name)
    sh = inp.shape
    score = "gate" if entry == "gate" else "swiglu"
    dev = _device(name, score)
    k = O.keep_count(0.9, sh.d_ff)
    x = inp.tokens(T, 5)
    zero_rows = [0] if T < 3 else [0, 2]
    x[zero_rows] = 0
    say(f"[case] zero token {name} T={T} entry={entry} rows={zero_rows}")
    got = _run(dev, x, k, entry)
    check_grouping(got, sh.n_experts, sh.top_k)
    for t in zero_rows:
        np.testing.assert_array_equal(got["ids"][t], np.arange(sh.top_k),
                                      err_msg=f"equal logits must pick the lowest ids (t={t})")
        np.testing.assert_allclose(got["w"][t], np.full(sh.top_k, 1.0 / sh.n_experts), rtol=1e-6)
        for s in range(sh.top_k):
            np.testing.assert_array_equal(got["idx"][t * sh.top_k + s, :k], np.arange(k),
                                          err_msg=f"all-zero scores keep the lowest ids (t={t} s={s})")
        assert np.all(got["y"][t] == 0), f"zero token t={t} gave a nonzero output"
    err = compare_layer(inp, x, got, k, score=score)
    say(f"   rel_l2={err:.3e}")


@functools.lru_cache(maxsize=2)
def _device(name, score):
    return DeviceLayer(_base(name), score)


# ------------------------------------------------------------------ signed zeros

SIGNED_CASES = [(1, "sparse"), (1, "layer"), (3, "sparse"), (8, "sparse"), (8, "dense"),
                (80, "dense"), (3, "gate"), (8, "gate")]


@functools.lru_cache(maxsize=2)
def _signed_zero_layer(score):
    # three neurons in four get a zero up row (SwiGLU score: h = silu(g) * 0 =
    # +0 or -0) or a zero gate row (gate score: silu(0) = 0)
    inp = _copy_inputs("olmoe-like")
    d = inp.shape.d_ff
    zero = (np.arange(d) % 4) != 1
    if score == "swiglu":
        inp.wu[:, zero, :] = 0
    else:
        inp.wg[:, zero, :] = 0
    return inp, DeviceLayer(inp, score)


@pytest.mark.parametrize("T,entry", SIGNED_CASES)
def test_signed_zero_scores_at_the_boundary(T, entry):
    score = "gate" if entry == "gate" else "swiglu"
    inp, dev = _signed_zero_layer(score)
    sh = inp.shape
    k = O.keep_count(0.5, sh.d_ff)          # 512 kept, 256 nonzero scores per pair
    x = inp.tokens(T, 6)
    say(f"[case] signed zeros T={T} entry={entry} k={k}")
    got = _run(dev, x, k, entry)
    ref = _oracle_forced(inp, x, got, k, score)
    nz = np.arange(sh.d_ff)[np.arange(sh.d_ff) % 4 == 1]
    for (t, s), keep in ref.keep.items():
        # the oracle's own statement: every nonzero neuron, then the lowest-index zeros
        sc = ref.h[(t, s)]
        assert np.count_nonzero(sc) == len(nz) and set(nz) <= set(keep.tolist())
        if score == "swiglu":
            assert np.any(np.signbit(sc[sc == 0])) and np.any(~np.signbit(sc[sc == 0]))
    _assert_masks_equal(got, ref, list(ref.keep), k, "signed zeros")
    err = compare_layer(inp, x, got, k, score=score)
    say(f"   rel_l2={err:.3e}")


# ------------------------------------------------------------------ duplicated gate/up rows

def _isolated(v, sel, others):
    """|v[sel]| (all equal) sits at least GAP relative from every other |v|."""
    a = np.abs(v)
    val = a[sel[0]]
    rest = np.delete(a, sel)
    return np.all(np.abs(rest - val) > GAP * val)


@functools.lru_cache(maxsize=2)
def _straddle_layer(score):
    """Duplicate one neuron's gate (and, for the SwiGLU score, up) row into
    four low-scoring neurons of token 0's first expert, with the value at
    rank k-1 (1-based): k-2 scores lie above it, so the two lowest-index of
    the five copies are kept.  Returns (inputs, device layer, token batch
    of 8, expert, copies, k)."""
    base = _base("olmoe-like")
    sh = base.shape
    k = O.keep_count(0.9, sh.d_ff)
    x = base.tokens(8, 8)
    xf = _f64(x, sh.dtype)
    ids, _, _, _ = O.route(xf, _f64(base.w_router, sh.dtype), None, sh.top_k, sh.norm_topk)
    for s in range(sh.top_k):                   # first slot that gives an isolated tie
        e = int(ids[0, s])
        wg, wu = _f64(base.wg[e], sh.dtype), _f64(base.wu[e], sh.dtype)
        v = O.expert_scores_batch(xf[:1], wg, wu, score)[0]
        order = np.lexsort((np.arange(sh.d_ff), -np.abs(v)))
        src = int(order[k - 2])
        low = [int(j) for j in order[::-1][:64]]           # the lowest-scoring neurons
        below = [j for j in low if j < src][:2]
        above = [j for j in low if j > src][:4 - len(below)]
        dst = below + above
        if len(dst) != 4:
            continue
        inp = _copy_inputs("olmoe-like")
        for j in dst:
            inp.wg[e, j] = inp.wg[e, src]
            if score == "swiglu":
                inp.wu[e, j] = inp.wu[e, src]
        v2 = O.expert_scores_batch(xf[:1], _f64(inp.wg[e], sh.dtype), _f64(inp.wu[e], sh.dtype),
                                   score)[0]
        copies = sorted([src] + dst)
        if not _isolated(v2, copies, None):
            continue
        n_gt = int(np.sum(np.abs(v2) > np.abs(v2[src])))
        assert n_gt == k - 2, (n_gt, k)
        return inp, DeviceLayer(inp, score), x, e, copies, k
    raise AssertionError("no slot of token 0 gives an isolated tie")


STRADDLE_CASES = [(1, "sparse"), (1, "layer"), (2, "layer"), (3, "sparse"), (8, "sparse"),
                  (8, "dense"), (80, "dense"), (1, "gate"), (8, "gate")]


@pytest.mark.parametrize("T,entry", STRADDLE_CASES)
def test_duplicated_rows_straddle_the_kth_score(T, entry):
    score = "gate" if entry == "gate" else "swiglu"
    inp, dev, x8, e, copies, k = _straddle_layer(score)
    sh = inp.shape
    x = x8[:T] if T <= 8 else np.concatenate([x8, inp.tokens(T - 8, 9)])
    say(f"[case] duplicated rows T={T} entry={entry} expert={e} copies={copies}")
    got = _run(dev, x, k, entry)
    ref = _oracle_forced(inp, x, got, k, score)
    slot = [s for s in range(sh.top_k) if int(got["ids"][0, s]) == e]
    assert slot, "token 0 must still route to the modified expert"
    keep = ref.keep[(0, slot[0])]
    assert sorted(set(copies) & set(keep.tolist())) == copies[:2]   # the oracle's rule
    _assert_masks_equal(got, ref, [(0, slot[0])], k, "straddling duplicates")
    err = compare_layer(inp, x, got, k, score=score)
    say(f"   rel_l2={err:.3e}")


# ------------------------------------------------------------------ equal router logits

@functools.lru_cache(maxsize=1)
def _router_tie_layer():
    """Token 0: copy the top expert's router row into an unselected expert
    (a tie inside the selection: both kept, the lower id first), which
    pushes every later expert down one place; then copy the expert that now
    holds the last place (the second-to-last before) into one lower and one
    higher unselected expert (a three-way tie at the boundary: the lowest id
    takes the slot).  Returns (inputs, device layer, token batch, the two
    tie sets)."""
    base = _base("olmoe-like")
    sh = base.shape
    x = base.tokens(8, 12)
    xf = _f64(x, sh.dtype)
    ids, _, l, _ = O.route(xf, _f64(base.w_router, sh.dtype), None, sh.top_k, sh.norm_topk)
    sel = [int(e) for e in ids[0]]
    last, top = sel[-2], sel[0]
    free = [e for e in range(sh.n_experts) if e not in sel]
    lo = [e for e in free if e < last]
    hi = [e for e in free if e > last]
    assert lo and hi
    e_lo, e_hi = lo[0], hi[-1]
    e_top = [e for e in free if e not in (e_lo, e_hi)][0]
    inp = _copy_inputs("olmoe-like")
    inp.w_router[e_lo] = inp.w_router[last]
    inp.w_router[e_hi] = inp.w_router[last]
    inp.w_router[e_top] = inp.w_router[top]
    l2 = _f64(x, sh.dtype)[:1] @ _f64(inp.w_router, sh.dtype).T
    for group in ([e_lo, last, e_hi], [top, e_top]):
        assert _isolated(l2[0], group, None), "tie value too close to another logit"
    return inp, DeviceLayer(inp), x, (e_lo, last, e_hi), (top, e_top)


@pytest.mark.parametrize("T,entry", [(1, "sparse"), (1, "layer"), (2, "layer"), (8, "sparse"),
                                     (300, "sparse")])
def test_equal_router_logits_pick_the_lower_id(T, entry):
    inp, dev, x8, edge, inner = _router_tie_layer()
    sh = inp.shape
    x = x8[:T] if T <= 8 else np.concatenate([x8, inp.tokens(T - 8, 13)])
    k = O.keep_count(0.9, sh.d_ff)
    say(f"[case] router ties T={T} entry={entry} edge={edge} inner={inner}")
    got = _run(dev, x, k, entry)
    ids0, w0, _, _ = O.route(_f64(x[:1], sh.dtype), _f64(inp.w_router, sh.dtype), None, sh.top_k,
                             sh.norm_topk)
    g = [int(e) for e in got["ids"][0]]
    np.testing.assert_array_equal(g, ids0[0], err_msg="router ties: ids and slot order")
    assert min(edge) in g and sorted(set(edge) - {min(edge)}) == sorted(set(edge) - set(g))
    a, b = sorted(inner)
    assert g.index(a) + 1 == g.index(b), "equal logits: lower id in the earlier slot"
    assert got["w"][0][g.index(a)] == got["w"][0][g.index(b)], "equal logits, equal weights"
    np.testing.assert_allclose(got["w"][0], w0[0], rtol=1e-4, atol=1e-7)
    check_grouping(got, sh.n_experts, sh.top_k)
    err = compare_layer(inp, x, got, k)
    say(f"   rel_l2={err:.3e}")
