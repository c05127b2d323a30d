"""CPU oracle of the intra-expert-sparse MoE decode layer.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, header,
table or helper with the HIP library; its only shared dependency is the
seeded input generator ``moe_synth`` (which holds no arithmetic of the
method).

It is a plain, slow, float64 restatement of what the layer computes.
Citations name sections of the page "Uncovering Intra-expert Activation
Sparsity for Efficient Mixture-of-Expert Model Execution" (gist.science
explainer of the paper by Park, Kim, Gu, Stoica and Cheung), called "the
page" below.

Layer definition (one token t):

    l[e]   = x_t . W_r[e] + b[e]                 router logits
    S_t    = the top_k experts by l (ties: lower e)
    p      = softmax(l) over all E; w_e = p_e (e in S_t),
             divided by sum_{S_t} p when norm_topk
    g, u   = W_g^e x_t, W_u^e x_t;  h = silu(g) * u     (dense, SwiGLU)
    K_t,e  = the k_keep neurons of largest |h_j| (ties: lower j)
    y_t    = sum_{e in S_t} w_e * sum_{j in K_t,e} h_j W_d^e[j, :]
             + sum over shared experts e' (weight 1, own mask) of the same

The sparse down projection reaches exactly (up to rounding order) the dense
down projection of the masked activation, so this file writes that
definition out directly and touches only kept W_d rows.

Gate-score variant (score="gate"), the page's own split (technical summary,
Methodology, vLLM implementation: the gate projection alone runs densely
and produces the activation scores; the fused up-down projection then
gathers only the active neurons' weights):

    s      = silu(W_g^e x_t)                      dense gate, the scores
    K_t,e  = the k_keep neurons of largest |s_j| (ties: lower j)
    h_j    = s_j * (W_u^e[j, :] . x_t)   for j in K_t,e only
    y_t    = as above, with this h on K_t,e

Only kept W_u and W_d rows are read.  With k_keep = d_ff both variants are
the dense SwiGLU MoE.

Threshold variant (the page's literal masking: technical summary,
Methodology, activation masking by a threshold in one O(n) pass, without a
top-k sort).  The page does not say how the threshold is chosen; the reading
here is a per-expert threshold tau_e calibrated offline so that the target
sparsity of the experiments holds on calibration tokens.  It replaces the
exact count:

    K_t,e  = { j : |h_j| > tau_e }                 (variable count per pair)
    tau_e  = the (c + 1)-th largest of the m calibration scores |h| of
             expert e (its calibration pairs x d_ff neurons), c = ceil((1 - s) m);
             the layer-wide value for an expert with no calibration pair

Every function below is pinned by tests (tests/test_oracle_pins.py) against
closed forms, brute force, library routines or invariants; none is
"parity unpinned".
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional, Sequence, Tuple

import numpy as np
import torch


# ---------------------------------------------------------------- inputs

def to_f64(a, dtype: str) -> np.ndarray:
    """Exact float64 value of an input tensor.

    ``dtype`` is "f32" (float32 array) or "bf16" (uint16 bit patterns:
    the value is the float32 whose upper 16 bits are the pattern).  bf16
    rounding is part of the input, never an error of the method."""
    a = np.asarray(a)
    if dtype == "f32":
        return a.astype(np.float64)
    if dtype == "bf16":
        if a.dtype != np.uint16:
            raise TypeError("bf16 inputs are passed as uint16 bit patterns")
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def _check_finite(name, a):
    if not np.all(np.isfinite(a)):
        raise ValueError(f"oracle: {name} holds NaN or Inf; such inputs are undefined")


# ---------------------------------------------------------------- router

def router_logits(x: np.ndarray, w_router: np.ndarray,
                  bias: Optional[np.ndarray]) -> np.ndarray:
    """l[t, e] = sum_h x[t, h] * W_r[e, h] + b[e]  ->  [T, E].

    The router is kept unchanged by the method (the page, technical summary,
    Methodology: vLLM implementation keeps the router logic).  A plain
    linear router with an optional additive per-expert bias."""
    l = x @ w_router.T
    if bias is not None:
        l = l + np.asarray(bias, dtype=np.float64)[None, :]
    return l


def softmax(l: np.ndarray) -> np.ndarray:
    """Row softmax over the last axis: p_e = exp(l_e) / sum_e' exp(l_e')."""
    m = np.max(l, axis=-1, keepdims=True)
    z = np.exp(l - m)
    return z / np.sum(z, axis=-1, keepdims=True)


def top_experts(l_row: np.ndarray, top_k: int) -> np.ndarray:
    """The top_k experts of one token by logit, in descending logit order;
    equal logits go to the lower expert id (stable order of (-l, e)).

    Selecting on logits selects the same set as selecting on softmax
    probabilities, since softmax is monotone."""
    E = l_row.shape[0]
    order = sorted(range(E), key=lambda e: (-float(l_row[e]), e))
    return np.asarray(order[:top_k], dtype=np.int64)


def route(x, w_router, bias, top_k: int, norm_topk: bool):
    """Router top-k with softmax weights.

    Returns (ids [T, top_k] int64 in descending-logit slot order,
    weights [T, top_k] float64, logits [T, E], probs [T, E])."""
    l = router_logits(x, w_router, bias)
    p = softmax(l)
    T = l.shape[0]
    ids = np.zeros((T, top_k), dtype=np.int64)
    w = np.zeros((T, top_k), dtype=np.float64)
    for t in range(T):
        ids[t] = top_experts(l[t], top_k)
        w[t] = p[t, ids[t]]
        if norm_topk:
            w[t] = w[t] / np.sum(w[t])
    return ids, w, l, p


# ---------------------------------------------------------------- expert FFN

def keep_count(sparsity: float, d_ff: int) -> int:
    """Kept neurons per (token, expert): ceil((1 - s) * d_ff), clamped to
    [0, d_ff].

    The page zeroes the lowest-scoring fraction s of each selected expert's
    neurons (technical summary, Methodology: empirical analysis; Results:
    sparsity levels).  A 1e-9 guard stops float noise from rounding an exact
    integer up (naive float gives 301 for s=0.7, d_ff=1000)."""
    k = math.ceil((1.0 - float(sparsity)) * d_ff - 1e-9)
    return max(0, min(d_ff, k))


def silu(z: np.ndarray) -> np.ndarray:
    """silu(z) = z * sigmoid(z) = z / (1 + exp(-z))."""
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def expert_activation(x_t: np.ndarray, w_gate_e: np.ndarray,
                      w_up_e: np.ndarray) -> np.ndarray:
    """h = silu(W_g x) * (W_u x) for one token and one expert  ->  [d_ff].

    Gate and up run densely for every selected (token, expert) pair; their
    SwiGLU product is the activation whose magnitude scores the neurons (the
    page, technical summary, Methodology: vLLM implementation, gate
    projection run densely to produce activation scores)."""
    g = w_gate_e @ x_t
    u = w_up_e @ x_t
    return silu(g) * u


def gate_scores(x_t: np.ndarray, w_gate_e: np.ndarray) -> np.ndarray:
    """s = silu(W_g x) for one token and one expert  ->  [d_ff].

    In the page's own split only the gate projection runs densely; its
    activation is the score that decides which neurons stay (technical
    summary, Methodology: vLLM implementation, gate projection)."""
    return silu(w_gate_e @ x_t)


def sparse_up(x_t: np.ndarray, s: np.ndarray, keep: np.ndarray,
              w_up_e: np.ndarray) -> np.ndarray:
    """h_j = s_j * (W_u[j, :] . x_t) for the kept neurons only  ->  [len(keep)].

    The up projection gathers only the active neurons' rows (technical
    summary, Methodology: fused up-down projection gathers only the active
    neurons' weights); the rest of W_u is never read."""
    if keep.size == 0:
        return np.zeros(0, dtype=np.float64)
    return s[keep] * (w_up_e[keep, :] @ x_t)


def kept_neurons(h: np.ndarray, k: int) -> np.ndarray:
    """The k neurons of largest |h| (ties: lower index), ascending.

    The lowest-scoring activations inside an expert are set to zero (the
    page, technical summary, Methodology: empirical analysis and activation
    masking).  -0 and +0 score equal."""
    d = h.shape[0]
    a = np.abs(np.asarray(h, dtype=np.float64))
    # a stable sort on (-|h|, j): the last key given to lexsort is the primary one
    order = np.lexsort((np.arange(d), -a))
    return np.sort(order[:max(0, min(k, d))]).astype(np.int64)


def threshold_neurons(h: np.ndarray, tau: float) -> np.ndarray:
    """The neurons with |h_j| > tau, ascending (a variable count).

    The page's literal masking: one pass comparing every activation with a
    threshold, with no sort (technical summary, Methodology: activation
    masking).  -0 and +0 score equal."""
    return np.nonzero(np.abs(h) > tau)[0].astype(np.int64)


def calibrated_threshold(scores: np.ndarray, sparsity: float) -> float:
    """tau such that 'keep |h| > tau' keeps c = ceil((1 - s) m) of the m
    calibration scores when they are distinct: the (c + 1)-th largest score
    (the largest one not kept); -1 when c = m (keep everything)."""
    v = np.sort(np.abs(np.asarray(scores, dtype=np.float64)).ravel())[::-1]
    m = v.size
    c = keep_count(sparsity, m)
    return -1.0 if c >= m else float(v[c])


def sparse_down(h: np.ndarray, keep: np.ndarray, w_down_e: np.ndarray) -> np.ndarray:
    """sum_{j in keep} h_j * W_d[j, :]  ->  [H].

    Only the kept neurons' down-projection rows are read; the zeroed neurons
    are never loaded (the page, "how it runs: skip-list system": unneeded
    neurons are not even loaded; technical summary, fused up-down projection
    gathers only the active neurons' weights)."""
    if keep.size == 0:
        return np.zeros(w_down_e.shape[1], dtype=np.float64)
    return h[keep] @ w_down_e[keep, :]


# ---------------------------------------------------------------- layer

@dataclass
class LayerResult:
    y: np.ndarray                       # [T, H] float64, routed + shared
    y_routed: np.ndarray                # [T, H]
    y_shared: np.ndarray                # [T, H]
    ids: np.ndarray                     # [T, top_k]
    weights: np.ndarray                 # [T, top_k]
    logits: np.ndarray                  # [T, E]
    probs: np.ndarray                   # [T, E]
    h: Dict[Tuple[int, int], np.ndarray] = field(default_factory=dict)        # (t, slot) -> scores [d_ff]
    keep: Dict[Tuple[int, int], np.ndarray] = field(default_factory=dict)     # (t, slot) -> idx
    h_shared: Dict[Tuple[int, int], np.ndarray] = field(default_factory=dict)     # (t, j)
    keep_shared: Dict[Tuple[int, int], np.ndarray] = field(default_factory=dict)  # (t, j)


def _select(scores, k_keep, tau, forced):
    if forced is not None:
        return np.asarray(forced, dtype=np.int64)
    if tau is not None:
        return threshold_neurons(scores, tau)
    return kept_neurons(scores, k_keep)


def expert_scores_batch(X: np.ndarray, w_gate_e: np.ndarray, w_up_e: np.ndarray,
                        score: str) -> np.ndarray:
    """The selection scores of several tokens of one expert at once  ->  [n, d_ff].

    Row i equals expert_activation(X[i], ...) (score="swiglu") or
    gate_scores(X[i], ...) (score="gate"): the same definition, with the
    expert's projections of its tokens taken as one matrix product."""
    g = X @ w_gate_e.T
    if score == "gate":
        return silu(g)
    if score == "swiglu":
        return silu(g) * (X @ w_up_e.T)
    raise ValueError(f"unknown score {score!r}")


def _pair_output(x_t, wg, wu, wd, k_keep, forced, score, tau=None, sc=None):
    """One (token, expert) pair: (its contribution before the routing
    weight [H], the selection scores [d_ff], the kept set).  ``tau`` (the
    expert's calibrated threshold) replaces the exact count when given;
    ``sc`` passes the pair's scores when they were computed with the other
    tokens of the expert (expert_scores_batch)."""
    if score == "swiglu":
        h = expert_activation(x_t, wg, wu) if sc is None else sc
        keep = _select(h, k_keep, tau, forced)
        return sparse_down(h, keep, wd), h, keep
    if score == "gate":
        sc = gate_scores(x_t, wg) if sc is None else sc
        keep = _select(sc, k_keep, tau, forced)
        h = np.zeros_like(sc)
        h[keep] = sparse_up(x_t, sc, keep, wu)
        return sparse_down(h, keep, wd), sc, keep
    raise ValueError(f"unknown score {score!r}")


def routed_experts(x, ids, weights, w_gate, w_up, w_down, k_keep, dtype,
                   forced_keep=None, keep_h=True, score="swiglu", thresholds=None):
    """Routed contribution sum_{slot} w * sum_{j in K} h_j W_d^e[j, :].

    Pairs are visited expert by expert so each expert's weights are
    converted once.  ``forced_keep[(t, slot)]`` replaces the computed kept
    set (used when a tested implementation's selection differs only on
    scores inside the comparison window).  Returns (y [T, H], scores,
    keep); the scores are h itself for score="swiglu" and silu(W_g x) for
    score="gate"."""
    T, H = x.shape
    y = np.zeros((T, H), dtype=np.float64)
    hs, keeps = {}, {}
    by_expert: Dict[int, list] = {}
    for t in range(T):
        for s in range(ids.shape[1]):
            by_expert.setdefault(int(ids[t, s]), []).append((t, s))
    for e in sorted(by_expert):
        wg, wu, wd = (to_f64(w[e], dtype) for w in (w_gate, w_up, w_down))
        pairs = by_expert[e]
        scores = expert_scores_batch(x[[t for t, _ in pairs]], wg, wu, score)
        for i, (t, s) in enumerate(pairs):
            forced = forced_keep.get((t, s)) if forced_keep is not None else None
            tau = None if thresholds is None else float(thresholds[e])
            out, sc, keep = _pair_output(x[t], wg, wu, wd, k_keep, forced, score, tau, scores[i])
            y[t] += weights[t, s] * out
            if keep_h:
                hs[(t, s)] = sc
            keeps[(t, s)] = keep
    return y, hs, keeps


def shared_experts(x, w_gate, w_up, w_down, n_shared, k_keep, dtype,
                   forced_keep=None, keep_h=True, score="swiglu", thresholds=None):
    """Always-on shared experts: every token, weight 1, each expert with its
    own per-(token, expert) mask of k_keep neurons.

    The page treats shared experts apart from routed ones (technical
    summary, Methodology: empirical analysis; vLLM implementation keeps
    shared-expert execution); with k_keep = d_ff they run dense."""
    T, H = x.shape
    y = np.zeros((T, H), dtype=np.float64)
    hs, keeps = {}, {}
    for j in range(n_shared):
        wg, wu, wd = (to_f64(w[j], dtype) for w in (w_gate, w_up, w_down))
        scores = expert_scores_batch(x, wg, wu, score)
        for t in range(T):
            forced = forced_keep.get((t, j)) if forced_keep is not None else None
            tau = None if thresholds is None else float(thresholds[j])
            out, sc, keep = _pair_output(x[t], wg, wu, wd, k_keep, forced, score, tau, scores[t])
            y[t] += out
            if keep_h:
                hs[(t, j)] = sc
            keeps[(t, j)] = keep
    return y, hs, keeps


def moe_layer(x, w_router, bias, w_gate, w_up, w_down, *, top_k: int,
              norm_topk: bool, k_keep: int, dtype: str,
              shared: Optional[Sequence] = None, k_keep_shared: Optional[int] = None,
              forced_ids: Optional[np.ndarray] = None,
              forced_keep: Optional[dict] = None,
              forced_keep_shared: Optional[dict] = None,
              keep_h: bool = True, score: str = "swiglu",
              thresholds: Optional[np.ndarray] = None,
              thresholds_shared: Optional[np.ndarray] = None) -> LayerResult:
    """The whole layer for a token batch.

    x [T, H], w_router [E, H] and the expert weights (indexable by expert,
    each [d_ff, H] neuron-major) are in the layer's input dtype ("f32" arrays
    or "bf16" uint16 bit patterns); bias is float32 [E] or None.  ``shared``
    is (w_gate, w_up, w_down) of the shared experts or None.

    ``forced_ids`` replaces the routed expert sets (slot order as given);
    the weights are then the softmax probabilities of those experts, so a
    tested implementation whose selection differs from this one only on
    logits inside the comparison window can be scored exactly.

    ``score`` is "swiglu" (mask by |silu(g) * u|, gate and up dense) or
    "gate" (the page's own split: mask by |silu(g)|, up and down gathered
    for the kept neurons only).  LayerResult.h holds the selection scores.
    ``thresholds`` [E] (and ``thresholds_shared`` [n_shared]) switch the
    mask from the exact count k_keep to 'score > tau_e' (variable count)."""
    xf = to_f64(x, dtype)
    _check_finite("x", xf)
    wr = to_f64(w_router, dtype)
    ids, w, l, p = route(xf, wr, bias, top_k, norm_topk)
    if forced_ids is not None:
        ids = np.asarray(forced_ids, dtype=np.int64).reshape(ids.shape)
        w = np.take_along_axis(p, ids, axis=1)
        if norm_topk:
            w = w / np.sum(w, axis=1, keepdims=True)
    y_r, hs, keeps = routed_experts(xf, ids, w, w_gate, w_up, w_down, k_keep,
                                    dtype, forced_keep, keep_h, score, thresholds)
    T, H = xf.shape
    y_s = np.zeros((T, H))
    hs_s, keeps_s = {}, {}
    if shared is not None:
        n_sh = len(shared[0])
        ks = k_keep_shared if k_keep_shared is not None else shared[0][0].shape[0]
        y_s, hs_s, keeps_s = shared_experts(xf, shared[0], shared[1], shared[2],
                                            n_sh, ks, dtype, forced_keep_shared, keep_h, score,
                                            thresholds_shared)
    return LayerResult(y=y_r + y_s, y_routed=y_r, y_shared=y_s, ids=ids, weights=w,
                       logits=l, probs=p, h=hs, keep=keeps, h_shared=hs_s,
                       keep_shared=keeps_s)


def calibrate_thresholds(x, w_router, bias, w_gate, w_up, *, top_k: int, norm_topk: bool,
                         dtype: str, sparsity: float, score: str = "swiglu",
                         shared: Optional[Sequence] = None,
                         forced_ids=None) -> Tuple[np.ndarray, Optional[np.ndarray]]:
    """Per-expert thresholds from calibration tokens x [T, H]: each routed
    expert's tau is calibrated_threshold over the scores of every
    (calibration token routed to it, neuron) pair; an expert no token reaches
    takes the value over all routed scores.  Shared experts (every token)
    get their own.  The page masks by a threshold (technical summary,
    Methodology: activation masking) without saying how it is set; this
    calibration for the target sparsity is the reading taken here.
    ``forced_ids`` replaces the router's choice (for checking a run whose
    near-tied router logits broke the other way)."""
    xf = to_f64(x, dtype)
    _check_finite("x", xf)
    if forced_ids is None:
        ids, _, _, _ = route(xf, to_f64(w_router, dtype), bias, top_k, norm_topk)
    else:
        ids = np.asarray(forced_ids)
    E = len(w_gate)
    per = {e: [] for e in range(E)}
    for e in range(E):
        rows = [t for t in range(xf.shape[0]) if e in ids[t]]
        if not rows:
            continue
        wg = to_f64(w_gate[e], dtype)
        wu = to_f64(w_up[e], dtype)
        per[e].extend(expert_scores_batch(xf[rows], wg, wu, score))
    everything = [v for e in range(E) for v in per[e]]
    tau_all = calibrated_threshold(np.concatenate(everything), sparsity) if everything else -1.0
    tau = np.array([calibrated_threshold(np.concatenate(per[e]), sparsity) if per[e] else tau_all
                    for e in range(E)], dtype=np.float64)
    tau_sh = None
    if shared is not None:
        tau_sh = []
        for j in range(len(shared[0])):
            wg, wu = to_f64(shared[0][j], dtype), to_f64(shared[1][j], dtype)
            sc = expert_scores_batch(xf, wg, wu, score)
            tau_sh.append(calibrated_threshold(sc.ravel(), sparsity))
        tau_sh = np.array(tau_sh, dtype=np.float64)
    return tau, tau_sh


# ---------------------------------------------------------------- roster routing
# The roster rule of the page "Predatory MoE: Serving Mixture-of-Experts with
# a Sequence-Local Expert Roster" (technical summary, section 2, the roster
# routing rule), restated for one MoE layer at decode time.  Batch row t is
# one sequence; usage[t, e] counts how often that sequence has selected
# expert e at this layer so far.
#
# Readings (the page is silent on these):
#   * the roster R_t is the m experts with the largest usage, ties to the
#     lower expert id (the same tie rule as the router's);
#   * the bias is added to the router logits before the softmax and the
#     top-k, as any additive router bias ("score gap" of 2 delta);
#   * pinned rows keep only roster members selectable: a bias of 0 for
#     members and -inf for the others;
#   * every selection of the step adds one to the row's usage, in every
#     phase (pinned rows included).

def roster(usage_row: np.ndarray, m: int) -> np.ndarray:
    """R_t: the m most-used experts of one sequence (ties: lower id),
    ascending."""
    E = usage_row.shape[0]
    order = sorted(range(E), key=lambda e: (-int(usage_row[e]), e))
    return np.asarray(sorted(order[:m]), dtype=np.int64)


def roster_bias(usage_row: np.ndarray, m: int, delta: float, pinned: bool) -> np.ndarray:
    """The logit bias [E] of one sequence for this step.

    Exploration (fewer than m distinct experts used so far): no bias.
    Barrier (m or more used): +delta for roster members, -delta for the
    rest, so a non-member must beat a member by more than 2 delta.
    Pinned (serving after the prefix): decoding stays inside the roster."""
    E = usage_row.shape[0]
    R = roster(usage_row, m)
    member = np.zeros(E, dtype=bool)
    member[R] = True
    if pinned:
        return np.where(member, 0.0, -np.inf)
    if int(np.count_nonzero(usage_row > 0)) < m:
        return np.zeros(E)
    return np.where(member, float(delta), -float(delta))


def route_roster(x, w_router, bias, usage, pinned, *, m: int, delta: float, top_k: int,
                 norm_topk: bool):
    """One decode step of roster routing: per row, router logits plus the
    row's roster bias, then the usual top-k and softmax weights (``route``),
    then the usage update.  ``usage`` [T, E] is not modified; the updated
    counts are returned.  ``pinned`` is a [T] bool array or None.  x and
    w_router are float arrays (bf16 data goes through to_f64 first); the
    arithmetic is float64.

    Returns (ids, weights, biased logits, usage after the step)."""
    l = router_logits(np.asarray(x, dtype=np.float64), np.asarray(w_router, dtype=np.float64),
                      bias)
    T, E = l.shape
    new = np.array(usage, dtype=np.int64, copy=True)
    ids = np.zeros((T, top_k), dtype=np.int64)
    w = np.zeros((T, top_k), dtype=np.float64)
    lb = np.zeros_like(l)
    for t in range(T):
        pin = bool(pinned[t]) if pinned is not None else False
        lb[t] = l[t] + roster_bias(np.asarray(usage[t]), m, delta, pin)
        p = softmax(lb[t])
        ids[t] = top_experts(lb[t], top_k)
        w[t] = p[ids[t]]
        if norm_topk:
            w[t] = w[t] / np.sum(w[t])
        new[t, ids[t]] += 1
    return ids, w, lb, new


# ---------------------------------------------------------------- residual stream
# Between the layers of a decode step (not part of the pages' method: the
# glue that chains layers, needed to run a multi-layer step as one graph).

def residual_stream(x, y, dtype: str) -> np.ndarray:
    """The next layer's input: x + y in float32, rounded to the layers'
    dtype (bf16: round to nearest, ties to even; returned as uint16 bit
    patterns).  The sum is taken in float32 because that is the precision
    in which the rounding to bf16 is decided (a quantisation decided in the
    kernel's precision); torch's float32 -> bfloat16 conversion does the
    rounding."""
    xf = to_f64(x, dtype).astype(np.float32)
    s = xf + np.asarray(y, dtype=np.float32)
    if dtype == "f32":
        return s
    return torch.from_numpy(s).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
