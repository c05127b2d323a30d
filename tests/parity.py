"""Parity helpers: run the HIP layer through its C ABI, run the oracle on the
same seeded inputs, and compare them with the selection-window rule.

Rule (floating point decides which experts / neurons are kept, so an index
whose score lies within 1e-4 relative of the selection boundary may go
either way):
  1. for a score row v with kept count k < n, beta = (v_(k) + v_(k+1)) / 2;
     index i is ambiguous if |v_i - beta| <= 1e-4 * max(|beta|, 1e-30);
  2. the tested selection must equal the oracle's on every non-ambiguous
     index;
  3. the oracle then re-runs with the tested selection forced, and the
     outputs are compared by relative L2 over [T, H]: <= 1e-5 for the fp32
     layer, <= 1e-2 for the bf16 layer.
"""
from __future__ import annotations

import numpy as np
import torch

import moe_synth as S
import oracle
from sparse_moe_expert_route_amd import binding as B

WINDOW = 1e-4
TOL = {"f32": 1e-5, "bf16": 1e-2}


# ------------------------------------------------------------------ inputs

class LayerInputs:
    """Seeded host inputs of one layer (weights as stacked arrays)."""

    def __init__(self, shape: S.LayerShape, seed: int = 0):
        self.shape = shape
        self.seed = seed
        self.w_router = S.router_matrix(shape, seed)
        self.bias = S.router_bias(shape)
        self.wg, self.wu, self.wd = S.expert_weights(shape, seed)
        self.shared = (S.expert_weights(shape, seed, group=S.SHARED)
                       if shape.n_shared else None)

    def tokens(self, T: int, seed: int = 1):
        return S.tokens(self.shape, seed, T)


def to_dev(a: np.ndarray):
    """numpy float32, or bf16 bits as uint16, to a contiguous device tensor."""
    if a.dtype == np.uint16:
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


class DeviceLayer:
    """Device copies of a LayerInputs' weights.  score="swiglu" runs
    moe_expert_ffn_sparse / _dense (gate and up packed); score="gate" runs
    moe_expert_ffn_sparse_updown (gate packed, up row-major)."""

    def __init__(self, inp: LayerInputs, score: str = "swiglu"):
        self.inp = inp
        self.score = score
        sh = inp.shape
        self.desc = B.make_desc(sh.hidden, sh.n_experts, sh.d_ff, sh.top_k, sh.norm_topk, sh.dtype,
                                gate_up_layout="packed")
        self.w_router = to_dev(inp.w_router)
        self.bias = to_dev(inp.bias) if inp.bias is not None else None
        pk_up = B.moe_pack_gate_up if score == "swiglu" else (lambda d, w: w)
        # gate (and, for the SwiGLU score, up) go to the FFN calls packed
        # (moe_pack_gate_up); down stays row-major
        self.w = (B.moe_pack_gate_up(self.desc, to_dev(inp.wg)),
                  pk_up(self.desc, to_dev(inp.wu)), to_dev(inp.wd))
        self.desc_sh = None
        if inp.shared is not None:
            self.desc_sh = B.make_desc(sh.hidden, sh.n_shared, sh.d_ff_shared, sh.n_shared, False,
                                       sh.dtype, gate_up_layout="packed")
            g, u, d = inp.shared
            self.w_sh = (B.moe_pack_gate_up(self.desc_sh, to_dev(g)),
                         pk_up(self.desc_sh, to_dev(u)), to_dev(d))
        torch.cuda.synchronize()

    def packed_down(self):
        """Descriptors with down_layout = packed and W_d copies packed by
        moe_pack_down (routed, shared or None), made on first use."""
        if getattr(self, "_pd", None) is None:
            sh = self.inp.shape
            d = B.make_desc(sh.hidden, sh.n_experts, sh.d_ff, sh.top_k, sh.norm_topk, sh.dtype,
                            gate_up_layout="packed", down_layout="packed")
            pd = [d, B.moe_pack_down(d, self.w[2]), None, None]
            if self.desc_sh is not None:
                ds = B.make_desc(sh.hidden, sh.n_shared, sh.d_ff_shared, sh.n_shared, False,
                                 sh.dtype, gate_up_layout="packed", down_layout="packed")
                pd[2:] = [ds, B.moe_pack_down(ds, self.w_sh[2])]
            torch.cuda.synchronize()
            self._pd = tuple(pd)
        return self._pd

    def _fn(self, path):
        if self.score == "gate":
            assert path == B.MOE_PATH_SPARSE, "the gate-score split has no dense form"
            return B.moe_expert_ffn_sparse_updown
        return B.moe_expert_ffn_sparse if path == B.MOE_PATH_SPARSE else B.moe_expert_ffn_dense

    def run(self, x_host: np.ndarray, k: int, path: int, k_sh=None, path_sh=None,
            poison_rows=None, poison_up=None, packed_down=False, want_idx=True):
        """One layer call; returns host copies of routing, masks and y.
        packed_down: the dense calls take W_d packed by moe_pack_down.
        want_idx=False: no active_idx_out (the kept lists stay internal; the
        returned masks are then all -1)."""
        sh = self.inp.shape
        T = x_host.shape[0]
        x = to_dev(x_host)
        R = B.Routing.allocate(T, sh.top_k, sh.n_experts)
        ws_r = torch.empty(B.moe_route_workspace_size(self.desc, T), dtype=torch.uint8, device="cuda")
        B.moe_route(self.desc, T, x, self.w_router, self.bias, R, ws_r)
        y = torch.full((T, sh.hidden), float("nan"), dtype=torch.float32, device="cuda")
        idx = torch.full((max(1, T * sh.top_k), max(1, k)), -1, dtype=torch.int32, device="cuda")
        ws = torch.empty(B.moe_ffn_workspace_size(self.desc, T, k, path), dtype=torch.uint8, device="cuda")
        fn = self._fn(path)
        wd = self.w[2] if poison_rows is None else poison_rows
        wu = self.w[1] if poison_up is None else poison_up
        desc = self.desc
        if packed_down and path == B.MOE_PATH_DENSE:
            desc, wd = self.packed_down()[:2]
        fn(desc, T, k, x, self.w[0], wu, wd, R, y, 0, idx if k > 0 and want_idx else None, ws)
        out = dict(T=T, k=k)
        idx_sh = None
        if self.desc_sh is not None:
            ds = self.desc_sh
            k_sh = ds.d_ff if k_sh is None else k_sh
            path_sh = path if path_sh is None else path_sh
            idx_sh = torch.full((max(1, T * ds.top_k), max(1, k_sh)), -1, dtype=torch.int32, device="cuda")
            ws2 = torch.empty(B.moe_ffn_workspace_size(ds, T, k_sh, path_sh), dtype=torch.uint8, device="cuda")
            fs = self._fn(path_sh)
            wsh = self.w_sh
            if packed_down and path_sh == B.MOE_PATH_DENSE:
                ds, wd_sh = self.packed_down()[2:]
                wsh = (wsh[0], wsh[1], wd_sh)
            fs(ds, T, k_sh, x, *wsh, None, y, 1, idx_sh if k_sh > 0 and want_idx else None, ws2)
            out["k_sh"] = k_sh
        torch.cuda.synchronize()
        out.update(ids=R.topk_ids.cpu().numpy()[:T], w=R.topk_w.cpu().numpy()[:T],
                   offsets=R.expert_offsets.cpu().numpy(), pairs=R.pair_by_expert.cpu().numpy(),
                   active=R.active_experts.cpu().numpy(), n_active=int(R.n_active.cpu()[0]),
                   idx=idx.cpu().numpy(), y=y.cpu().numpy())
        if idx_sh is not None:
            out["idx_sh"] = idx_sh.cpu().numpy()
        return out


    def run_threshold(self, x_host: np.ndarray, tau, tau_sh=None, outputs=True):
        """One layer call with threshold masking (tau: device float32 [E]);
        outputs=False asks the library for neither kept counts nor ids."""
        sh = self.inp.shape
        T = x_host.shape[0]
        x = to_dev(x_host)
        R = B.Routing.allocate(T, sh.top_k, sh.n_experts)
        ws_r = torch.empty(B.moe_route_workspace_size(self.desc, T), dtype=torch.uint8, device="cuda")
        B.moe_route(self.desc, T, x, self.w_router, self.bias, R, ws_r)
        y = torch.full((T, sh.hidden), float("nan"), dtype=torch.float32, device="cuda")
        P = T * sh.top_k
        idx = torch.full((P, sh.d_ff), -1, dtype=torch.int32, device="cuda")
        cnt = torch.full((P,), -1, dtype=torch.int32, device="cuda")
        ws = torch.empty(B.moe_ffn_threshold_workspace_size(self.desc, T), dtype=torch.uint8,
                         device="cuda")
        fn = (B.moe_expert_ffn_sparse_updown_threshold if self.score == "gate"
              else B.moe_expert_ffn_sparse_threshold)
        fn(self.desc, T, tau, x, *self.w, R, y, 0, cnt if outputs else None,
           idx if outputs else None, ws)
        out = dict(T=T)
        if self.desc_sh is not None:
            ds = self.desc_sh
            idx_sh = torch.full((T * ds.top_k, ds.d_ff), -1, dtype=torch.int32, device="cuda")
            cnt_sh = torch.full((T * ds.top_k,), -1, dtype=torch.int32, device="cuda")
            ws2 = torch.empty(B.moe_ffn_threshold_workspace_size(ds, T), dtype=torch.uint8,
                              device="cuda")
            fn(ds, T, tau_sh, x, *self.w_sh, None, y, 1, cnt_sh,
                                              idx_sh, ws2)
            torch.cuda.synchronize()
            out.update(idx_sh=idx_sh.cpu().numpy(), cnt_sh=cnt_sh.cpu().numpy())
        torch.cuda.synchronize()
        out.update(ids=R.topk_ids.cpu().numpy()[:T], w=R.topk_w.cpu().numpy()[:T],
                   idx=idx.cpu().numpy(), cnt=cnt.cpu().numpy(), y=y.cpu().numpy())
        return out

    def route_ids(self, x_host: np.ndarray) -> np.ndarray:
        """The library's expert ids [T, top_k] for tokens x."""
        T = x_host.shape[0]
        R = B.Routing.allocate(T, self.desc.top_k, self.desc.n_experts)
        ws_r = torch.empty(B.moe_route_workspace_size(self.desc, T), dtype=torch.uint8,
                           device="cuda")
        B.moe_route(self.desc, T, to_dev(x_host), self.w_router, self.bias, R, ws_r)
        torch.cuda.synchronize()
        return R.topk_ids.cpu().numpy()[:T]

    def calibrate(self, x_host: np.ndarray, sparsity: float, shared: bool = False):
        """moe_calibrate_thresholds on calibration tokens; host float32 [E]."""
        T = x_host.shape[0]
        x = to_dev(x_host)
        if shared:
            desc, w, R = self.desc_sh, self.w_sh, None
        else:
            desc, w = self.desc, self.w
            R = B.Routing.allocate(T, desc.top_k, desc.n_experts)
            ws_r = torch.empty(B.moe_route_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
            B.moe_route(desc, T, x, self.w_router, self.bias, R, ws_r)
        tau = torch.full((desc.n_experts,), float("nan"), dtype=torch.float32, device="cuda")
        ws = torch.empty(B.moe_calibrate_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
        if self.score == "gate":
            B.moe_calibrate_thresholds_gate(desc, T, x, w[0], R, sparsity, tau, ws)
        else:
            B.moe_calibrate_thresholds(desc, T, x, w[0], w[1], R, sparsity, tau, ws)
        torch.cuda.synchronize()
        return tau.cpu().numpy()


# ------------------------------------------------------------------ comparison

def ambiguous(scores: np.ndarray, k: int) -> np.ndarray:
    """Boolean mask of indices within the window of the k-selection boundary."""
    n = scores.shape[0]
    if k <= 0 or k >= n:
        return np.zeros(n, dtype=bool)
    order = np.lexsort((np.arange(n), -scores))
    beta = 0.5 * (scores[order[k - 1]] + scores[order[k]])
    return np.abs(scores - beta) <= WINDOW * max(abs(beta), 1e-30)


def check_selection(got, want, scores, k, what):
    """Sets must agree except on ambiguous indices; returns True if they differ."""
    got, want = set(int(i) for i in got), set(int(i) for i in want)
    assert len(got) == len(want) == min(k, len(scores)), (what, len(got), len(want), k)
    diff = got ^ want
    if not diff:
        return False
    amb = ambiguous(scores, k)
    bad = [i for i in diff if not amb[i]]
    assert not bad, f"{what}: selection differs on non-ambiguous indices {bad}"
    return True


def pack_reference(w: np.ndarray, dtype: str) -> np.ndarray:
    """numpy statement of the packed gate/up layout (the header's formula):
    fragment (e, nt, ks) holds W[e, 16 nt + r, KS ks + c] at element
    (r + 16 (c // (KS/4))) * (KS/4) + c % (KS/4)."""
    E, d, H = w.shape
    KS = 32 if dtype == "bf16" else 16
    q = KS // 4
    v = w.reshape(E, d // 16, 16, H // KS, 4, q)          # e, nt, r, ks, group, c%q
    v = v.transpose(0, 1, 3, 4, 2, 5)                      # e, nt, ks, group, r, c%q
    return np.ascontiguousarray(v).reshape(E, d, H)


def pack_down_reference(w: np.ndarray) -> np.ndarray:
    """numpy statement of the packed down layout (the header's formula):
    fragment (e, ct, ks) holds W_d[e, 32 ks + 8 g + i, 16 ct + r] at element
    8 (r + 16 g) + i."""
    E, d, H = w.shape
    v = w.reshape(E, d // 32, 4, 8, H // 16, 16)           # e, ks, g, i, ct, r
    v = v.transpose(0, 4, 1, 2, 5, 3)                      # e, ct, ks, g, r, i
    return np.ascontiguousarray(v).reshape(E, d, H)


def rel_l2(a, b) -> float:
    a, b = np.asarray(a, np.float64), np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_routing(inp: LayerInputs, xs, ids_g, tokens=None):
    """GPU expert ids for tokens xs against the oracle's router: equal as
    sets up to the window rule on the logits, slots in descending logit."""
    sh = inp.shape
    tokens = np.arange(xs.shape[0]) if tokens is None else tokens
    ids0, _, logits0, _ = oracle.route(oracle.to_f64(xs, sh.dtype),
                                       oracle.to_f64(inp.w_router, sh.dtype),
                                       inp.bias, sh.top_k, sh.norm_topk)
    for i, t in enumerate(tokens):
        check_selection(ids_g[i], ids0[i], logits0[i], sh.top_k, f"route t={t}")
        lg = logits0[i][ids_g[i]]
        assert np.all(np.diff(lg) <= WINDOW * np.abs(lg[:-1]) + 1e-30), f"slot order t={t}"


def compare_layer(inp: LayerInputs, x_host, got, k, k_sh=None, tokens=None, score="swiglu"):
    """Check a GPU layer result against the oracle; returns the rel L2 error.

    ``tokens`` restricts the check to a sample of token rows (the layer is
    token-separable, so the oracle runs on just those tokens); ``score``
    selects the oracle's mask score (the layer variant the GPU ran)."""
    sh = inp.shape
    T = x_host.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    xs = x_host[tokens]
    shared = inp.shared
    ks = None
    if shared is not None:
        ks = k_sh if k_sh is not None else sh.d_ff_shared
    kw = dict(top_k=sh.top_k, norm_topk=sh.norm_topk, k_keep=k, dtype=sh.dtype,
              shared=shared, k_keep_shared=ks, score=score)
    ids_g = got["ids"][tokens]
    # 1. routing: as sets, window rule on the logits; slot order descending
    check_routing(inp, xs, ids_g, tokens)
    # 2. masks against the oracle forced to the GPU's experts
    r1 = oracle.moe_layer(xs, inp.w_router, inp.bias, inp.wg, inp.wu, inp.wd,
                          forced_ids=ids_g, **kw)
    np.testing.assert_allclose(got["w"][tokens], r1.weights, rtol=1e-4, atol=1e-7)
    forced_keep, forced_keep_sh = {}, {}
    differs = False
    if k > 0:
        for i, t in enumerate(tokens):
            for s in range(sh.top_k):
                g = got["idx"][t * sh.top_k + s, :k]
                assert np.all(np.diff(g) > 0), f"kept ids not ascending t={t} s={s}"
                differs |= check_selection(g, r1.keep[(i, s)], np.abs(r1.h[(i, s)]), k,
                                           f"mask t={t} s={s}")
                forced_keep[(i, s)] = g
    if shared is not None and ks and ks > 0:
        for i, t in enumerate(tokens):
            for j in range(sh.n_shared):
                g = got["idx_sh"][t * sh.n_shared + j, :ks]
                assert np.all(np.diff(g) > 0)
                differs |= check_selection(g, r1.keep_shared[(i, j)],
                                           np.abs(r1.h_shared[(i, j)]), ks,
                                           f"shared mask t={t} j={j}")
                forced_keep_sh[(i, j)] = g
    r2 = r1
    if differs:
        r2 = oracle.moe_layer(xs, inp.w_router, inp.bias, inp.wg, inp.wu, inp.wd,
                              forced_ids=ids_g, forced_keep=forced_keep or None,
                              forced_keep_shared=forced_keep_sh or None, keep_h=False, **kw)
    y_g = got["y"][tokens]
    assert np.all(np.isfinite(y_g)), "non-finite output"
    err = rel_l2(y_g, r2.y)
    assert err <= TOL[sh.dtype], f"rel L2 {err:.3e} > {TOL[sh.dtype]}"
    return err


def check_threshold_selection(got, scores, tau, what):
    """A threshold mask may differ from the oracle's only on scores within
    the window of tau."""
    want = set(int(j) for j in np.nonzero(np.abs(scores) > tau)[0])
    got = set(int(j) for j in got)
    diff = got ^ want
    if tau >= 0:
        bad = [j for j in diff if abs(abs(scores[j]) - tau) > WINDOW * max(tau, 1e-30)]
    else:
        bad = sorted(diff)
    assert not bad, f"{what}: threshold mask differs away from tau at {bad[:8]}"
    return bool(diff)


def compare_threshold_layer(inp: LayerInputs, x_host, got, tau, tau_sh=None, tokens=None,
                            score="swiglu"):
    """Check a threshold-masked GPU layer against the oracle given the same
    (float32) thresholds and mask score; returns the rel L2 error."""
    sh = inp.shape
    T = x_host.shape[0]
    tokens = np.arange(T) if tokens is None else np.asarray(tokens)
    xs = x_host[tokens]
    tau64 = np.asarray(tau, dtype=np.float64)
    tsh64 = None if tau_sh is None else np.asarray(tau_sh, dtype=np.float64)
    kw = dict(top_k=sh.top_k, norm_topk=sh.norm_topk, k_keep=0, dtype=sh.dtype,
              shared=inp.shared, thresholds=tau64, thresholds_shared=tsh64, score=score)
    ids_g = got["ids"][tokens]
    check_routing(inp, xs, ids_g, tokens)
    r1 = oracle.moe_layer(xs, inp.w_router, inp.bias, inp.wg, inp.wu, inp.wd,
                          forced_ids=ids_g, **kw)
    np.testing.assert_allclose(got["w"][tokens], r1.weights, rtol=1e-4, atol=1e-7)
    fk, fks = {}, {}
    for i, t in enumerate(tokens):
        for s in range(sh.top_k):
            p = t * sh.top_k + s
            n = int(got["cnt"][p])
            g = got["idx"][p, :n]
            assert np.all(np.diff(g) > 0), f"kept ids not ascending t={t} s={s}"
            check_threshold_selection(g, r1.h[(i, s)], tau64[int(ids_g[i, s])], f"t={t} s={s}")
            fk[(i, s)] = g
        if inp.shared is not None:
            for j in range(sh.n_shared):
                p = t * sh.n_shared + j
                n = int(got["cnt_sh"][p])
                g = got["idx_sh"][p, :n]
                check_threshold_selection(g, r1.h_shared[(i, j)], tsh64[j], f"shared t={t} j={j}")
                fks[(i, j)] = g
    r2 = oracle.moe_layer(xs, inp.w_router, inp.bias, inp.wg, inp.wu, inp.wd, forced_ids=ids_g,
                          forced_keep=fk, forced_keep_shared=fks or None, keep_h=False, **kw)
    y_g = got["y"][tokens]
    assert np.all(np.isfinite(y_g)), "non-finite output"
    err = rel_l2(y_g, r2.y)
    assert err <= TOL[sh.dtype], f"rel L2 {err:.3e} > {TOL[sh.dtype]}"
    return err


def check_grouping(got, E, top_k):
    """moe_route's grouping outputs are a stable counting sort of topk_ids."""
    ids = got["ids"].reshape(-1)
    P = ids.shape[0]
    counts = np.bincount(ids, minlength=E)
    np.testing.assert_array_equal(got["offsets"], np.concatenate([[0], np.cumsum(counts)]))
    want = np.lexsort((np.arange(P), ids))          # by expert, then pair id
    np.testing.assert_array_equal(got["pairs"][:P], want)
    act = np.nonzero(counts)[0]
    assert got["n_active"] == len(act)
    np.testing.assert_array_equal(got["active"][:len(act)], act)
    for t in range(ids.shape[0] // top_k):       # distinct experts per token
        assert len(set(ids[t * top_k:(t + 1) * top_k])) == top_k
