#!/usr/bin/env python3
"""Benchmark of the intra-expert-sparse MoE decode layer on one MI355X.

Workload: the OLMoE-like layer (bf16 weights and tokens, fp32 accumulation;
hidden 2048, 64 routed experts, d_ff 1024, top-8, no shared expert) at 90%
intra-expert sparsity (k = 103 kept neurons per token-expert pair),
synthetic seeded inputs.  One step = one whole layer call on one token
batch: moe_route, then the routed expert FFN on the path the shape-only
dispatcher picks.  The headline batch is 16 tokens; batches 1 and 4 are
measured the same way and reported under "batches".

Timing: every step is a replay of a captured HIP graph of the layer's
library calls (replays are first checked bitwise against eager calls).
The weights are cycled over enough device copies, and the token batches
over as many seeded batches, that >= 1 GB is touched between reuses of a
copy, so the ~256 MB Infinity Cache cannot serve the weight stream.
Per-kernel durations come from HIP events the library records around each
of its launches, on the launch stream, in eager steps queued ahead of the
GPU (so each event pair spans its kernel, not the host's launch latency);
the dominant kernel's roofline uses its algorithmic bytes per launch.  The
CPU oracle is timed on a bounded sample of the same workload on the host
cores as a reported baseline.

    python bench.py [--steps K] [--warmup W] [--batch T] [--sweep 1,4,16]

`--crossover` instead times the whole Llama-4-like layer (hidden 5120, 16
routed experts and 1 shared expert of d_ff 8192, top-1, 90% sparsity) on
both forced paths at batches 1, 8, 64, 256 and 1024, and prints one JSON
line with the per-batch timings, the path the shape-only dispatcher picks
and the faster one.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E peak, GB/s
LAYER = "olmoe-like"
MALL_DEFEAT_BYTES = 1 << 30    # bytes touched between reuses of one weight copy
CAL_SEED, CAL_TOKENS = 1000, 256   # threshold calibration set (a seed no timed batch uses)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--batch", type=int, default=16)
    ap.add_argument("--sparsity", type=float, default=0.9)
    ap.add_argument("--sweep", default="1,4,16", help="extra batch sizes, or 'none'")
    ap.add_argument("--path", choices=["auto", "sparse", "dense"], default="auto")
    ap.add_argument("--timer-steps", type=int, default=50, help="eager steps timed per kernel")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-variant", action="store_true",
                    help="skip the variants beside the headline (split, thresholds, roster, decode step)")
    ap.add_argument("--crossover", action="store_true",
                    help="sparse-vs-dense sweep of the Llama-4-like layer (its own JSON line)")
    ap.add_argument("--layer", default=None, help="layer of the crossover sweep")
    ap.add_argument("--batches", default=None, help="batches of the crossover sweep")
    ap.add_argument("--paths", default="sparse,dense,auto",
                    help="paths of the crossover sweep (sparse, dense, auto; dense-pk and "
                         "auto-pk: the dense groups read W_d packed by moe_pack_down)")
    ap.add_argument("--sparsity-shared", type=float, default=None,
                    help="shared-expert sparsity of the crossover sweep (default: --sparsity)")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain 1 GiB device copy (counter calibration) and exit")
    return ap.parse_args()


class Workload:
    """Device-resident layer copies and token batches for one batch size."""

    def __init__(self, shape, host_w, dev_w0, T, sparsity, path_arg, dev_sh0=None,
                 sparsity_shared=None, score="swiglu", packed_down=False):
        import torch
        import moe_synth as S
        from sparse_moe_expert_route_amd import binding as B
        self.B, self.torch = B, torch
        self.shape, self.T = shape, T
        sh = shape
        self.desc = B.make_desc(sh.hidden, sh.n_experts, sh.d_ff, sh.top_k, sh.norm_topk, sh.dtype,
                                gate_up_layout="packed")
        self.k = B.moe_keep_count(sparsity, sh.d_ff)
        forced = {"sparse": B.MOE_PATH_SPARSE, "dense": B.MOE_PATH_DENSE}.get(path_arg)
        self.auto_path = B.moe_select_path(self.desc, T, self.k)
        self.path = self.auto_path if forced is None else forced
        self.score = score
        thr = score in ("threshold", "gate_threshold")
        if score != "swiglu":   # these masks have a sparse form only
            self.path = B.MOE_PATH_SPARSE
        # always-on shared experts (routing NULL, accumulated into y)
        self.desc_sh = None
        if dev_sh0 is not None:
            n_sh, d_sh = sh.n_shared, sh.d_ff_shared
            self.desc_sh = B.make_desc(sh.hidden, n_sh, d_sh, n_sh, False, sh.dtype,
                                       gate_up_layout="packed")
            s_sh = sparsity if sparsity_shared is None else sparsity_shared
            self.k_sh = B.moe_keep_count(s_sh, d_sh)
            self.auto_path_sh = B.moe_select_path(self.desc_sh, T, self.k_sh)
            self.path_sh = self.auto_path_sh if forced is None else forced
            self.ws_sh = torch.empty(B.moe_ffn_workspace_size(self.desc_sh, T, self.k_sh, self.path_sh),
                                     dtype=torch.uint8, device="cuda")
            self.ffn_sh = (B.moe_expert_ffn_sparse if self.path_sh == B.MOE_PATH_SPARSE
                           else B.moe_expert_ffn_dense)
        # bytes one call touches (gate/up of the expected active experts dominate)
        E, K = sh.n_experts, sh.top_k
        act = E * (1 - (1 - K / E) ** T)
        per_call = act * 3 * sh.hidden * sh.d_ff * 2
        if dev_sh0 is not None:
            per_call += sh.n_shared * 3 * sh.hidden * sh.d_ff_shared * 2
        self.L = max(2, min(24, 1 + math.ceil(MALL_DEFEAT_BYTES / per_call)))
        self.copies = [dev_w0] + [tuple(w.clone() for w in dev_w0) for _ in range(self.L - 1)]
        self.copies_sh = None
        if dev_sh0 is not None:
            self.copies_sh = [dev_sh0] + [tuple(w.clone() for w in dev_sh0) for _ in range(self.L - 1)]
        self.x_host = [S.tokens(sh, 1 + i, T) for i in range(self.L)]
        self.x = [host_w.to_dev(x) for x in self.x_host]
        # the layer's router bias (the Zipf skew of the Qwen3-MoE-like layer), or None
        self.bias = host_w.to_dev(host_w.bias) if host_w.bias is not None else None
        self.routing = [B.Routing.allocate(T, K, E) for _ in range(self.L)]
        self.ws_r = torch.empty(B.moe_route_workspace_size(self.desc, T), dtype=torch.uint8, device="cuda")
        self.ws = torch.empty(B.moe_ffn_workspace_size(self.desc, T, self.k, self.path),
                              dtype=torch.uint8, device="cuda")
        # plain routed layers on the sparse path run as one moe_layer_sparse
        # call (the same kernels as moe_route + moe_expert_ffn_sparse, and at
        # one token the selection runs inside the gate/up kernel)
        self.layer_call = score == "swiglu" and self.path == B.MOE_PATH_SPARSE and dev_sh0 is None
        self.ws_l = (torch.empty(B.moe_layer_workspace_size(self.desc, T, self.k), dtype=torch.uint8,
                                 device="cuda") if self.layer_call else None)
        self.y = [torch.empty((T, sh.hidden), dtype=torch.float32, device="cuda") for _ in range(self.L)]
        self.idx = torch.empty((T * K, max(1, self.k)), dtype=torch.int32, device="cuda")
        if thr:
            # per-expert tau for the target sparsity, calibrated once offline on
            # tokens of another seed (the thresholds are fixed before serving)
            x_cal = host_w.to_dev(S.tokens(sh, CAL_SEED, CAL_TOKENS))
            r_cal = B.Routing.allocate(CAL_TOKENS, K, E)
            ws_c = torch.empty(B.moe_route_workspace_size(self.desc, CAL_TOKENS), dtype=torch.uint8,
                               device="cuda")
            B.moe_route(self.desc, CAL_TOKENS, x_cal, dev_w0[0], self.bias, r_cal, ws_c)
            ws_c = torch.empty(B.moe_calibrate_workspace_size(self.desc, CAL_TOKENS),
                               dtype=torch.uint8, device="cuda")
            self.tau = torch.empty(E, dtype=torch.float32, device="cuda")
            if score == "gate_threshold":   # on the split's scores |silu(W_g x)|
                B.moe_calibrate_thresholds_gate(self.desc, CAL_TOKENS, x_cal, dev_w0[1], r_cal,
                                                sparsity, self.tau, ws_c)
            else:
                B.moe_calibrate_thresholds(self.desc, CAL_TOKENS, x_cal, dev_w0[1], dev_w0[2],
                                           r_cal, sparsity, self.tau, ws_c)
            torch.cuda.synchronize()
            del ws_c, r_cal, x_cal
            self.ws = torch.empty(B.moe_ffn_threshold_workspace_size(self.desc, T),
                                  dtype=torch.uint8, device="cuda")
            self.idx = torch.empty((T * K, sh.d_ff), dtype=torch.int32, device="cuda")
            self.counts = torch.empty(T * K, dtype=torch.int32, device="cuda")
        self.ffn = B.moe_expert_ffn_sparse if self.path == B.MOE_PATH_SPARSE else B.moe_expert_ffn_dense
        if score == "gate":   # the page's own split (w_up row-major in dev_w0)
            self.ffn = B.moe_expert_ffn_sparse_updown
        if thr:  # the page's literal mask: a score above tau[e], counts vary
            fn = (B.moe_expert_ffn_sparse_updown_threshold if score == "gate_threshold"
                  else B.moe_expert_ffn_sparse_threshold)
            self.ffn = lambda d, T_, k, x, wg, wu, wd, r, y, acc, idx, ws: \
                fn(d, T_, self.tau, x, wg, wu, wd, r, y, acc,
                   self.counts if idx is not None else None, idx, ws)
        if packed_down and sh.dtype == "bf16":
            self._pack_down()
        self.graphs = []

    def _pack_down(self):
        """The groups on the dense path read W_d packed by moe_pack_down (a
        deployment that serves both paths keeps both copies)."""
        B, sh = self.B, self.shape
        if self.path == B.MOE_PATH_DENSE:
            self.desc = B.make_desc(sh.hidden, sh.n_experts, sh.d_ff, sh.top_k, sh.norm_topk,
                                    sh.dtype, gate_up_layout="packed", down_layout="packed")
            self.copies = [(wr, wg, wu, B.moe_pack_down(self.desc, wd))
                           for wr, wg, wu, wd in self.copies]
        if self.desc_sh is not None and self.path_sh == B.MOE_PATH_DENSE:
            n_sh = sh.n_shared
            self.desc_sh = B.make_desc(sh.hidden, n_sh, sh.d_ff_shared, n_sh, False, sh.dtype,
                                       gate_up_layout="packed", down_layout="packed")
            self.copies_sh = [(sg, su, B.moe_pack_down(self.desc_sh, sd))
                              for sg, su, sd in self.copies_sh]
        self.torch.cuda.synchronize()

    def step(self, i, idx=None):
        B = self.B
        j = i % self.L
        wr, wg, wu, wd = self.copies[j]
        if self.layer_call:
            B.moe_layer_sparse(self.desc, self.T, self.k, self.x[j], wr, self.bias, wg, wu, wd,
                               self.routing[j], self.y[j], 0, idx, self.ws_l)
            return
        B.moe_route(self.desc, self.T, self.x[j], wr, self.bias, self.routing[j], self.ws_r)
        self.ffn(self.desc, self.T, self.k, self.x[j], wg, wu, wd, self.routing[j], self.y[j], 0,
                 idx, self.ws)
        if self.copies_sh is not None:
            sg, su, sd = self.copies_sh[j]
            self.ffn_sh(self.desc_sh, self.T, self.k_sh, self.x[j], sg, su, sd, None, self.y[j], 1,
                        None, self.ws_sh)

    def capture(self):
        torch = self.torch
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            for i in range(self.L):        # warm the allocator / code objects off-graph
                self.step(i)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        for i in range(self.L):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                self.step(i)
            self.graphs.append(g)
        torch.cuda.synchronize()

    def check_replays(self):
        """Graph replays reproduce eager calls bit for bit, replay after replay."""
        torch = self.torch
        ref = []
        for i in range(self.L):
            self.step(i)
            torch.cuda.synchronize()
            ref.append(self.y[i].clone())
        for rep in range(3):
            for i in range(self.L):
                self.y[i].fill_(float("nan"))
                self.graphs[i].replay()
                torch.cuda.synchronize()
                if not torch.equal(self.y[i], ref[i]):
                    raise RuntimeError(f"graph replay {rep} of copy {i} differs from the eager call")
                self.step(i)              # eager work between replays
                torch.cuda.synchronize()

    def bytes_per_call(self):
        """Algorithmic HBM bytes of each batch's layer call, from its routing and masks."""
        import numpy as np
        torch, sh, B = self.torch, self.shape, self.B
        out = []
        for i in range(self.L):
            self.step(i, idx=self.idx)
            torch.cuda.synchronize()
            ids = self.routing[i].topk_ids.cpu().numpy().reshape(-1)
            idx = self.idx.cpu().numpy()
            active = np.unique(ids)
            P = ids.shape[0]
            bw = 2 if sh.dtype == "bf16" else 4
            H, d = sh.hidden, sh.d_ff
            cnt = (self.counts.cpu().numpy() if self.score in ("threshold", "gate_threshold")
                   else np.full(P, self.k, dtype=np.int64))
            gate_only = self.score in ("gate", "gate_threshold")
            kept = [idx[p, :cnt[p]] for p in range(P)]
            union = sum(len(np.unique(np.concatenate([kept[p] for p in np.nonzero(ids == e)[0]])))
                        for e in active)
            rec = dict(
                active=int(len(active)), pairs=int(P),
                router=sh.n_experts * H * bw,
                gateup=(int(len(active)) * (1 if gate_only else 2) * H * d * bw
                        + self.T * H * bw + P * d * 4),
                up_rows=int(cnt.sum()) * H * bw if gate_only else 0,
                down_rows=int(cnt.sum()) * H * bw, mean_kept=float(cnt.mean()),
                down_union=union * H * bw,
                down_dense=int(len(active)) * d * H * bw,
                io=self.T * H * (bw + 4))
            path_down = rec["down_rows"] if self.path == B.MOE_PATH_SPARSE else rec["down_dense"]
            rec["layer"] = rec["router"] + rec["gateup"] + rec["up_rows"] + path_down + rec["io"]
            rec["layer_min"] = rec["router"] + rec["gateup"] + rec["up_rows"] + rec["down_union"] + rec["io"]
            # MFMA work of the dense contractions (2 flops per multiply-add)
            rec["flops_gateup"] = 2 * 2 * P * H * d
            rec["flops_down_dense"] = 2 * P * d * H
            if self.copies_sh is not None:
                n_sh, d_sh = sh.n_shared, sh.d_ff_shared
                sh_gu = n_sh * 2 * H * d_sh * bw + self.T * n_sh * d_sh * 4
                sh_dn = (self.T * n_sh * self.k_sh * H * bw if self.path_sh == B.MOE_PATH_SPARSE
                         else n_sh * d_sh * H * bw)
                rec["shared"] = sh_gu + sh_dn + self.T * H * 4
                rec["layer"] += rec["shared"]
                rec["layer_min"] += rec["shared"]
                rec["flops_gateup"] += 2 * 2 * self.T * n_sh * H * d_sh
                rec["flops_down_dense"] += 2 * self.T * n_sh * d_sh * H
            out.append(rec)
        return out


def time_graphs(wl, steps, warmup):
    torch = wl.torch
    for i in range(warmup):
        wl.graphs[i % wl.L].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        wl.graphs[i % wl.L].replay()
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) / steps


def time_kernels(wl, steps, chunk=10):
    """Per-kernel durations from HIP events the library records around each
    of its launches, on the launch stream (eager steps).  Each chunk of
    steps is queued behind a short GPU spin on the same stream, so the host
    has enqueued the whole chunk before the GPU reaches it: the event pairs
    then run back to back with their kernels instead of waiting for the
    host's next launch, and span little more than the kernel itself."""
    from sparse_moe_expert_route_amd import binding as B
    torch = wl.torch
    if steps <= 0:
        return {}
    timer = B.StageTimer(capacity=steps * 16 + 16)
    for i in range(wl.L):                 # warm the eager path
        wl.step(i)
    torch.cuda.synchronize()
    spin = getattr(torch.cuda, "_sleep", None)
    with timer:
        for c0 in range(0, steps, chunk):
            if spin is not None:
                spin(10_000_000)          # ~4 ms: longer than the host needs to enqueue a chunk
            for i in range(c0, min(steps, c0 + chunk)):
                wl.step(i)
            torch.cuda.synchronize()
    d = timer.durations()
    timer.close()
    return {k: dict(n=len(v), avg_us=1e3 * sum(v) / len(v), per_step_us=1e3 * sum(v) / steps)
            for k, v in d.items()}


def event_pair_overhead(reps=50, chunk=10):
    """What an event pair adds, measured the way time_kernels measures:
    pairs queued behind a GPU spin, around nothing and around a 16-byte
    moe_stream_read (a kernel that does almost nothing)."""
    import torch
    from sparse_moe_expert_route_amd import binding as B
    buf = torch.zeros(16, dtype=torch.uint8, device="cuda")
    sink = torch.empty(B.STREAM_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    spin = getattr(torch.cuda, "_sleep", None)
    out = {}
    for name, work in (("empty_pair_us", lambda: None),
                       ("tiny_kernel_pair_us", lambda: B.moe_stream_read(buf, sink))):
        work()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for c0 in range(0, reps, chunk):
            if spin is not None:
                spin(10_000_000)
            for i in range(c0, min(reps, c0 + chunk)):
                ev[i][0].record()
                work()
                ev[i][1].record()
            torch.cuda.synchronize()
        out[name] = round(sum(s.elapsed_time(e) for s, e in ev) * 1e3 / reps, 2)
    return out


def time_stages(fn, steps, chunk=10):
    """time_kernels for any callable that launches library kernels."""
    import torch
    from sparse_moe_expert_route_amd import binding as B
    timer = B.StageTimer(capacity=steps * 8 + 8)
    fn(0)
    torch.cuda.synchronize()
    spin = getattr(torch.cuda, "_sleep", None)
    with timer:
        for c0 in range(0, steps, chunk):
            if spin is not None:
                spin(10_000_000)
            for i in range(c0, min(steps, c0 + chunk)):
                fn(i)
            torch.cuda.synchronize()
    d = timer.durations()
    timer.close()
    return {k: round(1e3 * sum(v) / len(v), 2) for k, v in d.items()}


def roster_variant(shape, host, dev_w0, T=16, m=8, seq_len=256, deltas=(1.0, 2.0, 4.0)):
    """Roster routing (Predatory MoE, the roster routing rule) on this layer's
    router: the selection kernel's cost against plain routing, and the
    working set (distinct experts per sequence) over a synthetic decode of
    seq_len steps for T sequences, unconstrained, in the barrier phase at
    each delta, and pinned after a 20 % prefix."""
    import numpy as np
    import torch
    import moe_synth as S
    from sparse_moe_expert_route_amd import binding as B
    E, K = shape.n_experts, shape.top_k
    desc = B.make_desc(shape.hidden, E, shape.d_ff, K, shape.norm_topk, shape.dtype,
                       gate_up_layout="packed")
    wr = dev_w0[0]
    xs = [host.to_dev(S.tokens(shape, 2000 + i, T)) for i in range(seq_len)]
    R = B.Routing.allocate(T, K, E)
    ws = torch.empty(B.moe_route_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
    usage = torch.zeros((T, E), dtype=torch.int32, device="cuda")
    plain = time_stages(lambda i: B.moe_route(desc, T, xs[i % seq_len], wr, None, R, ws), 50)
    timed = time_stages(lambda i: B.moe_route_roster(desc, T, xs[i % seq_len], wr, None, usage,
                                                     None, m, 1.0, R, ws), 50)

    def working_set(delta, pin_after=None):
        u = torch.zeros((T, E), dtype=torch.int32, device="cuda")
        pinned = torch.zeros(T, dtype=torch.int32, device="cuda")
        for i in range(seq_len):
            if pin_after is not None and i == pin_after:
                pinned.fill_(1)
            if delta is None:
                B.moe_route(desc, T, xs[i], wr, None, R, ws)
                u.scatter_add_(1, R.topk_ids[:T].long(), torch.ones_like(R.topk_ids[:T]))
            else:
                B.moe_route_roster(desc, T, xs[i], wr, None, u, pinned if pin_after else None,
                                   m, delta, R, ws)
        torch.cuda.synchronize()
        return round(float((u > 0).sum(1).float().mean()), 2)

    out = {"T": T, "roster_size": m, "seq_len": seq_len,
           "select_us": {"plain": plain.get("router_topk"), "roster": timed.get("router_topk")},
           "working_set": {"unconstrained": working_set(None)}}
    for d in deltas:
        out["working_set"][f"delta_{d}"] = working_set(d)
    out["working_set"]["pinned_after_20pct_delta_4.0"] = working_set(4.0, pin_after=seq_len // 5)
    return out


def decode_step_variant(shape, args, n_layers=8, batches=(1, 16)):
    """A decode step through n_layers MoE layers of this shape with distinct
    weights (seeds 0 .. n_layers - 1): per layer route -> FFN (the
    dispatcher's path) -> residual, the whole step captured as one HIP graph.
    Distinct layers (>= 0.5 GB of weights per step at batch 1) keep the
    reads in HBM without rotating copies.  Replays are checked bitwise
    against an eager step before timing."""
    import torch
    import moe_synth as S
    from sparse_moe_expert_route_amd import binding as B
    desc = B.make_desc(shape.hidden, shape.n_experts, shape.d_ff, shape.top_k, shape.norm_topk,
                       shape.dtype, gate_up_layout="packed")
    to_dev = HostLayer.to_dev
    layers = []
    for s in range(n_layers):
        wg, wu, wd = S.expert_weights(shape, s)
        layers.append((to_dev(S.router_matrix(shape, s)), B.moe_pack_gate_up(desc, to_dev(wg)),
                       B.moe_pack_gate_up(desc, to_dev(wu)), to_dev(wd)))
        del wg, wu, wd
    torch.cuda.synchronize()
    E, K = shape.n_experts, shape.top_k
    k = B.moe_keep_count(args.sparsity, shape.d_ff)
    out = {"layers": n_layers, "what": "route -> FFN -> residual per layer, one graph per step; "
           "the sparse FFN call writes the next layer's input in its epilogue "
           "(moe_expert_ffn_sparse_residual), 'unfused' runs moe_residual_add after it"}
    for T in batches:
        path = B.moe_select_path(desc, T, k)
        ffn = B.moe_expert_ffn_sparse if path == B.MOE_PATH_SPARSE else B.moe_expert_ffn_dense
        x0 = to_dev(S.tokens(shape, 3000 + T, T))
        xs = [torch.empty_like(x0) for _ in layers]
        y = torch.empty((T, shape.hidden), dtype=torch.float32, device="cuda")
        Rs = [B.Routing.allocate(T, K, E) for _ in layers]
        ws_r = torch.empty(B.moe_route_workspace_size(desc, T), dtype=torch.uint8, device="cuda")
        ws = torch.empty(B.moe_ffn_workspace_size(desc, T, k, path), dtype=torch.uint8,
                         device="cuda")

        def step(fused):
            x = x0
            for (wr, wg, wu, wd), xo, R in zip(layers, xs, Rs):
                B.moe_route(desc, T, x, wr, None, R, ws_r)
                if fused and path == B.MOE_PATH_SPARSE:
                    B.moe_expert_ffn_sparse_residual(desc, T, k, x, wg, wu, wd, R, y, x, xo, 0,
                                                     None, ws)
                else:
                    ffn(desc, T, k, x, wg, wu, wd, R, y, 0, None, ws)
                    B.moe_residual_add(desc, T, x, y, xo)
                x = xo

        step(False)
        torch.cuda.synchronize()
        ref = xs[-1].clone()
        timed = {}
        for fused in (True, False):
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step(fused)
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step(fused)
            torch.cuda.synchronize()
            xs[-1].fill_(0)
            g.replay()
            torch.cuda.synchronize()
            if not torch.equal(xs[-1], ref):
                raise RuntimeError("decode-step graph replay differs from the eager step")
            for _ in range(args.warmup):
                g.replay()
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(args.steps):
                g.replay()
            torch.cuda.synchronize()
            timed[fused] = (time.perf_counter() - t0) / args.steps * 1e6
            del g
        us = timed[True]
        out[str(T)] = {"path": "sparse" if path == B.MOE_PATH_SPARSE else "dense",
                       "us_per_step": round(us, 1), "us_per_layer": round(us / n_layers, 2),
                       "us_per_token_per_layer": round(us / n_layers / T, 3),
                       "unfused_us_per_layer": round(timed[False] / n_layers, 2)}
        del xs, Rs, ws, ws_r, y
        torch.cuda.empty_cache()
    del layers
    torch.cuda.empty_cache()
    return out


def cpu_baseline(shape, host, wl, seconds):
    """The oracle as it stands, on the host, over a bounded sample of steps."""
    import oracle
    import threadpoolctl
    # the host cores this process may run on, and the BLAS pool the oracle's
    # products actually use (the box caps pools by OMP_NUM_THREADS)
    cores = len(os.sched_getaffinity(0))
    info = threadpoolctl.threadpool_info()
    blas_threads = max([i.get("num_threads", 1) for i in info] or [1])
    import numpy as np
    T = wl.T
    wl.step(0)                           # the timed batch 0 once more, for the parity check
    wl.torch.cuda.synchronize()
    y_gpu = wl.y[0].cpu().numpy().astype(np.float64)

    def call(i):
        x = wl.x_host[i % wl.L]
        return oracle.moe_layer(x, host.w_router, host.bias, host.wg, host.wu, host.wd, top_k=shape.top_k,
                                norm_topk=shape.norm_topk, k_keep=wl.k, dtype=shape.dtype,
                                keep_h=False)

    times, y_first, t0 = [], None, time.perf_counter()
    while True:
        c0 = time.perf_counter()
        r = call(len(times))
        times.append(time.perf_counter() - c0)
        if y_first is None:
            y_first = r.y
        el = time.perf_counter() - t0
        if el >= seconds or len(times) >= 50:
            break
    done = len(times)
    med = float(np.median(times))
    # one BLAS thread, a few calls (bounded to about a fifth of the sample's time)
    t1 = []
    try:
        with threadpoolctl.threadpool_limits(limits=1):
            s0 = time.perf_counter()
            while len(t1) < 3 and (not t1 or time.perf_counter() - s0 < seconds / 5):
                c0 = time.perf_counter()
                call(len(t1))
                t1.append(time.perf_counter() - c0)
    except Exception:  # pragma: no cover
        t1 = []
    bpc = wl.bytes_per_call()
    layer_bytes = sum(r["layer"] for r in bpc) / len(bpc)
    # the oracle's own routing and masks, no forcing: a near-tie that breaks
    # the other way would show here as a larger error (tests/ apply the
    # window rule; this is a sanity gate on the timed workload)
    rel = float(np.linalg.norm(y_gpu - y_first) / max(np.linalg.norm(y_first), 1e-300))
    out = {"value": round(med * 1e6 / T, 1), "unit": "us/token", "cores": int(cores),
           "blas_threads": int(blas_threads), "kind": "oracle",
           "sample": f"{done} layer calls of {T} tokens ({done * T} tokens) of the same layer, "
                     f"{el:.1f} s, float64 numpy oracle; value = median call / T",
           "tokens_per_s": round(T / med, 2),
           "implied_gbs": round(layer_bytes / med / 1e9, 3),
           "parity_rel_l2_batch0": float(f"{rel:.3e}")}
    if t1:
        out["one_thread"] = {"us_per_token": round(float(np.median(t1)) * 1e6 / T, 1),
                             "calls": len(t1)}
    return out


class HostLayer:
    def __init__(self, shape, shared=False):
        import moe_synth as S
        self.w_router = S.router_matrix(shape, 0)
        self.bias = S.router_bias(shape)
        self.wg, self.wu, self.wd = S.expert_weights(shape, 0)
        self.shared = S.expert_weights(shape, 0, group=S.SHARED) if shared else None

    @staticmethod
    def to_dev(a):
        import numpy as np
        import torch
        if a.dtype == np.uint16:
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def measure(shape, host, dev_w0, T, args, path=None, dev_sh0=None, score="swiglu",
            sparsity=None, sparsity_shared=None, packed_down=False):
    wl = Workload(shape, host, dev_w0, T, args.sparsity if sparsity is None else sparsity,
                  path or args.path, dev_sh0=dev_sh0, score=score,
                  sparsity_shared=sparsity_shared, packed_down=packed_down)
    log(f"[bench] {shape.name} T={T} k={wl.k} path={'sparse' if wl.path == 0 else 'dense'} "
        f"copies={wl.L}")
    wl.capture()
    wl.check_replays()
    bpc = wl.bytes_per_call()
    sec = time_graphs(wl, args.steps, args.warmup)
    kern = time_kernels(wl, args.timer_steps)
    mean = lambda key: sum(r[key] for r in bpc) / len(bpc)
    res = dict(T=T, k=wl.k, path="sparse" if wl.path == 0 else "dense", copies=wl.L,
               us_per_call=sec * 1e6, us_per_token=sec * 1e6 / T, tokens_per_s=T / sec,
               layer_bytes=mean("layer"), layer_min_bytes=mean("layer_min"),
               gateup_bytes=mean("gateup"), down_bytes=mean("down_rows"),
               down_union_bytes=mean("down_union"), active_experts=mean("active"),
               mean_kept=mean("mean_kept"),
               flops_gateup=mean("flops_gateup"), flops_down_dense=mean("flops_down_dense"),
               auto_path="sparse" if wl.auto_path == 0 else "dense", kernels=kern)
    res["hbm_gbs"] = res["layer_bytes"] / sec / 1e9
    res["hbm_frac"] = res["hbm_gbs"] / HBM_PEAK_GBS
    # the fused decode-batch launch moves the gate/up stream, the kept down
    # rows and y in one kernel
    res["fused_bytes"] = res["gateup_bytes"] + res["down_bytes"] + T * shape.hidden * 4
    return wl, res


KERNEL_SOURCES = ("sparse_moe_expert_route_amd/csrc/ffn.hip",
                  "sparse_moe_expert_route_amd/csrc/ffn_common.h",
                  "sparse_moe_expert_route_amd/csrc/device_common.h",
                  "sparse_moe_expert_route_amd/csrc/route.hip",
                  "sparse_moe_expert_route_amd/csrc/route_common.h")
PMC_SUMMARY = os.path.join(ROOT, "profiles", "olmoe_like_T16_pmc_traffic.txt")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(stage):
    """HBM bytes per launch from the committed counter summary, or None when
    it is missing, covers another kernel, or predates the current sources."""
    try:
        top, sec = {}, {}
        cur = top
        with open(PMC_SUMMARY) as f:
            for line in f:
                line = line.strip()
                if not line or line.startswith("#"):
                    continue
                if line.startswith("[") and line.endswith("]"):
                    cur = sec.setdefault(line[1:-1], {})
                elif ":" in line:
                    k, v = line.split(":", 1)
                    cur[k.strip()] = v.strip()
        if top.get("source_hash") != kernel_source_hash() or stage not in sec:
            return None
        return int(float(sec[stage]["traffic_bytes_per_launch"]))
    except (OSError, KeyError, ValueError):
        return None


def roofline(res, stage, bytes_key, practical=None, sized=None):
    k = res["kernels"].get(stage)
    if not k:
        return None
    gbs = res[bytes_key] / (k["avg_us"] * 1e-6) / 1e9
    out = {"bound": "hbm", "kernel": stage, "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
           "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4),
           "traffic": measured_traffic(stage),
           "avg_us": round(k["avg_us"], 2), "bytes_per_launch": int(res[bytes_key])}
    if practical:
        out["frac_practical"] = round(gbs / practical["gbs"], 4)
    if sized:
        out["size_matched_read"] = sized
        out["frac_size_matched"] = round(gbs / sized["gbs"], 4)
    return out


DOWN_TARGET = 0.70


def down_target(batches):
    """The sparse down projection against its target (>= 70 % of 8 TB/s on
    the bytes it loads, at every decode batch 1-16), batch by batch: where
    the kept W_down rows stream in a launch of their own, that launch's rate
    over those rows; where they stream inside the fused FFN launch (gate/up,
    masks, down and combine in one kernel), that launch's rate over all its
    bytes.  Event durations include the markers' own few microseconds."""
    out = {"what": "sparse down projection >= 70% of 8 TB/s on the bytes loaded, batches 1-16",
           "target_frac": DOWN_TARGET, "batches": {}}
    for T, b in sorted(batches.items(), key=lambda kv: int(kv[0])):
        k = b.get("kernels_us", {})
        if "down_rows" in k:
            us, nb, how = k["down_rows"], b["down_bytes"], "own launch (kept rows only)"
        elif "fused_ffn" in k:
            us, nb, how = k["fused_ffn"], b["fused_bytes"], "fused FFN launch (gate/up + kept rows)"
        else:
            continue
        gbs = nb / (us * 1e-6) / 1e9
        out["batches"][T] = {"launch": how, "bytes": int(nb), "event_us": round(us, 2),
                             "gbs": round(gbs, 1), "frac": round(gbs / HBM_PEAK_GBS, 4),
                             "met": gbs / HBM_PEAK_GBS >= DOWN_TARGET}
    out["met_at_every_batch"] = bool(out["batches"]) and all(v["met"] for v in out["batches"].values())
    return out


def size_matched_read(nbytes, reps=40, chunk=10):
    """A plain streaming read (moe_stream_read) of exactly `nbytes`, timed
    like the library's kernels: event pairs on the launch stream, queued
    behind a GPU spin so they run back to back with the kernel.  Buffers
    rotate over >= 1.2 GB so the reads come from HBM, not the caches.  The
    rate a kernel of that size can reach, ramp and drain included."""
    import torch
    from sparse_moe_expert_route_amd import binding as B
    nbytes = max(16, int(round(nbytes / 16)) * 16)   # the read takes 16-byte multiples
    nb = max(2, math.ceil(1.2e9 / nbytes))
    bufs = [torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1) for _ in range(nb)]
    sink = torch.empty(B.STREAM_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    for b in bufs:
        B.moe_stream_read(b, sink)
    torch.cuda.synchronize()
    spin = getattr(torch.cuda, "_sleep", None)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(reps)]
    for c0 in range(0, reps, chunk):
        if spin is not None:
            spin(10_000_000)
        for i in range(c0, min(reps, c0 + chunk)):
            ev[i][0].record()
            B.moe_stream_read(bufs[i % nb], sink)
            ev[i][1].record()
        torch.cuda.synchronize()
    us = sum(s.elapsed_time(e) for s, e in ev) * 1e3 / reps
    del bufs
    torch.cuda.empty_cache()
    return {"bytes": int(nbytes), "avg_us": round(us, 2), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}


def practical_read_peak(gib=4, reps=5):
    """The practical HBM read peak: a plain streaming read of a buffer much
    larger than the caches (moe_stream_read), best of `reps` event-timed
    runs on the launch stream."""
    import torch
    from sparse_moe_expert_route_amd import binding as B
    n = gib << 30
    buf = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    sink = torch.empty(B.STREAM_READ_SINK_WORDS, dtype=torch.int32, device="cuda")
    B.moe_stream_read(buf, sink)
    torch.cuda.synchronize()
    best = 0.0
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        B.moe_stream_read(buf, sink)
        e.record()
        e.synchronize()
        best = max(best, n / (s.elapsed_time(e) * 1e-3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return {"gbs": round(best, 1), "kernel": f"moe_stream_read: {gib} GiB, non-temporal 16-byte loads",
            "reps": reps}


def calibrate_copy():
    """A plain device copy of known size: what FETCH_SIZE / WRITE_SIZE read
    for it gives the counters' scale factors."""
    import torch
    n = 1 << 30
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    reps = 5
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / reps
    print(json.dumps({"calibrate_copy_bytes": n, "reps": reps,
                      "read_plus_write_gbs": round(2 * n / dt / 1e9, 1)}), flush=True)


def dev_layer(shape, host, B):
    desc = B.make_desc(shape.hidden, shape.n_experts, shape.d_ff, shape.top_k, shape.norm_topk,
                       shape.dtype, gate_up_layout="packed")
    dev_w0 = (host.to_dev(host.w_router), B.moe_pack_gate_up(desc, host.to_dev(host.wg)),
              B.moe_pack_gate_up(desc, host.to_dev(host.wu)), host.to_dev(host.wd))
    dev_sh0 = None
    if host.shared is not None:
        n_sh = shape.n_shared
        dsh = B.make_desc(shape.hidden, n_sh, shape.d_ff_shared, n_sh, False, shape.dtype,
                          gate_up_layout="packed")
        g, u, d = host.shared
        dev_sh0 = (B.moe_pack_gate_up(dsh, host.to_dev(g)), B.moe_pack_gate_up(dsh, host.to_dev(u)),
                   host.to_dev(d))
    return dev_w0, dev_sh0


def crossover(args):
    """Both forced paths of one layer over a batch sweep: where the dense
    MFMA path overtakes the sparse one, next to the dispatcher's pick."""
    import torch
    import moe_synth as S
    from sparse_moe_expert_route_amd import binding as B
    shape = S.LAYERS[args.layer or "llama4-like"]
    batches = ([int(t) for t in args.batches.split(",")] if args.batches else list(shape.batches))
    log(f"[bench] generating {shape.name} weights")
    host = HostLayer(shape, shared=shape.n_shared > 0)
    dev_w0, dev_sh0 = dev_layer(shape, host, B)
    host.wg = host.wu = host.wd = host.shared = None     # device copies suffice from here on
    torch.cuda.synchronize()
    paths = [p for p in args.paths.split(",") if p]
    assert paths and all(p in ("sparse", "dense", "auto", "dense-pk", "auto-pk")
                         for p in paths), args.paths
    rows = []
    for T in batches:
        row = {"T": T}
        for path in paths:
            wl, res = measure(shape, host, dev_w0, T, args, path=path.split("-")[0],
                              dev_sh0=dev_sh0, sparsity_shared=args.sparsity_shared,
                              packed_down=path.endswith("-pk"))
            kern = {k: round(v["per_step_us"], 2) for k, v in res["kernels"].items()}
            ent = {"us_per_call": round(res["us_per_call"], 2),
                   "us_per_token": round(res["us_per_token"], 3),
                   "layer_bytes": int(res["layer_bytes"]),
                   "hbm_gbs": round(res["hbm_gbs"], 1),
                   "hbm_frac": round(res["hbm_frac"], 4),
                   "active_experts": round(res["active_experts"], 2),
                   "down_bytes": int(res["down_bytes"]),
                   "kernels_us_per_step": kern}
            if path.startswith("dense") and "down_dense" in res["kernels"]:
                k = res["kernels"]["down_dense"]
                ent["down_dense_tflops"] = round(res["flops_down_dense"] / (k["per_step_us"] * 1e-6) / 1e12, 2)
            if "gateup_swiglu" in res["kernels"]:
                k = res["kernels"]["gateup_swiglu"]
                ent["gateup_tflops"] = round(res["flops_gateup"] / (k["per_step_us"] * 1e-6) / 1e12, 2)
            if path.startswith("auto"):   # the dispatcher's own choice, per routed / shared call
                ent["routed"] = res["auto_path"]
                if wl.desc_sh is not None:
                    ent["shared"] = "sparse" if wl.auto_path_sh == 0 else "dense"
            row[path] = ent
            log(f"[bench] {shape.name} T={T} {path}: {res['us_per_call']:.1f} us/call; kernels/step "
                + ", ".join(f"{k} {v}" for k, v in kern.items()))
            del wl
            torch.cuda.empty_cache()
        if "sparse" in row and "dense" in row:
            row["faster"] = ("sparse" if row["sparse"]["us_per_call"] <= row["dense"]["us_per_call"]
                             else "dense")
            best = min(row["sparse"]["us_per_call"], row["dense"]["us_per_call"])
            if "auto" in row:
                row["auto_vs_best"] = round(row["auto"]["us_per_call"] / best, 3)
        if "dense" in row and "dense-pk" in row:
            row["dense_pk_vs_dense"] = round(row["dense-pk"]["us_per_call"] /
                                             row["dense"]["us_per_call"], 3)
        rows.append(row)
    print(json.dumps({"metric": "sparse-vs-dense crossover: MoE-layer us/call per forced path",
                      "layer": shape.name, "sparsity": args.sparsity,
                      "sparsity_shared": (args.sparsity if args.sparsity_shared is None
                                          else args.sparsity_shared),
                      "steps": args.steps, "warmup": args.warmup, "launch": "hip-graph replay per step",
                      "rows": rows}), flush=True)


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU: the layer is a single-GPU kernel path and this build "
              f"has no multi-GPU mode (asked for --gpus {args.gpus}, WORLD_SIZE {world}).",
              file=sys.stderr)
        sys.exit(2)
    import torch
    import moe_synth as S
    from sparse_moe_expert_route_amd import binding as B

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    B.lib()
    if args.crossover:
        crossover(args)
        return
    shape = S.LAYERS[LAYER]
    log(f"[bench] generating {LAYER} weights")
    host = HostLayer(shape)
    dev_w0, _ = dev_layer(shape, host, B)
    torch.cuda.synchronize()
    sweep = [] if args.sweep == "none" else [int(t) for t in args.sweep.split(",") if t]
    batches = {}
    main_wl, main_res = None, None
    for T in sorted(set(sweep + [args.batch])):
        wl, res = measure(shape, host, dev_w0, T, args)
        batches[str(T)] = {k: (round(v, 3) if isinstance(v, float) else v)
                           for k, v in res.items() if k != "kernels"}
        batches[str(T)]["kernels_us"] = {k: round(v["avg_us"], 2) for k, v in res["kernels"].items()}
        for stage, key, name in (("down_rows", "down_bytes", "down"),
                                 ("gateup_swiglu", "gateup_bytes", "gateup"),
                                 ("fused_ffn", "fused_bytes", "fused")):
            if stage in res["kernels"]:
                sm = size_matched_read(res[key])
                gbs = res[key] / (res["kernels"][stage]["avg_us"] * 1e-6) / 1e9
                batches[str(T)][f"{name}_vs_size_matched_read"] = {
                    f"{name}_gbs": round(gbs, 1), "read": sm, "frac": round(gbs / sm["gbs"], 4)}
        log(f"[bench] T={T}: {res['us_per_call']:.1f} us/call, {res['us_per_token']:.2f} us/token, "
            f"{res['hbm_gbs']:.0f} GB/s ({100 * res['hbm_frac']:.1f}% of 8 TB/s); kernels "
            + ", ".join(f"{k} {v['avg_us']:.1f}" for k, v in res["kernels"].items()))
        if T == args.batch:
            main_wl, main_res = wl, res
        else:
            del wl
            torch.cuda.empty_cache()

    log("[bench] practical read peak")
    practical = practical_read_peak()
    log(f"[bench] moe_stream_read: {practical['gbs']:.0f} GB/s")
    # the variants beside the headline (different masks, same layer):
    #   updown          the page's own split: gate-only scores, sparse up and down
    #   threshold       the page's literal mask on |h|: calibrated tau, counts vary
    #   updown_threshold the split with the threshold mask: the page's pipeline
    variants = {"updown": {}, "threshold": {}, "updown_threshold": {}}
    if not args.no_variant:
        dev_gate = (dev_w0[0], dev_w0[1], host.to_dev(host.wu), dev_w0[3])
        runs = (("updown", dev_gate, "gate"), ("threshold", dev_w0, "threshold"),
                ("updown_threshold", dev_gate, "gate_threshold"))
        for name, weights, score in runs:
            for T in sorted(set(sweep + [args.batch])):
                wl, res = measure(shape, host, weights, T, args, score=score)
                variants[name][str(T)] = {
                    "us_per_call": round(res["us_per_call"], 3),
                    "us_per_token": round(res["us_per_token"], 3),
                    "mean_kept": round(res["mean_kept"], 1),
                    "layer_bytes": int(res["layer_bytes"]),
                    "hbm_gbs": round(res["hbm_gbs"], 1),
                    "kernels_us": {k: round(v["avg_us"], 2) for k, v in res["kernels"].items()}}
                log(f"[bench] {name} T={T}: {res['us_per_call']:.1f} us/call, "
                    f"{res['us_per_token']:.2f} us/token, mean kept {res['mean_kept']:.1f}; kernels "
                    + ", ".join(f"{k} {v['avg_us']:.1f}" for k, v in res["kernels"].items()))
                del wl
                torch.cuda.empty_cache()
        del dev_gate
    # the layer across the sparsity sweep of this workload (s = 0 is the
    # unmasked dense SwiGLU MoE, which the dispatcher sends to the dense path)
    sweep_s = {}
    if not args.no_variant:
        for s in (0.0, 0.5, 0.75):
            for T in (1, args.batch):
                wl, res = measure(shape, host, dev_w0, T, args, sparsity=s)
                sweep_s[f"s={s},T={T}"] = {"k": res["k"], "path": res["path"],
                                           "us_per_call": round(res["us_per_call"], 3),
                                           "us_per_token": round(res["us_per_token"], 3)}
                log(f"[bench] sparsity {s} T={T}: k={res['k']} {res['path']}, "
                    f"{res['us_per_call']:.1f} us/call")
                del wl
                torch.cuda.empty_cache()
    roster = step = None
    if not args.no_variant:
        roster = roster_variant(shape, host, dev_w0)
        log("[bench] decode step through 8 layers")
        step = decode_step_variant(shape, args)
        log(f"[bench] decode step: {step}")
        log(f"[bench] roster: select {roster['select_us']}, working set {roster['working_set']}")
    cpu = None
    if not args.no_cpu:
        log("[bench] timing the CPU oracle")
        cpu = cpu_baseline(shape, host, main_wl, args.cpu_seconds)
    r = main_res
    line = {
        "metric": "MoE-layer us/token + achieved HBM GB/s (% of peak) at batch 1-16, 90% sparsity",
        "value": round(r["us_per_token"], 3),
        "unit": "us/token",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(r["us_per_call"] / 1e3, 5),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{LAYER} MoE layer: hidden 2048, 64 routed experts, d_ff 1024, "
                               f"top-8, bf16 weights/tokens with fp32 accumulation, "
                               f"sparsity {args.sparsity} (k={r['k']}), batch {args.batch} tokens",
                   "batch": args.batch, "sparsity": args.sparsity, "k_keep": r["k"],
                   "path": r["path"], "launch": "hip-graph replay per step",
                   "weight_copies": r["copies"], "global_batch": args.batch},
        "tokens_per_s": round(r["tokens_per_s"], 1),
        "hbm_gbs": round(r["hbm_gbs"], 1),
        "hbm_frac": round(r["hbm_frac"], 4),
        "layer_bytes": int(r["layer_bytes"]),
        "roofline": (roofline(r, "fused_ffn", "fused_bytes", practical,
                              size_matched_read(r["fused_bytes"]))
                     if "fused_ffn" in r["kernels"] else
                     roofline(r, "gateup_swiglu", "gateup_bytes", practical,
                              size_matched_read(r["gateup_bytes"]))),
        "roofline_down": roofline(r, "down_rows", "down_bytes", practical,
                                  size_matched_read(r["down_bytes"])),
        "down_target": down_target(batches),
        "practical_read_peak": practical,
        "event_overhead": event_pair_overhead(),
        "updown_variant": {"what": "the page's own split: dense gate scores |silu(W_g x)|, "
                                   "up and down gathered on the kept rows (a different mask)",
                           "batches": variants["updown"]} if variants["updown"] else None,
        "threshold_variant": {"what": "the page's literal mask: keep |h| > tau[e], tau per expert "
                                      f"calibrated for sparsity {args.sparsity} on {CAL_TOKENS} "
                                      f"tokens of seed {CAL_SEED}; kept count varies per pair",
                              "batches": variants["threshold"]} if variants["threshold"] else None,
        "updown_threshold_variant": {
            "what": "the page's pipeline: dense gate scores, keep |silu(g)| > tau[e] (calibrated "
                    f"on the gate scores, sparsity {args.sparsity}), up and down on the kept rows",
            "batches": variants["updown_threshold"]} if variants["updown_threshold"] else None,
        "sparsity_sweep": sweep_s or None,
        "roster_variant": roster,
        "decode_step_variant": step,
        "cpu_baseline": cpu,
        "batches": batches,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
