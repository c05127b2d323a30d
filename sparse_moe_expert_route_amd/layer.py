"""MoELayer: the decode MoE layer as a sequence of C-ABI calls.

route -> routed experts (sparse or dense path, overwriting y) -> always-on
shared experts (accumulating into y); on the sparse path the first two run
as one moe_layer_sparse call.  Torch provides device memory and the stream;
every step runs in libmoe_mi355x's kernels.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import binding as B


class MoELayer:
    def __init__(self, *, hidden: int, n_experts: int, d_ff: int, top_k: int, norm_topk: bool,
                 dtype: str, w_router, w_gate, w_up, w_down, bias=None,
                 shared: Optional[Sequence] = None, d_ff_shared: Optional[int] = None,
                 packed: bool = False, pack_down: bool = False):
        """Weights are device tensors [E, d_ff, H] (router [E, H]).  Gate and
        up are packed here with moe_pack_gate_up unless `packed` says the
        caller already did.  pack_down (bf16): also keep a copy of each W_d
        packed by moe_pack_down, which the dense path then reads (the sparse
        path reads the row-major one)."""
        self.desc = B.make_desc(hidden, n_experts, d_ff, top_k, norm_topk, dtype,
                                gate_up_layout="packed")
        self.w_router, self.bias = w_router, bias
        pk = (lambda d, w: w) if packed else B.moe_pack_gate_up
        self.w = (pk(self.desc, w_gate), pk(self.desc, w_up), w_down)
        pack_down = pack_down and dtype == "bf16"
        self.dense = (self.desc, self.w)   # descriptor and weights of the dense calls
        if pack_down:
            dd = B.make_desc(hidden, n_experts, d_ff, top_k, norm_topk, dtype,
                             gate_up_layout="packed", down_layout="packed")
            self.dense = (dd, (self.w[0], self.w[1], B.moe_pack_down(dd, w_down)))
        self.shared = None
        self.desc_shared = None
        if shared is not None:
            g, u, dn = shared
            n_sh = g.shape[0]
            d_sh = d_ff_shared or g.shape[1]
            self.desc_shared = B.make_desc(hidden, n_sh, d_sh, n_sh, False, dtype,
                                           gate_up_layout="packed")
            self.shared = (pk(self.desc_shared, g), pk(self.desc_shared, u), dn)
            self.dense_shared = (self.desc_shared, self.shared)
            if pack_down:
                ds = B.make_desc(hidden, n_sh, d_sh, n_sh, False, dtype, gate_up_layout="packed",
                                 down_layout="packed")
                self.dense_shared = (ds, (self.shared[0], self.shared[1], B.moe_pack_down(ds, dn)))
        self._ws = {}

    def _workspace(self, key, nbytes: int, device):
        buf = self._ws.get(key)
        if buf is None or buf.numel() < nbytes:
            buf = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
            self._ws[key] = buf
        return buf

    def select_path(self, T: int, k_keep: int, shared: bool = False) -> int:
        return B.moe_select_path(self.desc_shared if shared else self.desc, T, k_keep)

    def route(self, x, routing: Optional[B.Routing] = None) -> B.Routing:
        T = x.shape[0]
        d = self.desc
        routing = routing or B.Routing.allocate(T, d.top_k, d.n_experts, x.device)
        ws = self._workspace("route", B.moe_route_workspace_size(d, T), x.device)
        B.moe_route(d, T, x, self.w_router, self.bias, routing, ws)
        return routing

    def forward(self, x, k_keep: int, k_keep_shared: Optional[int] = None,
                path: Optional[int] = None, path_shared: Optional[int] = None,
                y=None, active_idx=None, routing: Optional[B.Routing] = None):
        """y [T, H] fp32 for tokens x [T, H]; k_keep kept neurons per pair."""
        T = x.shape[0]
        d = self.desc
        if y is None:
            y = torch.empty((T, d.hidden), dtype=torch.float32, device=x.device)
        path = self.select_path(T, k_keep) if path is None else path
        if path == B.MOE_PATH_SPARSE:   # route + routed FFN in one call
            routing = routing or B.Routing.allocate(T, d.top_k, d.n_experts, x.device)
            ws = self._workspace("layer", B.moe_layer_workspace_size(d, T, k_keep), x.device)
            B.moe_layer_sparse(d, T, k_keep, x, self.w_router, self.bias, *self.w, routing, y, 0,
                               active_idx, ws)
        else:
            routing = self.route(x, routing)
            ws = self._workspace(("ffn", path), B.moe_ffn_workspace_size(d, T, k_keep, path),
                                 x.device)
            dd, wd = self.dense
            B.moe_expert_ffn_dense(dd, T, k_keep, x, *wd, routing, y, 0, active_idx, ws)
        if self.shared is not None:
            ds = self.desc_shared
            ks = ds.d_ff if k_keep_shared is None else k_keep_shared
            ps = self.select_path(T, ks, shared=True) if path_shared is None else path_shared
            wss = self._workspace(("shared", ps), B.moe_ffn_workspace_size(ds, T, ks, ps), x.device)
            if ps == B.MOE_PATH_SPARSE:
                B.moe_expert_ffn_sparse(ds, T, ks, x, *self.shared, None, y, 1, None, wss)
            else:
                dd, wd = self.dense_shared
                B.moe_expert_ffn_dense(dd, T, ks, x, *wd, None, y, 1, None, wss)
        return y
