"""ctypes binding of libmoe_mi355x.so (include/moe_mi355x.h).

Argument marshalling only: torch tensors supply device pointers, the
current torch stream supplies the HIP stream, and every step of the layer
runs in the library's kernels.  If the library is not built, loading fails
loudly; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
import re
from dataclasses import dataclass
from typing import Optional

from .build import INCLUDE, LIB_PATH

MOE_F32, MOE_BF16 = 0, 1
MOE_PATH_SPARSE, MOE_PATH_DENSE = 0, 1
MOE_LAYOUT_ROWMAJOR, MOE_LAYOUT_PACKED = 0, 1
STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID_ARG", 2: "MOE_ERR_MISALIGNED", 3: "MOE_ERR_WORKSPACE",
          4: "MOE_ERR_UNSUPPORTED", 5: "MOE_ERR_HIP"}
HEADER = os.path.join(INCLUDE, "moe_mi355x.h")


class MoeError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{STATUS.get(status, status)}: {detail}")
        self.status = status
        self.detail = detail


class MoeDesc(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("n_experts", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("norm_topk", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("gate_up_layout", ctypes.c_int32), ("down_layout", ctypes.c_int32)]


class MoeRouting(ctypes.Structure):
    _fields_ = [("topk_ids", ctypes.c_void_p), ("topk_w", ctypes.c_void_p),
                ("expert_offsets", ctypes.c_void_p), ("pair_by_expert", ctypes.c_void_p),
                ("active_experts", ctypes.c_void_p), ("n_active", ctypes.c_void_p)]


_V, _I32, _SZ, _D = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t, ctypes.c_double
_PD, _PR = ctypes.POINTER(MoeDesc), ctypes.POINTER(MoeRouting)
_SIGS = {
    "moe_route": (_I32, [_PD, _I32, _V, _V, _V, _PR, _V, _SZ, _V]),
    "moe_residual_add": (_I32, [_PD, _I32, _V, _V, _V, _V]),
    "moe_expert_ffn_sparse_updown_threshold": (_I32, [_PD, _I32, _V, _V, _V, _V, _V, _PR, _V, _I32,
                                                      _V, _V, _V, _SZ, _V]),
    "moe_calibrate_thresholds_gate": (_I32, [_PD, _I32, _V, _V, _PR, _D, _V, _V, _SZ, _V]),
    "moe_route_roster": (_I32, [_PD, _I32, _V, _V, _V, _V, _V, _I32, ctypes.c_float, _PR, _V, _SZ,
                                _V]),
    "moe_expert_ffn_sparse": (_I32, [_PD, _I32, _I32, _V, _V, _V, _V, _PR, _V, _I32, _V, _V, _SZ, _V]),
    "moe_expert_ffn_sparse_residual": (_I32, [_PD, _I32, _I32, _V, _V, _V, _V, _PR, _V, _I32, _V,
                                              _V, _V, _V, _SZ, _V]),
    "moe_layer_sparse": (_I32, [_PD, _I32, _I32, _V, _V, _V, _V, _V, _V, _PR, _V, _I32, _V, _V,
                                _V, _V, _SZ, _V]),
    "moe_layer_workspace_size": (_SZ, [_PD, _I32, _I32]),
    "moe_layer_sparse_noalloc": (_I32, [_PD, _I32, _I32, _V, _V, _V, _V, _V, _V, _PR, _V, _I32,
                                        _V, _V, _V, _V]),
    "moe_expert_ffn_dense": (_I32, [_PD, _I32, _I32, _V, _V, _V, _V, _PR, _V, _I32, _V, _V, _SZ, _V]),
    "moe_expert_ffn_sparse_updown": (_I32, [_PD, _I32, _I32, _V, _V, _V, _V, _PR, _V, _I32, _V, _V, _SZ, _V]),
    "moe_expert_ffn_sparse_threshold": (_I32, [_PD, _I32, _V, _V, _V, _V, _V, _PR, _V, _I32, _V, _V, _V, _SZ, _V]),
    "moe_calibrate_thresholds": (_I32, [_PD, _I32, _V, _V, _V, _PR, _D, _V, _V, _SZ, _V]),
    "moe_ffn_threshold_workspace_size": (_SZ, [_PD, _I32]),
    "moe_calibrate_workspace_size": (_SZ, [_PD, _I32]),
    "moe_pack_gate_up": (_I32, [_PD, _V, _V, _V]),
    "moe_unpack_gate_up": (_I32, [_PD, _V, _V, _V]),
    "moe_pack_down": (_I32, [_PD, _V, _V, _V]),
    "moe_unpack_down": (_I32, [_PD, _V, _V, _V]),
    "moe_route_workspace_size": (_SZ, [_PD, _I32]),
    "moe_ffn_workspace_size": (_SZ, [_PD, _I32, _I32, _I32]),
    "moe_workspace_size": (_SZ, [_PD, _I32, _I32, _I32]),
    "moe_keep_count": (_I32, [_D, _I32]),
    "moe_select_path": (_I32, [_PD, _I32, _I32]),
    "moe_timer_attach": (_I32, [ctypes.POINTER(_V), ctypes.POINTER(_I32), _I32]),
    "moe_timer_detach": (_I32, []),
    "moe_stream_read": (_I32, [_V, _SZ, _V, _V]),
    "moe_status_string": (ctypes.c_char_p, [_I32]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_version": (ctypes.c_char_p, []),
}

_lib = None


def header_functions():
    """Names of the functions include/moe_mi355x.h declares."""
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_]+)\s*\(", text)))


def lib() -> ctypes.CDLL:
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: build it with `python -m sparse_moe_expert_route_amd.build` "
                "(the layer has no fallback)")
        # torch ships its own HIP runtime under the same soname; loading torch
        # first makes this library bind to that one, so the process holds a
        # single runtime (two runtimes in one process do not share devices).
        import torch  # noqa: F401
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def _check(status: int):
    if status != 0:
        raise MoeError(status, lib().moe_last_error().decode())


def make_desc(hidden, n_experts, d_ff, top_k, norm_topk, dtype,
              gate_up_layout="rowmajor", down_layout="rowmajor") -> MoeDesc:
    """moe_desc; gate_up_layout says how w_gate / w_up are passed to the FFN
    calls ("packed" after moe_pack_gate_up; "rowmajor" ones are refused);
    down_layout how w_down is ("packed" after moe_pack_down: the dense bf16
    call only)."""
    dt = {"f32": MOE_F32, "bf16": MOE_BF16, MOE_F32: MOE_F32, MOE_BF16: MOE_BF16}[dtype]
    lay = {"rowmajor": MOE_LAYOUT_ROWMAJOR, "packed": MOE_LAYOUT_PACKED,
           MOE_LAYOUT_ROWMAJOR: MOE_LAYOUT_ROWMAJOR, MOE_LAYOUT_PACKED: MOE_LAYOUT_PACKED}
    return MoeDesc(int(hidden), int(n_experts), int(d_ff), int(top_k), int(bool(norm_topk)), dt,
                   lay.get(gate_up_layout, gate_up_layout), lay.get(down_layout, down_layout))


# ------------------------------------------------------------ tensor marshalling

def _ptr(t) -> Optional[int]:
    if t is None:
        return None
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError("tensors passed to the HIP library must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the HIP library must be contiguous")
    return t.data_ptr()


def _stream(stream) -> int:
    import torch
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


@dataclass
class Routing:
    """Device buffers of one token batch's routing (moe_routing)."""
    topk_ids: "object"
    topk_w: "object"
    expert_offsets: "object"
    pair_by_expert: "object"
    active_experts: "object"
    n_active: "object"

    @classmethod
    def allocate(cls, T: int, top_k: int, n_experts: int, device="cuda"):
        import torch
        P = max(1, T * top_k)
        i32 = dict(dtype=torch.int32, device=device)
        return cls(torch.empty((max(T, 1), top_k), **i32),
                   torch.empty((max(T, 1), top_k), dtype=torch.float32, device=device),
                   torch.empty(n_experts + 1, **i32), torch.empty(P, **i32),
                   torch.empty(n_experts, **i32), torch.empty(1, **i32))

    def as_c(self) -> MoeRouting:
        return MoeRouting(*(_ptr(getattr(self, f)) for f, _ in MoeRouting._fields_))


# ------------------------------------------------------------ the C entry points

def moe_route(desc: MoeDesc, T: int, x, w_router, bias, routing: Routing, workspace, stream=None):
    r = routing.as_c()
    ws = _ptr(workspace)
    _check(lib().moe_route(ctypes.byref(desc), int(T), _ptr(x), _ptr(w_router), _ptr(bias),
                           ctypes.byref(r), ws, workspace.numel() * workspace.element_size() if ws else 0,
                           _stream(stream)))


def moe_route_roster(desc: MoeDesc, T: int, x, w_router, bias, usage, pinned, roster_size: int,
                     delta: float, routing: Routing, workspace, stream=None):
    """moe_route with the roster bias; usage [T, E] int32 is updated in place."""
    r = routing.as_c()
    ws = _ptr(workspace)
    _check(lib().moe_route_roster(ctypes.byref(desc), int(T), _ptr(x), _ptr(w_router), _ptr(bias),
                                  _ptr(usage), _ptr(pinned), int(roster_size), float(delta),
                                  ctypes.byref(r), ws,
                                  workspace.numel() * workspace.element_size() if ws else 0,
                                  _stream(stream)))


def moe_residual_add(desc: MoeDesc, T: int, x_in, y, x_out, stream=None):
    """x_out = x_in + y rounded to the layer dtype (x_out may be x_in)."""
    _check(lib().moe_residual_add(ctypes.byref(desc), int(T), _ptr(x_in), _ptr(y), _ptr(x_out),
                                  _stream(stream)))


def _ffn(fn, desc, T, k_keep, x, w_gate, w_up, w_down, routing, y, accumulate, active_idx_out,
         workspace, stream):
    r = routing.as_c() if routing is not None else None
    ws = _ptr(workspace)
    _check(fn(ctypes.byref(desc), int(T), int(k_keep), _ptr(x), _ptr(w_gate), _ptr(w_up),
              _ptr(w_down), ctypes.byref(r) if r is not None else None, _ptr(y), int(accumulate),
              _ptr(active_idx_out), ws,
              workspace.numel() * workspace.element_size() if ws else 0, _stream(stream)))


def moe_expert_ffn_sparse(desc, T, k_keep, x, w_gate, w_up, w_down, routing, y, accumulate=0,
                          active_idx_out=None, workspace=None, stream=None):
    _ffn(lib().moe_expert_ffn_sparse, desc, T, k_keep, x, w_gate, w_up, w_down, routing, y,
         accumulate, active_idx_out, workspace, stream)


def moe_expert_ffn_sparse_residual(desc, T, k_keep, x, w_gate, w_up, w_down, routing, y, x_res,
                                   x_next, accumulate=0, active_idx_out=None, workspace=None,
                                   stream=None):
    """moe_expert_ffn_sparse, then x_next = x_res + y (rounded to the layer
    dtype) in the down projection's epilogue; the last FFN call of a layer."""
    r = routing.as_c() if routing is not None else None
    ws = _ptr(workspace)
    _check(lib().moe_expert_ffn_sparse_residual(
        ctypes.byref(desc), int(T), int(k_keep), _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
        ctypes.byref(r) if r is not None else None, _ptr(y), int(accumulate),
        _ptr(active_idx_out), _ptr(x_res), _ptr(x_next), ws,
        workspace.numel() * workspace.element_size() if ws else 0, _stream(stream)))


def moe_layer_sparse(desc, T, k_keep, x, w_router, bias, w_gate, w_up, w_down, routing, y,
                     accumulate=0, active_idx_out=None, workspace=None, stream=None, x_res=None,
                     x_next=None):
    """moe_route then moe_expert_ffn_sparse (or, with x_res and x_next, the
    residual-fused FFN) in one call; fused further at one token."""
    r = routing.as_c()
    ws = _ptr(workspace)
    _check(lib().moe_layer_sparse(
        ctypes.byref(desc), int(T), int(k_keep), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), ctypes.byref(r), _ptr(y), int(accumulate), _ptr(active_idx_out),
        _ptr(x_res), _ptr(x_next), ws, workspace.numel() * workspace.element_size() if ws else 0,
        _stream(stream)))


NOALLOC_SCRATCH_BYTES = 16 << 20


def moe_layer_sparse_noalloc(desc, T, k_keep, x, w_router, bias, w_gate, w_up, w_down, routing, y,
                             accumulate=0, active_idx_out=None, stream=None, x_res=None,
                             x_next=None):
    """moe_layer_sparse with the library's static per-device scratch as its
    workspace: nothing is allocated.  Calls that overlap on one GPU race."""
    r = routing.as_c()
    _check(lib().moe_layer_sparse_noalloc(
        ctypes.byref(desc), int(T), int(k_keep), _ptr(x), _ptr(w_router), _ptr(bias), _ptr(w_gate),
        _ptr(w_up), _ptr(w_down), ctypes.byref(r), _ptr(y), int(accumulate), _ptr(active_idx_out),
        _ptr(x_res), _ptr(x_next), _stream(stream)))


def moe_layer_workspace_size(desc, T, k_keep):
    return int(lib().moe_layer_workspace_size(ctypes.byref(desc), int(T), int(k_keep)))


def moe_expert_ffn_dense(desc, T, k_keep, x, w_gate, w_up, w_down, routing, y, accumulate=0,
                         active_idx_out=None, workspace=None, stream=None):
    _ffn(lib().moe_expert_ffn_dense, desc, T, k_keep, x, w_gate, w_up, w_down, routing, y,
         accumulate, active_idx_out, workspace, stream)


def moe_expert_ffn_sparse_updown(desc, T, k_keep, x, w_gate, w_up, w_down, routing, y,
                                 accumulate=0, active_idx_out=None, workspace=None, stream=None):
    """The gate-score split: w_gate packed, w_up and w_down row-major."""
    _ffn(lib().moe_expert_ffn_sparse_updown, desc, T, k_keep, x, w_gate, w_up, w_down, routing,
         y, accumulate, active_idx_out, workspace, stream)


def moe_expert_ffn_sparse_threshold(desc, T, tau, x, w_gate, w_up, w_down, routing, y,
                                    accumulate=0, counts_out=None, active_idx_out=None,
                                    workspace=None, stream=None):
    """Threshold masking: keep |h_j| > tau[e]; tau a device float32 [E]."""
    r = routing.as_c() if routing is not None else None
    ws = _ptr(workspace)
    _check(lib().moe_expert_ffn_sparse_threshold(
        ctypes.byref(desc), int(T), _ptr(tau), _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
        ctypes.byref(r) if r is not None else None, _ptr(y), int(accumulate), _ptr(counts_out),
        _ptr(active_idx_out), ws, workspace.numel() * workspace.element_size() if ws else 0,
        _stream(stream)))


def moe_calibrate_thresholds(desc, T, x, w_gate, w_up, routing, sparsity, tau_out,
                             workspace=None, stream=None):
    """Per-expert thresholds for a target sparsity from calibration tokens."""
    r = routing.as_c() if routing is not None else None
    ws = _ptr(workspace)
    _check(lib().moe_calibrate_thresholds(
        ctypes.byref(desc), int(T), _ptr(x), _ptr(w_gate), _ptr(w_up),
        ctypes.byref(r) if r is not None else None, float(sparsity), _ptr(tau_out), ws,
        workspace.numel() * workspace.element_size() if ws else 0, _stream(stream)))


def moe_expert_ffn_sparse_updown_threshold(desc, T, tau, x, w_gate, w_up, w_down, routing, y,
                                           accumulate=0, counts_out=None, active_idx_out=None,
                                           workspace=None, stream=None):
    """The split with threshold masks on the gate scores (w_up row-major)."""
    r = routing.as_c() if routing is not None else None
    ws = _ptr(workspace)
    _check(lib().moe_expert_ffn_sparse_updown_threshold(
        ctypes.byref(desc), int(T), _ptr(tau), _ptr(x), _ptr(w_gate), _ptr(w_up), _ptr(w_down),
        ctypes.byref(r) if r is not None else None, _ptr(y), int(accumulate), _ptr(counts_out),
        _ptr(active_idx_out), ws, workspace.numel() * workspace.element_size() if ws else 0,
        _stream(stream)))


def moe_calibrate_thresholds_gate(desc, T, x, w_gate, routing, sparsity, tau_out,
                                  workspace=None, stream=None):
    """Per-expert thresholds on the gate scores |silu(W_g x)|."""
    r = routing.as_c() if routing is not None else None
    ws = _ptr(workspace)
    _check(lib().moe_calibrate_thresholds_gate(
        ctypes.byref(desc), int(T), _ptr(x), _ptr(w_gate),
        ctypes.byref(r) if r is not None else None, float(sparsity), _ptr(tau_out), ws,
        workspace.numel() * workspace.element_size() if ws else 0, _stream(stream)))


def moe_ffn_threshold_workspace_size(desc: MoeDesc, T: int) -> int:
    return int(lib().moe_ffn_threshold_workspace_size(ctypes.byref(desc), int(T)))


def moe_calibrate_workspace_size(desc: MoeDesc, T: int) -> int:
    return int(lib().moe_calibrate_workspace_size(ctypes.byref(desc), int(T)))


def moe_pack_gate_up(desc: MoeDesc, src, dst=None, stream=None):
    """Pack a row-major gate or up tensor [E, d_ff, H]; returns dst."""
    import torch
    dst = torch.empty_like(src) if dst is None else dst
    _check(lib().moe_pack_gate_up(ctypes.byref(desc), _ptr(src), _ptr(dst), _stream(stream)))
    return dst


def moe_unpack_gate_up(desc: MoeDesc, src, dst=None, stream=None):
    """Inverse of moe_pack_gate_up; returns dst."""
    import torch
    dst = torch.empty_like(src) if dst is None else dst
    _check(lib().moe_unpack_gate_up(ctypes.byref(desc), _ptr(src), _ptr(dst), _stream(stream)))
    return dst


def moe_pack_down(desc: MoeDesc, src, dst=None, stream=None):
    """Pack a row-major bf16 down tensor [E, d_ff, H] for the dense call
    (desc.down_layout = packed); returns dst."""
    import torch
    dst = torch.empty_like(src) if dst is None else dst
    _check(lib().moe_pack_down(ctypes.byref(desc), _ptr(src), _ptr(dst), _stream(stream)))
    return dst


def moe_unpack_down(desc: MoeDesc, src, dst=None, stream=None):
    """Inverse of moe_pack_down; returns dst."""
    import torch
    dst = torch.empty_like(src) if dst is None else dst
    _check(lib().moe_unpack_down(ctypes.byref(desc), _ptr(src), _ptr(dst), _stream(stream)))
    return dst


def moe_route_workspace_size(desc: MoeDesc, T: int) -> int:
    return int(lib().moe_route_workspace_size(ctypes.byref(desc), int(T)))


def moe_ffn_workspace_size(desc: MoeDesc, T: int, k_keep: int, path: int) -> int:
    return int(lib().moe_ffn_workspace_size(ctypes.byref(desc), int(T), int(k_keep), int(path)))


def moe_workspace_size(desc: MoeDesc, T_max: int, k_keep: int, path: int) -> int:
    return int(lib().moe_workspace_size(ctypes.byref(desc), int(T_max), int(k_keep), int(path)))


def moe_keep_count(sparsity: float, d_ff: int) -> int:
    return int(lib().moe_keep_count(float(sparsity), int(d_ff)))


def moe_select_path(desc: MoeDesc, T: int, k_keep: int) -> int:
    return int(lib().moe_select_path(ctypes.byref(desc), int(T), int(k_keep)))


def moe_status_string(status: int) -> str:
    return lib().moe_status_string(int(status)).decode()


def moe_last_error() -> str:
    return lib().moe_last_error().decode()


def moe_version() -> str:
    return lib().moe_version().decode()


STREAM_READ_SINK_WORDS = 65536


def moe_stream_read(buf, sink, stream=None) -> None:
    """Measurement helper: one streaming read of every byte of `buf` (device
    tensor); `sink` is a device int32 tensor of STREAM_READ_SINK_WORDS."""
    assert sink.numel() * sink.element_size() >= 4 * STREAM_READ_SINK_WORDS
    _check(lib().moe_stream_read(_ptr(buf), buf.numel() * buf.element_size(), _ptr(sink),
                                 _stream(stream)))


# ------------------------------------------------------------ per-kernel timing

class StageTimer:
    """Brackets every kernel the library launches with HIP timing events
    (moe_timer_attach), then reports per-stage durations.  Host-side
    plumbing for measurement; events come from the process's HIP runtime."""

    STAGES = ["router_logits", "router_topk", "route_group", "gateup_swiglu", "neuron_topk",
              "down_rows", "down_dense", "combine", "zero", "up_rows", "fused_ffn",
              "union_rows", "down_union"]

    def __init__(self, capacity: int):
        lib()
        self.hip = ctypes.CDLL("libamdhip64.so.7")   # the runtime already loaded by torch
        self.cap = int(capacity)
        self.events = (ctypes.c_void_p * (2 * self.cap))()
        self.stages = (ctypes.c_int32 * self.cap)()
        for i in range(2 * self.cap):
            rc = self.hip.hipEventCreate(ctypes.byref(self.events, i * ctypes.sizeof(ctypes.c_void_p)))
            if rc != 0:
                raise RuntimeError(f"hipEventCreate failed ({rc})")
        self.n = 0

    def __enter__(self):
        _check(lib().moe_timer_attach(self.events, self.stages, self.cap))
        return self

    def __exit__(self, *exc):
        self.n = lib().moe_timer_detach()
        return False

    def durations(self):
        """{stage name: [ms, ...]} of the recorded launches (synchronises)."""
        out = {}
        ms = ctypes.c_float()
        for i in range(self.n):
            self.hip.hipEventSynchronize(ctypes.c_void_p(self.events[2 * i + 1]))
            rc = self.hip.hipEventElapsedTime(ctypes.byref(ms), ctypes.c_void_p(self.events[2 * i]),
                                              ctypes.c_void_p(self.events[2 * i + 1]))
            if rc != 0:
                raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
            out.setdefault(self.STAGES[self.stages[i]], []).append(ms.value)
        return out

    def close(self):
        for i in range(2 * self.cap):
            self.hip.hipEventDestroy(ctypes.c_void_p(self.events[i]))
        self.cap = 0
