"""C ABI checks that need no GPU: the library loads, exports every function
the header declares, and rejects every invalid argument before it enqueues
anything (so no HIP call is made).  Pointers here are fake, aligned
integers: the calls must return on validation alone."""
import ctypes
import math
import os
import subprocess
from fractions import Fraction

import pytest

from oracle import moe_oracle as O
from sparse_moe_expert_route_amd import binding as B
from sparse_moe_expert_route_amd.build import LIB_PATH

L = B.lib()
FAKE = 0x7F0000000000          # 16-byte aligned, never dereferenced
MIS = FAKE + 4                 # misaligned


def test_exports_every_header_function():
    declared = B.header_functions()
    assert declared == sorted(B._SIGS)           # the binding covers the header
    out = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in declared:
        assert name in exported, name


def test_version_and_status_strings():
    assert "gfx950" in B.moe_version()
    for code, name in B.STATUS.items():
        assert B.moe_status_string(code) == name
    assert B.moe_status_string(99) == "MOE_ERR_UNKNOWN"


def _golden_keep():
    rows = []
    with open(os.path.join(os.path.dirname(__file__), "golden", "keep_counts.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                s, d, k = line.split()[:3]
                rows.append((float(s), int(d), int(k)))
    return rows


@pytest.mark.parametrize("s,d,k", _golden_keep())
def test_keep_count_golden(s, d, k):
    assert B.moe_keep_count(s, d) == k


def test_keep_count_matches_exact_rationals():
    for d in (512, 768, 1000, 1024, 1536, 8192):
        for m in range(1001):
            s = Fraction(m, 1000)
            assert B.moe_keep_count(float(s), d) == math.ceil((1 - s) * d) == O.keep_count(float(s), d)
    assert B.moe_keep_count(1.5, 64) == 0 and B.moe_keep_count(-0.5, 64) == 64
    assert B.moe_keep_count(float("nan"), 64) == -1 and B.moe_keep_count(0.5, -1) == -1


def _desc(**kw):
    base = dict(hidden=2048, n_experts=64, d_ff=1024, top_k=8, norm_topk=False, dtype="bf16",
                gate_up_layout="packed")
    base.update(kw)
    return B.make_desc(**base)


def test_select_path_is_shape_only_and_monotone(monkeypatch):
    monkeypatch.delenv("MOE_FORCE_PATH", raising=False)
    d = _desc(hidden=5120, n_experts=16, d_ff=8192, top_k=1)
    k = B.moe_keep_count(0.9, 8192)
    paths = [B.moe_select_path(d, T, k) for T in (1, 8, 64, 256, 1024)]
    assert paths[0] == B.MOE_PATH_SPARSE and paths[-1] == B.MOE_PATH_DENSE
    assert paths == sorted(paths)                         # switches once, sparse -> dense
    assert B.moe_select_path(d, 1, 8192) == B.MOE_PATH_DENSE   # no masking: dense rows
    monkeypatch.setenv("MOE_FORCE_PATH", "dense")
    assert B.moe_select_path(d, 1, k) == B.MOE_PATH_DENSE
    monkeypatch.setenv("MOE_FORCE_PATH", "sparse")
    assert B.moe_select_path(d, 1024, k) == B.MOE_PATH_SPARSE


def test_workspace_sizes():
    d = _desc()
    for path in (B.MOE_PATH_SPARSE, B.MOE_PATH_DENSE):
        sizes = [B.moe_ffn_workspace_size(d, T, 103, path) for T in (1, 2, 4, 16, 64, 1024)]
        assert all(s > 0 and s % 256 == 0 for s in sizes)
        assert sizes == sorted(sizes)
        # a workspace for T serves every smaller T
        assert all(B.moe_ffn_workspace_size(d, t, 103, path) <= sizes[-1] for t in range(1, 1025, 37))
    assert B.moe_ffn_workspace_size(d, 4, 2000, 0) == 0
    assert B.moe_ffn_workspace_size(_desc(hidden=100), 4, 10, 0) == 0
    assert B.moe_route_workspace_size(d, 16) >= 16 * 64 * 4


def test_layer_workspace_size_covers_every_call():
    # moe_workspace_size: one buffer for moe_route, the FFN call on the path
    # and (sparse) moe_layer_sparse, for any T up to T_max
    d = _desc()
    for path in (B.MOE_PATH_SPARSE, B.MOE_PATH_DENSE):
        for T in (1, 4, 16, 64, 1024):
            w = B.moe_workspace_size(d, T, 103, path)
            assert w > 0 and w % 256 == 0
            assert w >= B.moe_route_workspace_size(d, T)
            assert w >= B.moe_ffn_workspace_size(d, T, 103, path)
            if path == B.MOE_PATH_SPARSE:
                assert w >= B.moe_layer_workspace_size(d, T, 103)
            assert all(B.moe_workspace_size(d, t, 103, path) <= w for t in range(1, T + 1, 7))
    assert B.moe_workspace_size(d, 4, 2000, 0) == 0
    assert B.moe_workspace_size(d, 4, 10, 7) == 0
    assert B.moe_workspace_size(_desc(hidden=100), 4, 10, 0) == 0


ROWMAJOR_REFUSED = ["moe_expert_ffn_sparse", "moe_expert_ffn_dense", "moe_expert_ffn_sparse_updown"]


@pytest.mark.parametrize("fn_name", ROWMAJOR_REFUSED)
def test_rowmajor_gate_up_is_refused(fn_name):
    # a descriptor left at MOE_LAYOUT_ROWMAJOR (zero) never reaches a kernel:
    # the FFN calls read packed gate/up and say so instead of misreading
    fn = getattr(L, fn_name)
    assert _ffn(fn, _desc(gate_up_layout="rowmajor"), 4, 10) == UNS
    assert "moe_pack_gate_up" in B.moe_last_error()
    assert _ffn(fn, _desc(gate_up_layout=7), 4, 10) == INV
    assert _ffn(fn, _desc(), 4, 10) != UNS      # packed: validation goes on (fake pointers)


def test_rowmajor_refused_by_the_other_ffn_calls():
    d = _desc(gate_up_layout="rowmajor")
    r = B.MoeRouting(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert L.moe_expert_ffn_sparse_residual(ctypes.byref(d), 4, 10, FAKE, FAKE, FAKE, FAKE,
                                            ctypes.byref(r), FAKE, 0, None, FAKE, FAKE, FAKE,
                                            1 << 34, None) == UNS
    assert L.moe_layer_sparse(ctypes.byref(d), 4, 10, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                              ctypes.byref(r), FAKE, 0, None, None, None, FAKE, 1 << 34, None) == UNS
    for name in ("moe_expert_ffn_sparse_threshold", "moe_expert_ffn_sparse_updown_threshold"):
        assert getattr(L, name)(ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(r),
                                FAKE, 0, None, None, FAKE, 1 << 34, None) == UNS
    assert L.moe_calibrate_thresholds(ctypes.byref(d), 4, FAKE, FAKE, FAKE, ctypes.byref(r), 0.9,
                                      FAKE, FAKE, 1 << 34, None) == UNS
    assert L.moe_calibrate_thresholds_gate(ctypes.byref(d), 4, FAKE, FAKE, ctypes.byref(r), 0.9,
                                           FAKE, FAKE, 1 << 34, None) == UNS
    # the router does not read gate/up: a row-major descriptor validates there
    assert _route(d, 4, wsb=0) == WSP


def test_packed_down_only_on_the_dense_bf16_call():
    # moe_pack_down's layout is read by the dense bf16 down GEMM alone; the
    # sparse calls gather row-major W_d rows and refuse it before any launch
    d = _desc(down_layout="packed")
    for name in ("moe_expert_ffn_sparse", "moe_expert_ffn_sparse_updown"):
        assert _ffn(getattr(L, name), d, 4, 10) == UNS, name
        assert "moe_pack_down" in B.moe_last_error()
    r = B.MoeRouting(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    assert L.moe_layer_sparse(ctypes.byref(d), 4, 10, FAKE, FAKE, None, FAKE, FAKE, FAKE,
                              ctypes.byref(r), FAKE, 0, None, None, None, FAKE, 1 << 34, None) == UNS
    for name in ("moe_expert_ffn_sparse_threshold", "moe_expert_ffn_sparse_updown_threshold"):
        assert getattr(L, name)(ctypes.byref(d), 4, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(r),
                                FAKE, 0, None, None, FAKE, 1 << 34, None) == UNS
    assert _ffn(L.moe_expert_ffn_dense, _desc(down_layout="packed", dtype="f32"), 4, 10) == UNS
    assert _ffn(L.moe_expert_ffn_dense, _desc(down_layout=7), 4, 10) == INV
    # the dense bf16 call validates on (fake pointers: stops at the workspace)
    assert _ffn(L.moe_expert_ffn_dense, d, 4, 10, wsb=0) == WSP
    # calibration reads no W_d: the packed descriptor is fine there
    assert L.moe_calibrate_thresholds(ctypes.byref(d), 4, FAKE, FAKE, FAKE, ctypes.byref(r), 0.9,
                                      FAKE, FAKE, 0, None) == WSP


def test_pack_down_validation():
    d = _desc(down_layout="packed")
    assert L.moe_pack_down(ctypes.byref(_desc(dtype="f32")), FAKE, FAKE + (1 << 32), None) == UNS
    assert L.moe_pack_down(ctypes.byref(d), FAKE, FAKE + 64, None) == INV       # overlap
    assert L.moe_unpack_down(ctypes.byref(d), FAKE, None, None) == INV
    assert L.moe_pack_down(ctypes.byref(d), MIS, FAKE + (1 << 32), None) == MISA
    assert L.moe_pack_down(None, FAKE, FAKE + (1 << 32), None) == INV


def _route(d, T, x=FAKE, w=FAKE, bias=None, out="ok", ws=FAKE, wsb=1 << 30):
    r = B.MoeRouting(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) if out == "ok" else out
    return L.moe_route(ctypes.byref(d) if d is not None else None, T, x, w, bias,
                       ctypes.byref(r) if r is not None else None, ws, wsb, None)


def _ffn(fn, d, T, k, x=FAKE, wg=FAKE, wu=FAKE, wd=FAKE, routing="ok", y=FAKE, acc=0, idx=None,
         ws=FAKE, wsb=1 << 34):
    r = B.MoeRouting(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) if routing == "ok" else routing
    return fn(ctypes.byref(d) if d is not None else None, T, k, x, wg, wu, wd,
              ctypes.byref(r) if r is not None else None, y, acc, idx, ws, wsb, None)


INV, MISA, WSP, UNS = 1, 2, 3, 4


@pytest.mark.parametrize("fn_name", ["moe_expert_ffn_sparse", "moe_expert_ffn_dense",
                                     "moe_expert_ffn_sparse_updown"])
def test_ffn_validation(fn_name):
    fn = getattr(L, fn_name)
    d = _desc()
    assert _ffn(fn, None, 4, 10) == INV
    assert _ffn(fn, _desc(top_k=65), 4, 10) == INV
    assert _ffn(fn, _desc(hidden=100), 4, 10) == UNS
    assert _ffn(fn, _desc(d_ff=96), 4, 10) == UNS
    assert _ffn(fn, _desc(d_ff=16384), 4, 10) == UNS
    assert _ffn(fn, _desc(n_experts=2048), 4, 10) == UNS
    assert _ffn(fn, _desc(dtype=0).__class__(2048, 64, 1024, 8, 0, 7), 4, 10) == UNS
    assert _ffn(fn, _desc(norm_topk=False).__class__(2048, 64, 1024, 8, 2, 1), 4, 10) == INV
    assert _ffn(fn, d, -1, 10) == INV
    assert _ffn(fn, d, 1 << 20, 10) == UNS
    assert _ffn(fn, d, 4, -1) == INV
    assert _ffn(fn, d, 4, 1025) == INV
    assert _ffn(fn, d, 4, 10, acc=2) == INV
    assert _ffn(fn, d, 4, 10, routing=None) == INV          # always-on group needs top_k == E
    assert _ffn(fn, d, 4, 10, x=None) == INV
    assert _ffn(fn, d, 4, 10, wd=None) == INV
    assert _ffn(fn, d, 4, 10, y=None) == INV
    assert _ffn(fn, d, 4, 10, x=MIS) == MISA
    assert _ffn(fn, d, 4, 10, wg=MIS) == MISA
    assert _ffn(fn, d, 4, 10, idx=MIS) == MISA
    assert _ffn(fn, d, 4, 10, routing=B.MoeRouting(FAKE, FAKE, None, FAKE, FAKE, FAKE)) == INV
    assert _ffn(fn, d, 4, 10, routing=B.MoeRouting(FAKE, FAKE, FAKE, MIS, FAKE, FAKE)) == MISA
    assert _ffn(fn, d, 4, 10, ws=None) == WSP
    assert _ffn(fn, d, 4, 10, ws=MIS) == MISA
    path = 0 if "sparse" in fn_name else 1
    need = B.moe_ffn_workspace_size(d, 4, 10, path)
    assert _ffn(fn, d, 4, 10, wsb=need - 1) == WSP
    assert "workspace" in B.moe_last_error()
    # T == 0 is a valid no-op, even with NULL tensors
    assert _ffn(fn, d, 0, 10, x=None, y=None, ws=None) == 0
    assert B.moe_last_error() == ""


def test_ffn_residual_validation():
    fn = L.moe_expert_ffn_sparse_residual
    d = _desc()

    def R(T=4, k=10, xr=FAKE, xn=FAKE, x=FAKE, ws=FAKE, acc=0):
        r = B.MoeRouting(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
        return fn(ctypes.byref(d), T, k, x, FAKE, FAKE, FAKE, ctypes.byref(r), FAKE, acc, None,
                  xr, xn, ws, 1 << 34, None)
    assert R(xr=None) == INV
    assert R(xn=None) == INV
    assert R(xr=MIS) == MISA
    assert R(xn=MIS) == MISA
    assert "x_res" in B.moe_last_error()
    # the rest is validated as for moe_expert_ffn_sparse
    assert R(k=-1) == INV
    assert R(x=None) == INV
    assert R(acc=2) == INV
    assert R(ws=None) == WSP
    assert R(T=0, xr=None, xn=None, x=None, ws=None) == 0


def test_layer_validation():
    fn = L.moe_layer_sparse
    d = _desc()

    def Ly(dd=d, T=4, k=10, x=FAKE, wr=FAKE, bias=None, wg=FAKE, wd=FAKE, out="ok", y=FAKE,
           acc=0, xr=None, xn=None, ws=FAKE, wsb=1 << 34):
        r = B.MoeRouting(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE) if out == "ok" else out
        return fn(ctypes.byref(dd) if dd is not None else None, T, k, x, wr, bias, wg, FAKE, wd,
                  ctypes.byref(r) if r is not None else None, y, acc, None, xr, xn, ws, wsb, None)
    assert Ly(xr=FAKE) == INV                   # x_res and x_next: both or neither
    assert Ly(xn=FAKE) == INV
    assert Ly(xr=MIS, xn=FAKE) == MISA
    assert Ly(dd=None) == INV
    assert Ly(T=-1) == INV
    assert Ly(k=-1) == INV
    assert Ly(k=1025) == INV
    assert Ly(x=None) == INV
    assert Ly(wr=None) == INV
    assert Ly(wd=None) == INV
    assert Ly(y=None) == INV
    assert Ly(out=None) == INV
    assert Ly(out=B.MoeRouting(FAKE, None, FAKE, FAKE, FAKE, FAKE)) == INV
    assert Ly(bias=MIS + 1) == MISA
    assert Ly(acc=2) == INV
    assert Ly(ws=None) == WSP
    assert Ly(ws=MIS) == MISA
    need = B.moe_layer_workspace_size(d, 4, 10)
    assert need >= B.moe_route_workspace_size(d, 4) + B.moe_ffn_workspace_size(d, 4, 10, 0)
    assert Ly(wsb=need - 1) == WSP
    assert B.moe_layer_workspace_size(d, 4, 1025) == 0
    assert Ly(T=0, x=None, y=None, ws=None) == 0


def test_threshold_and_calibration_validation():
    d = _desc()
    r = B.MoeRouting(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    ws = B.moe_ffn_threshold_workspace_size(d, 4)
    assert ws > B.moe_ffn_workspace_size(d, 4, 1024, 0) - 1
    F = lambda dd, tau=FAKE, counts=None, wsb=ws: L.moe_expert_ffn_sparse_threshold(
        ctypes.byref(dd), 4, tau, FAKE, FAKE, FAKE, FAKE, ctypes.byref(r), FAKE, 0, counts, None,
        FAKE, wsb, None)
    assert F(d, tau=None) == INV
    assert F(d, tau=FAKE + 2) == MISA
    assert F(d, counts=FAKE + 2) == MISA
    assert F(d, wsb=ws - 1) == WSP
    assert F(_desc(d_ff=2112)) == UNS            # no register layout for this width
    C = lambda dd, s=0.9, tau=FAKE, wsb=1 << 34: L.moe_calibrate_thresholds(
        ctypes.byref(dd), 4, FAKE, FAKE, FAKE, ctypes.byref(r), s, tau, FAKE, wsb, None)
    assert C(d, s=1.5) == INV
    assert C(d, s=float("nan")) == INV
    assert C(d, tau=None) == INV
    assert C(d, wsb=B.moe_calibrate_workspace_size(d, 4) - 1) == WSP
    assert C(_desc(d_ff=2112)) == UNS
    assert B.moe_calibrate_workspace_size(_desc(hidden=100), 4) == 0
    # the split with thresholds, and calibration on the gate scores (no w_up)
    U = lambda dd, tau=FAKE, wu=FAKE, wsb=ws: L.moe_expert_ffn_sparse_updown_threshold(
        ctypes.byref(dd), 4, tau, FAKE, FAKE, wu, FAKE, ctypes.byref(r), FAKE, 0, None, None,
        FAKE, wsb, None)
    assert U(d, tau=None) == INV
    assert U(d, tau=FAKE + 2) == MISA
    assert U(d, wu=None) == INV
    assert U(d, wsb=ws - 1) == WSP
    assert U(_desc(d_ff=2112)) == UNS
    CG = lambda dd, s=0.9, tau=FAKE, wsb=1 << 34: L.moe_calibrate_thresholds_gate(
        ctypes.byref(dd), 4, FAKE, FAKE, ctypes.byref(r), s, tau, FAKE, wsb, None)
    assert CG(d, s=-0.1) == INV
    assert CG(d, tau=None) == INV
    assert CG(d, wsb=B.moe_calibrate_workspace_size(d, 4) - 1) == WSP
    assert CG(_desc(d_ff=2112)) == UNS


def test_pack_validation():
    d = _desc()
    nbytes = 64 * 1024 * 2048 * 2
    P = L.moe_pack_gate_up
    assert P(None, FAKE, FAKE + nbytes, None) == INV
    assert P(ctypes.byref(d), None, FAKE + nbytes, None) == INV
    assert P(ctypes.byref(d), MIS, FAKE + nbytes, None) == MISA
    assert P(ctypes.byref(d), FAKE, FAKE + nbytes - 4096, None) == INV     # overlap
    assert L.moe_unpack_gate_up(ctypes.byref(_desc(hidden=96)), FAKE, FAKE + nbytes, None) == UNS


def test_stream_read_validation():
    S = L.moe_stream_read
    assert S(None, 64, FAKE, None) == INV
    assert S(FAKE, 64, None, None) == INV
    assert S(FAKE, 0, FAKE, None) == INV
    assert S(FAKE, 72, FAKE, None) == INV
    assert S(MIS, 64, FAKE, None) == MISA
    assert S(FAKE, 64, MIS, None) == MISA


def test_route_validation():
    d = _desc()
    assert _route(None, 4) == INV
    assert _route(d, 4, out=None) == INV
    assert _route(d, -3) == INV
    assert _route(d, 4, x=None) == INV
    assert _route(d, 4, w=MIS) == MISA
    assert _route(d, 4, bias=FAKE + 2) == MISA
    assert _route(d, 4, out=B.MoeRouting(FAKE, None, FAKE, FAKE, FAKE, FAKE)) == INV
    assert _route(d, 4, ws=None) == WSP
    assert _route(d, 4, wsb=B.moe_route_workspace_size(d, 4) - 1) == WSP
    assert _route(d, 0, x=None) == 0


def test_residual_validation():
    d = _desc()
    Rz = lambda dd=d, T=4, x=FAKE, y=FAKE, o=FAKE: L.moe_residual_add(
        ctypes.byref(dd) if dd is not None else None, T, x, y, o, None)
    assert Rz(dd=None) == INV
    assert Rz(T=-1) == INV
    assert Rz(x=None) == INV
    assert Rz(y=None) == INV
    assert Rz(o=None) == INV
    assert Rz(x=MIS) == MISA
    assert Rz(y=MIS) == MISA
    assert Rz(o=MIS) == MISA
    assert Rz(T=0, x=None, y=None, o=None) == 0


def test_route_roster_validation():
    d = _desc()                       # 64 experts, top-8
    out = B.MoeRouting(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)
    ws = B.moe_route_workspace_size(d, 4)
    R = lambda usage=FAKE, pinned=None, m=8, delta=1.0, dd=d: L.moe_route_roster(
        ctypes.byref(dd), 4, FAKE, FAKE, None, usage, pinned, m, ctypes.c_float(delta),
        ctypes.byref(out), FAKE, ws, None)
    assert R(usage=None) == INV
    assert R(usage=FAKE + 2) == MISA
    assert R(pinned=FAKE + 2) == MISA
    assert R(m=0) == INV
    assert R(m=65) == INV
    assert R(pinned=FAKE, m=7) == INV             # pinned rows need m >= top_k
    assert R(delta=-1.0) == INV
    assert R(delta=float("nan")) == INV
    assert R(delta=float("inf")) == INV
    assert R(dd=_desc(hidden=100)) == UNS
