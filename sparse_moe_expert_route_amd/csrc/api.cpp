// C ABI of libmoe_mi355x.so: argument validation, workspace carve-up and
// launch sequencing.  Every check runs before anything is enqueued, so an
// error leaves the stream and all outputs untouched.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "moe_mi355x.h"
#include "internal.h"

namespace moe {
StageTimer &stage_timer() {
  static thread_local StageTimer t;
  return t;
}
}  // namespace moe

namespace {

thread_local char g_err[512] = "";

moe_status fail(moe_status s, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return s;
}

constexpr size_t kAlign = 256;
size_t up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

moe_status check_desc(const moe_desc *d) {
  if (!d) return fail(MOE_ERR_INVALID_ARG, "desc is NULL");
  if (d->dtype != MOE_F32 && d->dtype != MOE_BF16)
    return fail(MOE_ERR_UNSUPPORTED, "dtype %d is not MOE_F32 or MOE_BF16", d->dtype);
  if (d->hidden <= 0 || d->n_experts <= 0 || d->d_ff <= 0 || d->top_k <= 0)
    return fail(MOE_ERR_INVALID_ARG, "hidden, n_experts, d_ff and top_k must be positive");
  if (d->top_k > d->n_experts)
    return fail(MOE_ERR_INVALID_ARG, "top_k %d exceeds n_experts %d", d->top_k, d->n_experts);
  if (d->norm_topk != 0 && d->norm_topk != 1)
    return fail(MOE_ERR_INVALID_ARG, "norm_topk must be 0 or 1");
  if (d->gate_up_layout != MOE_LAYOUT_ROWMAJOR && d->gate_up_layout != MOE_LAYOUT_PACKED)
    return fail(MOE_ERR_INVALID_ARG, "gate_up_layout %d is not a moe_layout", d->gate_up_layout);
  if (d->down_layout != MOE_LAYOUT_ROWMAJOR && d->down_layout != MOE_LAYOUT_PACKED)
    return fail(MOE_ERR_INVALID_ARG, "down_layout %d is not a moe_layout", d->down_layout);
  if (d->hidden > MOE_MAX_HIDDEN || d->hidden % 64)
    return fail(MOE_ERR_UNSUPPORTED, "hidden %d: need a multiple of 64 up to %d", d->hidden,
                MOE_MAX_HIDDEN);
  if (d->d_ff > MOE_MAX_DFF || d->d_ff % 64)
    return fail(MOE_ERR_UNSUPPORTED, "d_ff %d: need a multiple of 64 up to %d", d->d_ff, MOE_MAX_DFF);
  if (d->n_experts > MOE_MAX_EXPERTS)
    return fail(MOE_ERR_UNSUPPORTED, "n_experts %d exceeds %d", d->n_experts, MOE_MAX_EXPERTS);
  if (d->top_k > MOE_MAX_TOPK)
    return fail(MOE_ERR_UNSUPPORTED, "top_k %d exceeds %d", d->top_k, MOE_MAX_TOPK);
  return MOE_OK;
}

moe_status check_T(int32_t T) {
  if (T < 0) return fail(MOE_ERR_INVALID_ARG, "T %d is negative", T);
  if (T > MOE_MAX_TOKENS) return fail(MOE_ERR_UNSUPPORTED, "T %d exceeds %d", T, MOE_MAX_TOKENS);
  return MOE_OK;
}

moe_status need_ptr(const void *p, const char *name) {
  if (!p) return fail(MOE_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(MOE_ERR_MISALIGNED, "%s is not 16-byte aligned", name);
  return MOE_OK;
}

#define TRY(expr)                      \
  do {                                 \
    moe_status _s = (expr);            \
    if (_s != MOE_OK) return _s;       \
  } while (0)

size_t elem_bytes(const moe_desc *d) { return d->dtype == MOE_BF16 ? 2 : 4; }

// FFN workspace layout (each segment 256-byte aligned).
struct FfnLayout {
  size_t h, idx, hact, partial, hm, fpart, sync, urow, ucnt, hmu, ubuf, counts, total;
  bool has_union;
};

// What an FFN-shaped call does (all share validation and the carve-up).
enum RunMode {
  kRunSparse, kRunDense, kRunUpdown, kRunThreshold, kRunCalibrate,
  kRunUpdownThreshold,  // the split with threshold masks on the gate scores
  kRunCalibrateGate     // calibration on the gate scores (no w_up)
};

FfnLayout ffn_layout(const moe_desc *d, int32_t T, int32_t k, moe_path path) {
  const size_t P = (size_t)T * d->top_k;
  const int bf16 = d->dtype == MOE_BF16;
  FfnLayout L{};
  size_t off = 0;
  L.h = off;
  off += up(P * d->d_ff * 4);
  // the fused decode-batch FFN's counters, directly after h (its gate/up
  // blocks find them from h's address), then its per-pair partial outputs
  // (sized for min(T, kFusedMaxTokens): the fused launch takes no larger batch)
  const int Tf = T < moe::kFusedMaxTokens ? T : moe::kFusedMaxTokens;
  L.sync = off;
  if (path == MOE_PATH_SPARSE) off += up(moe::fused_sync_words(Tf, d->n_experts, d->hidden) * 4);
  L.fpart = off;
  if (path == MOE_PATH_SPARSE) off += up((size_t)Tf * d->top_k * d->hidden * 4);
  L.idx = off;
  off += up(P * (size_t)k * 4);
  L.hact = off;
  if (path == MOE_PATH_SPARSE) off += up(P * (size_t)k * 4);
  // the packed-rows down projection of the sparse path (larger batches;
  // its shape rule grows monotonically with T, so a workspace for T serves
  // every smaller call): union lists, union counts, compacted
  // coefficients, the build's scratch, and the partials the dense-path
  // down GEMM also uses
  L.has_union = path == MOE_PATH_SPARSE && moe::union_layout_ok(T, d->hidden, d->d_ff, bf16) &&
                moe::union_form(T, d->n_experts, d->top_k, d->hidden, d->d_ff);
  L.urow = off;
  if (L.has_union) off += up((size_t)d->n_experts * d->d_ff * 4);
  L.ucnt = off;
  if (L.has_union) off += up((size_t)d->n_experts * 4);
  L.hmu = off;
  if (L.has_union) off += up(P * d->d_ff * 2);
  L.ubuf = off;
  if (L.has_union) off += up(moe::union_scratch_words(T, d->n_experts, d->d_ff) * 4);
  L.partial = off;
  if ((path == MOE_PATH_DENSE && bf16) || L.has_union)
    off += up(moe::dense_down_partial_rows(T, d->n_experts, d->top_k, d->hidden) * d->hidden * 4);
  L.hm = off;
  if (path == MOE_PATH_DENSE) off += up(P * d->d_ff * elem_bytes(d));
  L.counts = off;
  L.total = off;
  return L;
}

// Threshold masking: kept lists at row stride d_ff, plus per-pair counts.
FfnLayout threshold_layout(const moe_desc *d, int32_t T) {
  FfnLayout L = ffn_layout(d, T, d->d_ff, MOE_PATH_SPARSE);
  L.counts = L.total;
  L.total += up((size_t)T * d->top_k * 4);
  return L;
}

// Calibration: the scores h, then the layer-wide threshold (one float).
FfnLayout calibrate_layout(const moe_desc *d, int32_t T) {
  FfnLayout L{};
  L.h = 0;
  L.counts = up((size_t)T * d->top_k * d->d_ff * 4);
  L.total = L.counts + kAlign;
  return L;
}

// Extra inputs and outputs of the threshold and calibration modes.
struct ModeArgs {
  const float *tau = nullptr;   // threshold: [E] per-expert thresholds (device)
  int32_t *counts = nullptr;    // threshold: optional [P] kept counts (device)
  double sparsity = 0.0;        // calibrate: target sparsity
  float *tau_out = nullptr;     // calibrate: [E] thresholds (device)
  const void *xres = nullptr;   // sparse: residual epilogue input [T, H] (device)
  void *xnext = nullptr;        // sparse: residual epilogue output [T, H] (device)
  bool validate_only = false;   // check every argument, enqueue nothing
  const moe::RouteArgs *layer_route = nullptr;  // sparse: run the router first (whole layer)
};

moe_status run_ffn(RunMode mode, const moe_desc *d, int32_t T, int32_t k_keep, const void *x,
                   const void *w_gate, const void *w_up, const void *w_down,
                   const moe_routing *routing, float *y, int32_t accumulate,
                   int32_t *active_idx_out, void *workspace, size_t workspace_bytes,
                   hipStream_t stream, const ModeArgs &m = ModeArgs{}) {
  g_err[0] = 0;
  TRY(check_desc(d));
  TRY(check_T(T));
  if (d->gate_up_layout != MOE_LAYOUT_PACKED)
    return fail(MOE_ERR_UNSUPPORTED, "the FFN calls read w_gate%s packed by moe_pack_gate_up: pack "
                "it and set desc->gate_up_layout = MOE_LAYOUT_PACKED",
                mode == kRunUpdown || mode == kRunUpdownThreshold || mode == kRunCalibrateGate
                    ? "" : " and w_up");
  const moe_path path = mode == kRunDense ? MOE_PATH_DENSE : MOE_PATH_SPARSE;
  if (d->down_layout == MOE_LAYOUT_PACKED && mode != kRunCalibrate && mode != kRunCalibrateGate) {
    if (path != MOE_PATH_DENSE)
      return fail(MOE_ERR_UNSUPPORTED, "the sparse calls read kept rows of the row-major w_down: "
                  "set desc->down_layout = MOE_LAYOUT_ROWMAJOR (moe_pack_down is for the dense call)");
    if (d->dtype != MOE_BF16)
      return fail(MOE_ERR_UNSUPPORTED, "a packed w_down is bf16 only");
  }
  const bool thr = mode == kRunThreshold || mode == kRunUpdownThreshold;
  const bool cal = mode == kRunCalibrate || mode == kRunCalibrateGate;
  if (thr || cal) k_keep = d->d_ff;
  if (k_keep < 0 || k_keep > d->d_ff)
    return fail(MOE_ERR_INVALID_ARG, "k_keep %d outside [0, d_ff=%d]", k_keep, d->d_ff);
  if ((thr || cal) && !moe::threshold_supported(d->d_ff))
    return fail(MOE_ERR_UNSUPPORTED, "threshold masking needs d_ff <= 2048 (a multiple of 64) or "
                "a multiple of 512 up to 8192; got %d", d->d_ff);
  if (thr && !m.tau) return fail(MOE_ERR_INVALID_ARG, "tau is NULL");
  if (thr && ((uintptr_t)m.tau & 3u)) return fail(MOE_ERR_MISALIGNED, "tau is not 4-byte aligned");
  if (thr && m.counts && ((uintptr_t)m.counts & 3u))
    return fail(MOE_ERR_MISALIGNED, "counts_out is not 4-byte aligned");
  if (cal && !(m.sparsity >= 0.0 && m.sparsity <= 1.0))
    return fail(MOE_ERR_INVALID_ARG, "sparsity must lie in [0, 1]");
  if (cal && !m.tau_out) return fail(MOE_ERR_INVALID_ARG, "tau_out is NULL");
  if (cal && (long long)T * d->top_k * d->d_ff > 0x7fffffffLL)
    return fail(MOE_ERR_UNSUPPORTED, "calibration set too large: T * top_k * d_ff = %lld >= 2^31",
                (long long)T * d->top_k * d->d_ff);
  if (cal && ((uintptr_t)m.tau_out & 3u))
    return fail(MOE_ERR_MISALIGNED, "tau_out is not 4-byte aligned");
  if (accumulate != 0 && accumulate != 1)
    return fail(MOE_ERR_INVALID_ARG, "accumulate must be 0 or 1");
  if (!routing && d->top_k != d->n_experts)
    return fail(MOE_ERR_INVALID_ARG,
                "routing == NULL (always-on group) needs top_k == n_experts (%d != %d)", d->top_k,
                d->n_experts);
  if (T == 0) return MOE_OK;
  TRY(need_ptr(x, "x"));
  TRY(need_ptr(w_gate, "w_gate"));
  if (mode != kRunCalibrateGate) TRY(need_ptr(w_up, "w_up"));
  if (!cal) {
    TRY(need_ptr(w_down, "w_down"));
    TRY(need_ptr(y, "y"));
  }
  if (routing) {
    TRY(need_ptr(routing->topk_ids, "routing->topk_ids"));
    TRY(need_ptr(routing->topk_w, "routing->topk_w"));
    TRY(need_ptr(routing->expert_offsets, "routing->expert_offsets"));
    TRY(need_ptr(routing->pair_by_expert, "routing->pair_by_expert"));
    TRY(need_ptr(routing->active_experts, "routing->active_experts"));
    TRY(need_ptr(routing->n_active, "routing->n_active"));
  }
  if (active_idx_out && !aligned16(active_idx_out))
    return fail(MOE_ERR_MISALIGNED, "active_idx_out is not 16-byte aligned");
  const FfnLayout L = thr ? threshold_layout(d, T)
                     : cal ? calibrate_layout(d, T) : ffn_layout(d, T, k_keep, path);
  if (!workspace) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(MOE_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  if (workspace_bytes < L.total)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, L.total);
  if (m.validate_only) return MOE_OK;

  char *ws = static_cast<char *>(workspace);
  moe::FfnArgs a{};
  a.T = T;
  a.H = d->hidden;
  a.E = d->n_experts;
  a.d_ff = d->d_ff;
  a.top_k = d->top_k;
  a.k_keep = k_keep;
  a.bf16 = d->dtype == MOE_BF16;
  a.down_packed = d->down_layout == MOE_LAYOUT_PACKED;
  a.implicit = routing == nullptr;
  a.accumulate = accumulate;
  a.x = x;
  a.w_gate = w_gate;
  a.w_up = w_up;
  a.w_down = w_down;
  if (routing) {
    a.topk_ids = routing->topk_ids;
    a.topk_w = routing->topk_w;
    a.offsets = routing->expert_offsets;
    a.pair_by_expert = routing->pair_by_expert;
    a.active = routing->active_experts;
    a.n_active = routing->n_active;
  }
  a.y = y;
  a.h = reinterpret_cast<float *>(ws + L.h);
  a.idx = active_idx_out ? active_idx_out : reinterpret_cast<int32_t *>(ws + L.idx);
  a.want_idx = active_idx_out != nullptr;
  a.hact = path == MOE_PATH_SPARSE ? reinterpret_cast<float *>(ws + L.hact) : nullptr;
  a.partial = reinterpret_cast<float *>(ws + L.partial);
  a.hm = path == MOE_PATH_DENSE ? static_cast<void *>(ws + L.hm) : nullptr;
  a.xres = m.xres;
  a.xnext = m.xnext;
  a.fpart = path == MOE_PATH_SPARSE ? reinterpret_cast<float *>(ws + L.fpart) : nullptr;
  a.sync = path == MOE_PATH_SPARSE ? reinterpret_cast<int32_t *>(ws + L.sync) : nullptr;
  a.sync_zeroed = 0;
  if (L.has_union) {
    a.urow = reinterpret_cast<int32_t *>(ws + L.urow);
    a.ucnt = reinterpret_cast<int32_t *>(ws + L.ucnt);
    a.hmu = reinterpret_cast<uint16_t *>(ws + L.hmu);
    a.ubuf = reinterpret_cast<uint32_t *>(ws + L.ubuf);
  }
  hipError_t e;
  switch (mode) {
    case kRunUpdown: e = moe::launch_ffn_updown(a, stream); break;
    case kRunThreshold:
      e = moe::launch_ffn_threshold(
          a, m.tau, m.counts ? m.counts : reinterpret_cast<int32_t *>(ws + L.counts),
          m.counts != nullptr, active_idx_out != nullptr, stream);
      break;
    case kRunUpdownThreshold:
      e = moe::launch_ffn_updown_threshold(
          a, m.tau, m.counts ? m.counts : reinterpret_cast<int32_t *>(ws + L.counts), stream);
      break;
    case kRunCalibrate:
    case kRunCalibrateGate:
      e = moe::launch_calibrate(a, m.sparsity, m.tau_out, reinterpret_cast<float *>(ws + L.counts),
                                mode == kRunCalibrateGate, stream);
      break;
    case kRunDense: e = moe::launch_ffn_dense(a, stream); break;
    default:
      if (m.layer_route && moe::layer_small_ok(*m.layer_route, a)) {
        e = moe::launch_layer_small(*m.layer_route, a, stream);
      } else if (m.layer_route) {
        moe::RouteArgs r = *m.layer_route;
        if (moe::fused_ffn_ok(a)) {  // the router zeroes the fused FFN's counters
          r.zero = a.sync;
          r.nzero = (int)moe::fused_sync_words(T, d->n_experts, d->hidden);
          a.sync_zeroed = 1;
        }
        e = moe::launch_route(r, stream);
        if (e == hipSuccess) e = moe::launch_ffn_sparse(a, stream);
      } else {
        e = moe::launch_ffn_sparse(a, stream);
      }
  }
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

}  // namespace

extern "C" {

static moe_status route_check(const moe_desc *d, int32_t T, const void *x, const void *w_router,
                              const float *bias, const moe::RosterArgs &ro,
                              const moe_routing *out, void *workspace, size_t workspace_bytes) {
  TRY(check_desc(d));
  TRY(check_T(T));
  if (!out) return fail(MOE_ERR_INVALID_ARG, "routing output struct is NULL");
  if (ro.usage) {
    if ((uintptr_t)ro.usage & 3u) return fail(MOE_ERR_MISALIGNED, "usage is not 4-byte aligned");
    if (ro.pinned && ((uintptr_t)ro.pinned & 3u))
      return fail(MOE_ERR_MISALIGNED, "pinned is not 4-byte aligned");
    if (ro.m < 1 || ro.m > d->n_experts)
      return fail(MOE_ERR_INVALID_ARG, "roster size %d outside [1, n_experts=%d]", ro.m,
                  d->n_experts);
    if (ro.pinned && ro.m < d->top_k)
      return fail(MOE_ERR_INVALID_ARG, "pinned rows need roster size >= top_k (%d < %d)", ro.m,
                  d->top_k);
    if (!(ro.delta >= 0.f && ro.delta <= 3.0e38f))
      return fail(MOE_ERR_INVALID_ARG, "delta must be finite and >= 0");
  }
  if (T == 0) return MOE_OK;
  TRY(need_ptr(x, "x"));
  TRY(need_ptr(w_router, "w_router"));
  if (bias && ((uintptr_t)bias & 3u)) return fail(MOE_ERR_MISALIGNED, "bias is not 4-byte aligned");
  TRY(need_ptr(out->topk_ids, "out->topk_ids"));
  TRY(need_ptr(out->topk_w, "out->topk_w"));
  TRY(need_ptr(out->expert_offsets, "out->expert_offsets"));
  TRY(need_ptr(out->pair_by_expert, "out->pair_by_expert"));
  TRY(need_ptr(out->active_experts, "out->active_experts"));
  TRY(need_ptr(out->n_active, "out->n_active"));
  const size_t need = moe_route_workspace_size(d, T);
  if (!workspace) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(MOE_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  return MOE_OK;
}

static moe::RouteArgs route_args(const moe_desc *d, int32_t T, const void *x,
                                 const void *w_router, const float *bias,
                                 const moe::RosterArgs &ro, const moe_routing *out,
                                 void *workspace) {
  moe::RouteArgs a{};
  a.T = T;
  a.H = d->hidden;
  a.E = d->n_experts;
  a.top_k = d->top_k;
  a.norm_topk = d->norm_topk;
  a.bf16 = d->dtype == MOE_BF16;
  a.x = x;
  a.w_router = w_router;
  a.bias = bias;
  a.roster = ro;
  a.logits = static_cast<float *>(workspace);
  a.topk_ids = out->topk_ids;
  a.topk_w = out->topk_w;
  a.offsets = out->expert_offsets;
  a.pair_by_expert = out->pair_by_expert;
  a.active = out->active_experts;
  a.n_active = out->n_active;
  return a;
}

static moe_status route_impl(const moe_desc *d, int32_t T, const void *x, const void *w_router,
                             const float *bias, const moe::RosterArgs &ro,
                             const moe_routing *out, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  g_err[0] = 0;
  TRY(route_check(d, T, x, w_router, bias, ro, out, workspace, workspace_bytes));
  if (T == 0) return MOE_OK;
  const moe::RouteArgs a = route_args(d, T, x, w_router, bias, ro, out, workspace);
  const hipError_t e = moe::launch_route(a, stream);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

moe_status moe_route(const moe_desc *d, int32_t T, const void *x, const void *w_router,
                     const float *bias, const moe_routing *out, void *workspace,
                     size_t workspace_bytes, hipStream_t stream) {
  return route_impl(d, T, x, w_router, bias, moe::RosterArgs{}, out, workspace, workspace_bytes,
                    stream);
}

moe_status moe_route_roster(const moe_desc *d, int32_t T, const void *x, const void *w_router,
                            const float *bias, int32_t *usage, const int32_t *pinned,
                            int32_t roster_size, float delta, const moe_routing *out,
                            void *workspace, size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (!usage) return fail(MOE_ERR_INVALID_ARG, "usage is NULL");
  moe::RosterArgs ro{usage, pinned, roster_size, delta};
  return route_impl(d, T, x, w_router, bias, ro, out, workspace, workspace_bytes, stream);
}

moe_status moe_expert_ffn_sparse(const moe_desc *d, int32_t T, int32_t k_keep, const void *x,
                                 const void *w_gate, const void *w_up, const void *w_down,
                                 const moe_routing *routing, float *y, int32_t accumulate,
                                 int32_t *active_idx_out, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream) {
  return run_ffn(kRunSparse, d, T, k_keep, x, w_gate, w_up, w_down, routing, y, accumulate,
                 active_idx_out, workspace, workspace_bytes, stream);
}

moe_status moe_expert_ffn_sparse_residual(const moe_desc *d, int32_t T, int32_t k_keep,
                                          const void *x, const void *w_gate, const void *w_up,
                                          const void *w_down, const moe_routing *routing,
                                          float *y, int32_t accumulate, int32_t *active_idx_out,
                                          const void *x_res, void *x_next, void *workspace,
                                          size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  if (T > 0) {
    if (!x_res || !x_next) return fail(MOE_ERR_INVALID_ARG, "x_res and x_next must be non-NULL");
    if (!aligned16(x_res) || !aligned16(x_next))
      return fail(MOE_ERR_MISALIGNED, "x_res and x_next must be 16-byte aligned");
  }
  ModeArgs m;
  m.xres = x_res;
  m.xnext = x_next;
  return run_ffn(kRunSparse, d, T, k_keep, x, w_gate, w_up, w_down, routing, y, accumulate,
                 active_idx_out, workspace, workspace_bytes, stream, m);
}

size_t moe_layer_workspace_size(const moe_desc *d, int32_t T, int32_t k_keep) {
  const size_t r = moe_route_workspace_size(d, T);
  const size_t f = moe_ffn_workspace_size(d, T, k_keep, MOE_PATH_SPARSE);
  if (check_desc(d) != MOE_OK || T < 0 || k_keep < 0 || k_keep > d->d_ff) return 0;
  return up(r) + f;
}

moe_status moe_layer_sparse(const moe_desc *d, int32_t T, int32_t k_keep, const void *x,
                            const void *w_router, const float *bias, const void *w_gate,
                            const void *w_up, const void *w_down, const moe_routing *routing_out,
                            float *y, int32_t accumulate, int32_t *active_idx_out,
                            const void *x_res, void *x_next, void *workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  g_err[0] = 0;
  TRY(check_desc(d));
  TRY(check_T(T));
  if (T == 0) return MOE_OK;
  if ((x_res == nullptr) != (x_next == nullptr))
    return fail(MOE_ERR_INVALID_ARG, "x_res and x_next must both be given or both be NULL");
  if (x_res && (!aligned16(x_res) || !aligned16(x_next)))
    return fail(MOE_ERR_MISALIGNED, "x_res and x_next must be 16-byte aligned");
  if (!workspace) return fail(MOE_ERR_WORKSPACE, "workspace is NULL");
  if (!aligned16(workspace)) return fail(MOE_ERR_MISALIGNED, "workspace is not 16-byte aligned");
  const size_t need = moe_layer_workspace_size(d, T, k_keep);
  if (need == 0) return fail(MOE_ERR_INVALID_ARG, "k_keep %d outside [0, d_ff=%d]", k_keep, d->d_ff);
  if (workspace_bytes < need)
    return fail(MOE_ERR_WORKSPACE, "workspace %zu bytes < %zu needed", workspace_bytes, need);
  const size_t rws = up(moe_route_workspace_size(d, T));
  char *ws = static_cast<char *>(workspace);
  // every argument of both halves is checked before anything is enqueued
  TRY(route_check(d, T, x, w_router, bias, moe::RosterArgs{}, routing_out, ws, rws));
  ModeArgs m;
  m.validate_only = true;
  m.xres = x_res;
  m.xnext = x_next;
  TRY(run_ffn(kRunSparse, d, T, k_keep, x, w_gate, w_up, w_down, routing_out, y, accumulate,
              active_idx_out, ws + rws, workspace_bytes - rws, stream, m));
  const moe::RouteArgs ra = route_args(d, T, x, w_router, bias, moe::RosterArgs{}, routing_out, ws);
  m.validate_only = false;
  m.layer_route = &ra;
  return run_ffn(kRunSparse, d, T, k_keep, x, w_gate, w_up, w_down, routing_out, y, accumulate,
                 active_idx_out, ws + rws, workspace_bytes - rws, stream, m);
}

moe_status moe_layer_sparse_noalloc(const moe_desc *d, int32_t T, int32_t k_keep, const void *x,
                                    const void *w_router, const float *bias, const void *w_gate,
                                    const void *w_up, const void *w_down,
                                    const moe_routing *routing_out, float *y, int32_t accumulate,
                                    int32_t *active_idx_out, const void *x_res, void *x_next,
                                    hipStream_t stream) {
  g_err[0] = 0;
  TRY(check_desc(d));
  TRY(check_T(T));
  if (T == 0) return MOE_OK;
  const size_t need = moe_layer_workspace_size(d, T, k_keep);
  if (need == 0) return fail(MOE_ERR_INVALID_ARG, "k_keep %d outside [0, d_ff=%d]", k_keep, d->d_ff);
  if (need > (size_t)MOE_NOALLOC_SCRATCH_BYTES)
    return fail(MOE_ERR_WORKSPACE,
                "this call needs %zu bytes of scratch; the static scratch holds %zu (call "
                "moe_layer_sparse with a caller workspace)", need, (size_t)MOE_NOALLOC_SCRATCH_BYTES);
  void *ws = nullptr;
  const hipError_t e = moe::noalloc_scratch(&ws);
  if (e != hipSuccess)
    return fail(MOE_ERR_HIP, "device address of the static scratch: %s", hipGetErrorString(e));
  return moe_layer_sparse(d, T, k_keep, x, w_router, bias, w_gate, w_up, w_down, routing_out, y,
                          accumulate, active_idx_out, x_res, x_next, ws,
                          (size_t)MOE_NOALLOC_SCRATCH_BYTES, stream);
}

moe_status moe_expert_ffn_dense(const moe_desc *d, int32_t T, int32_t k_keep, const void *x,
                                const void *w_gate, const void *w_up, const void *w_down,
                                const moe_routing *routing, float *y, int32_t accumulate,
                                int32_t *active_idx_out, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
  return run_ffn(kRunDense, d, T, k_keep, x, w_gate, w_up, w_down, routing, y, accumulate,
                 active_idx_out, workspace, workspace_bytes, stream);
}

moe_status moe_expert_ffn_sparse_updown(const moe_desc *d, int32_t T, int32_t k_keep,
                                        const void *x, const void *w_gate, const void *w_up,
                                        const void *w_down, const moe_routing *routing, float *y,
                                        int32_t accumulate, int32_t *active_idx_out,
                                        void *workspace, size_t workspace_bytes,
                                        hipStream_t stream) {
  return run_ffn(kRunUpdown, d, T, k_keep, x, w_gate, w_up, w_down, routing, y,
                 accumulate, active_idx_out, workspace, workspace_bytes, stream);
}

moe_status moe_expert_ffn_sparse_threshold(const moe_desc *d, int32_t T, const float *tau,
                                           const void *x, const void *w_gate, const void *w_up,
                                           const void *w_down, const moe_routing *routing,
                                           float *y, int32_t accumulate, int32_t *counts_out,
                                           int32_t *active_idx_out, void *workspace,
                                           size_t workspace_bytes, hipStream_t stream) {
  ModeArgs m;
  m.tau = tau;
  m.counts = counts_out;
  return run_ffn(kRunThreshold, d, T, 0, x, w_gate, w_up, w_down, routing, y, accumulate,
                 active_idx_out, workspace, workspace_bytes, stream, m);
}

moe_status moe_expert_ffn_sparse_updown_threshold(const moe_desc *d, int32_t T, const float *tau,
                                                  const void *x, const void *w_gate,
                                                  const void *w_up, const void *w_down,
                                                  const moe_routing *routing, float *y,
                                                  int32_t accumulate, int32_t *counts_out,
                                                  int32_t *active_idx_out, void *workspace,
                                                  size_t workspace_bytes, hipStream_t stream) {
  ModeArgs m;
  m.tau = tau;
  m.counts = counts_out;
  return run_ffn(kRunUpdownThreshold, d, T, 0, x, w_gate, w_up, w_down, routing, y, accumulate,
                 active_idx_out, workspace, workspace_bytes, stream, m);
}

moe_status moe_calibrate_thresholds_gate(const moe_desc *d, int32_t T, const void *x,
                                         const void *w_gate, const moe_routing *routing,
                                         double sparsity, float *tau_out, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream) {
  ModeArgs m;
  m.sparsity = sparsity;
  m.tau_out = tau_out;
  return run_ffn(kRunCalibrateGate, d, T, 0, x, w_gate, nullptr, nullptr, routing, nullptr, 0,
                 nullptr, workspace, workspace_bytes, stream, m);
}

moe_status moe_calibrate_thresholds(const moe_desc *d, int32_t T, const void *x,
                                    const void *w_gate, const void *w_up,
                                    const moe_routing *routing, double sparsity, float *tau_out,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream) {
  ModeArgs m;
  m.sparsity = sparsity;
  m.tau_out = tau_out;
  return run_ffn(kRunCalibrate, d, T, 0, x, w_gate, w_up, nullptr, routing, nullptr, 0, nullptr,
                 workspace, workspace_bytes, stream, m);
}

static moe_status pack_impl(const moe_desc *d, const void *src, void *dst, int unpack,
                            hipStream_t stream) {
  g_err[0] = 0;
  TRY(check_desc(d));
  TRY(need_ptr(src, "src"));
  TRY(need_ptr(dst, "dst"));
  const size_t bytes = (size_t)d->n_experts * d->d_ff * d->hidden * elem_bytes(d);
  const char *s = static_cast<const char *>(src), *t = static_cast<const char *>(dst);
  if (s < t + bytes && t < s + bytes) return fail(MOE_ERR_INVALID_ARG, "src and dst overlap");
  const hipError_t e = moe::launch_pack_gate_up(src, dst, d->n_experts, d->d_ff, d->hidden,
                                                d->dtype == MOE_BF16, unpack, stream);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

moe_status moe_pack_gate_up(const moe_desc *d, const void *src_rowmajor, void *dst_packed,
                            hipStream_t stream) {
  return pack_impl(d, src_rowmajor, dst_packed, 0, stream);
}

static moe_status pack_down_impl(const moe_desc *d, const void *src, void *dst, int unpack,
                                 hipStream_t stream) {
  g_err[0] = 0;
  TRY(check_desc(d));
  if (d->dtype != MOE_BF16) return fail(MOE_ERR_UNSUPPORTED, "a packed w_down is bf16 only");
  if (!src || !dst) return fail(MOE_ERR_INVALID_ARG, "src and dst must be non-NULL");
  if (!aligned16(src) || !aligned16(dst)) return fail(MOE_ERR_MISALIGNED, "src and dst must be 16-byte aligned");
  const size_t bytes = (size_t)d->n_experts * d->d_ff * d->hidden * 2;
  const char *s = static_cast<const char *>(src), *t = static_cast<const char *>(dst);
  if (s < t + bytes && t < s + bytes) return fail(MOE_ERR_INVALID_ARG, "src and dst overlap");
  const hipError_t e = moe::launch_pack_down(src, dst, d->n_experts, d->d_ff, d->hidden, unpack, stream);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

moe_status moe_pack_down(const moe_desc *d, const void *src_rowmajor, void *dst_packed,
                         hipStream_t stream) {
  return pack_down_impl(d, src_rowmajor, dst_packed, 0, stream);
}

moe_status moe_unpack_down(const moe_desc *d, const void *src_packed, void *dst_rowmajor,
                           hipStream_t stream) {
  return pack_down_impl(d, src_packed, dst_rowmajor, 1, stream);
}

moe_status moe_unpack_gate_up(const moe_desc *d, const void *src_packed, void *dst_rowmajor,
                              hipStream_t stream) {
  return pack_impl(d, src_packed, dst_rowmajor, 1, stream);
}

size_t moe_route_workspace_size(const moe_desc *d, int32_t T) {
  if (check_desc(d) != MOE_OK || check_T(T) != MOE_OK) return 0;
  return up((size_t)moe::kRouterSplits * (T > 0 ? T : 1) * d->n_experts * 4);
}

size_t moe_ffn_workspace_size(const moe_desc *d, int32_t T, int32_t k_keep, moe_path path) {
  if (check_desc(d) != MOE_OK || check_T(T) != MOE_OK) return 0;
  if (k_keep < 0 || k_keep > d->d_ff) return 0;
  if (path != MOE_PATH_SPARSE && path != MOE_PATH_DENSE) return 0;
  return ffn_layout(d, T > 0 ? T : 1, k_keep, path).total;
}

size_t moe_workspace_size(const moe_desc *d, int32_t T_max, int32_t k_keep, moe_path path) {
  const size_t r = moe_route_workspace_size(d, T_max);
  const size_t f = moe_ffn_workspace_size(d, T_max, k_keep, path);
  if (r == 0 || f == 0) return 0;
  // route's region first, then the FFN's: the layout moe_layer_sparse uses,
  // and a superset of what moe_route or the FFN call alone needs
  return up(r) + f;
}

size_t moe_ffn_threshold_workspace_size(const moe_desc *d, int32_t T) {
  if (check_desc(d) != MOE_OK || check_T(T) != MOE_OK) return 0;
  return threshold_layout(d, T > 0 ? T : 1).total;
}

size_t moe_calibrate_workspace_size(const moe_desc *d, int32_t T) {
  if (check_desc(d) != MOE_OK || check_T(T) != MOE_OK) return 0;
  return calibrate_layout(d, T > 0 ? T : 1).total;
}

int32_t moe_keep_count(double sparsity, int32_t d_ff) {
  if (d_ff < 0 || !isfinite(sparsity)) return -1;
  double k = ceil((1.0 - sparsity) * (double)d_ff - 1e-9);
  if (k < 0) k = 0;
  if (k > d_ff) k = d_ff;
  return (int32_t)k;
}

moe_path moe_select_path(const moe_desc *d, int32_t T, int32_t k_keep) {
  const char *force = getenv("MOE_FORCE_PATH");
  if (force) {
    if (!strcmp(force, "sparse")) return MOE_PATH_SPARSE;
    if (!strcmp(force, "dense")) return MOE_PATH_DENSE;
  }
  if (check_desc(d) != MOE_OK || T <= 0 || k_keep < 0 || k_keep > d->d_ff) return MOE_PATH_SPARSE;
  // Both paths stream the same gate/up bytes; they differ in the down
  // projection: the sparse path reads k_keep rows per (token, expert) pair,
  // the dense path every d_ff row once per active expert.  Expected active
  // experts under uniform routing: A = E * (1 - (1 - top_k / E)^T), with
  // n_e = T * top_k / A tokens each.  A token's kept rows repeat among the
  // other tokens of its expert: d_ff * (1 - (1 - k / d_ff)^n_e) distinct rows
  // per expert come from HBM, the repeats mostly from the caches.  Measured
  // sparse-vs-dense sweeps (OLMoE-, Qwen3-MoE-, DeepSeek-V2- and Llama-4-like
  // layers, T = 1 .. 1024) fit a repeat cost of 0.3 row and a dense-GEMM
  // cost of 1.2 rows per row (costs in rows of H weights).  Without masking
  // (k_keep == d_ff) the dense path always wins.
  if (k_keep >= d->d_ff) return MOE_PATH_DENSE;
  const double E = d->n_experts, K = d->top_k, D = d->d_ff;
  const double active = E * (1.0 - pow(1.0 - K / E, (double)T));
  const double n_e = (double)T * K / active;
  const double total = (double)T * K * k_keep;
  const double unique = active * D * (1.0 - pow(1.0 - (double)k_keep / D, n_e));
  double sparse_cost = unique + 0.3 * (total - unique);
  // Where it takes the packed-rows form (bf16, many tokens per expert) the
  // sparse path reads each expert's union of kept rows once, through a
  // gathering GEMM (measured ~1.1x the dense GEMM's cost per row), after a
  // union build of ~12 us (~72 MB of streaming).
  if (d->dtype == MOE_BF16 && moe::union_form(T, d->n_experts, d->top_k, d->hidden, d->d_ff))
    sparse_cost = 1.32 * unique + 72e6 / (2.0 * d->hidden);
  const double dense_cost = 1.2 * active * D;
  return sparse_cost < dense_cost ? MOE_PATH_SPARSE : MOE_PATH_DENSE;
}

const char *moe_status_string(moe_status s) {
  switch (s) {
    case MOE_OK: return "MOE_OK";
    case MOE_ERR_INVALID_ARG: return "MOE_ERR_INVALID_ARG";
    case MOE_ERR_MISALIGNED: return "MOE_ERR_MISALIGNED";
    case MOE_ERR_WORKSPACE: return "MOE_ERR_WORKSPACE";
    case MOE_ERR_UNSUPPORTED: return "MOE_ERR_UNSUPPORTED";
    case MOE_ERR_HIP: return "MOE_ERR_HIP";
  }
  return "MOE_ERR_UNKNOWN";
}

moe_status moe_timer_attach(hipEvent_t *events, int32_t *stages, int32_t capacity) {
  g_err[0] = 0;
  if (!events || !stages || capacity <= 0)
    return fail(MOE_ERR_INVALID_ARG, "timer needs events, stages and a positive capacity");
  moe::StageTimer &t = moe::stage_timer();
  t.events = events;
  t.stages = stages;
  t.capacity = capacity;
  t.n = 0;
  return MOE_OK;
}

int32_t moe_timer_detach(void) {
  moe::StageTimer &t = moe::stage_timer();
  const int32_t n = t.n;
  t = moe::StageTimer{};
  return n;
}

moe_status moe_residual_add(const moe_desc *d, int32_t T, const void *x_in, const float *y,
                            void *x_out, hipStream_t stream) {
  g_err[0] = 0;
  TRY(check_desc(d));
  TRY(check_T(T));
  if (T == 0) return MOE_OK;
  TRY(need_ptr(x_in, "x_in"));
  TRY(need_ptr(y, "y"));
  TRY(need_ptr(x_out, "x_out"));
  if (!aligned16(x_in) || !aligned16(y) || !aligned16(x_out))
    return fail(MOE_ERR_MISALIGNED, "x_in, y and x_out must be 16-byte aligned");
  const hipError_t e = moe::launch_residual(x_in, y, x_out, (size_t)T * d->hidden,
                                            d->dtype == MOE_BF16, stream);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

moe_status moe_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream) {
  g_err[0] = 0;
  if (!src || !sink) return fail(MOE_ERR_INVALID_ARG, "stream_read needs src and sink");
  if (bytes == 0 || bytes % 16) return fail(MOE_ERR_INVALID_ARG, "bytes must be a positive multiple of 16");
  if (!aligned16(src) || !aligned16(sink)) return fail(MOE_ERR_MISALIGNED, "src and sink must be 16-byte aligned");
  const hipError_t e = moe::launch_stream_read(src, bytes, sink, MOE_STREAM_READ_SINK_WORDS / 4, stream);
  if (e != hipSuccess) return fail(MOE_ERR_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return MOE_OK;
}

const char *moe_last_error(void) { return g_err; }

const char *moe_version(void) { return "moe_mi355x 0.1 (gfx950)"; }

}  // extern "C"
