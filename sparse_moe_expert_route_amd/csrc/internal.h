// Host-side launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Optional per-launch event bracketing (the moe_timer_attach hook).
struct StageTimer {
  hipEvent_t *events = nullptr;
  int32_t *stages = nullptr;
  int capacity = 0;
  int n = 0;
};
StageTimer &stage_timer();

inline void timer_begin(int stage, hipStream_t s) {
  StageTimer &t = stage_timer();
  if (t.events && t.n < t.capacity) {
    (void)hipEventRecord(t.events[2 * t.n], s);
    t.stages[t.n] = stage;
  }
}
inline void timer_end(hipStream_t s) {
  StageTimer &t = stage_timer();
  if (t.events && t.n < t.capacity) {
    (void)hipEventRecord(t.events[2 * t.n + 1], s);
    ++t.n;
  }
}

// Stage ids (mirror moe_stage in the public header).
enum { kStageLogits = 0, kStageTopk, kStageGroup, kStageGateup, kStageMask, kStageDownRows,
       kStageDownDense, kStageCombine, kStageZero, kStageUpRows, kStageFused, kStageUnionRows,
       kStageDownUnion };

// Roster routing state (usage == nullptr: plain routing).
struct RosterArgs {
  int32_t *usage;          // [T, E] per-sequence expert usage, updated in place
  const int32_t *pinned;   // [T] nonzero = pinned row, or nullptr
  int m;                   // roster size
  float delta;             // barrier bias
};

struct RouteArgs {
  int T, H, E, top_k, norm_topk, bf16;
  const void *x, *w_router;
  const float *bias;
  RosterArgs roster;
  float *logits;  // workspace [kRouterSplits, T, E] partial logits
  int32_t *topk_ids;
  float *topk_w;
  int32_t *offsets, *pair_by_expert, *active, *n_active;
  // optional: words the logits kernel zeroes (the counters of a fused FFN
  // launch that follows on the stream); null to skip
  int32_t *zero = nullptr;
  int nzero = 0;
};

// Router split-K: logits are written as kRouterSplits-at-most partials.
constexpr int kRouterSplits = 8;
int router_splits(int T, int H, int E, int bf16);
hipError_t launch_route(const RouteArgs &a, hipStream_t stream);
// The logits kernel alone (split-K partials into a.logits); returns the
// number of splits.
int launch_router_logits(const RouteArgs &a, hipStream_t stream);

// One FFN call (routed group, or an implicit shared group).
struct FfnArgs {
  int T, H, E, d_ff, top_k, k_keep, bf16, implicit, accumulate;
  int down_packed = 0;  // dense path: w_down in the moe_pack_down layout
  const void *x, *w_gate, *w_up, *w_down;
  // routing (ignored when implicit)
  const int32_t *topk_ids;
  const float *topk_w;
  const int32_t *offsets, *pair_by_expert, *active, *n_active;
  float *y;
  // workspace carve-up
  float *h;          // [P, d_ff] fp32
  int32_t *idx;      // [P, k_keep]
  int want_idx;      // idx is the caller's active_idx_out (must be written)
  float *hact;       // [P, k_keep]   w * h at the kept neurons
  float *partial;    // dense bf16 path: [P, H] per-pair down outputs
  void *hm;          // dense path: [P, d_ff] masked, weighted h (bf16 or fp32)
  // optional residual epilogue (sparse path): x_next = x_res + y, rounded to
  // the layer dtype, written where each y element is final; null to skip
  const void *xres;
  void *xnext;
  // the fused decode-batch FFN (sparse path): per-pair partial outputs
  // [P, H] and its counters (kFusedSyncWords(T, E, H) words), zero before
  // the launch; sync_zeroed says an earlier kernel of the call zeroed them
  float *fpart;
  int32_t *sync;
  int sync_zeroed;
  // the packed-rows down projection (sparse path, bf16, experts holding
  // several tokens): per-expert ascending union of kept rows [E, d_ff] and
  // its count [E], and the coefficients at union positions [P, d_ff] bf16;
  // null when the workspace carries no such segments
  int32_t *urow = nullptr, *ucnt = nullptr;
  uint16_t *hmu = nullptr;
  uint32_t *ubuf = nullptr;  // the union build's scratch (union_scratch_words)
};

// The packed-rows down projection takes experts that hold at least
// union_min_tokens(W) tokens on average (shape only: P / min(E, P) routed,
// T shared), W = the expected active experts' W_d bytes.  Below that, each
// token's kept rows are streamed on their own and the rows the expert's
// other tokens also keep come back from the caches (L2, and the 256 MB
// last-level cache while W fits it), which beat the union's build; measured
// on four layer families (union vs per-token rows, per layer call: e.g.
// Llama-4-like, W = 1.3 GB: 791 vs 799 us at 8 tokens per expert, 902 vs
// 1003 at 16; OLMoE-like, W = 268 MB: 192 vs 184 at 16, 227 vs 236 at 32;
// a lone shared expert of 84 MB loses at 32 tokens).
#ifndef MOE_UNION_MIN_TOKENS_LARGE
#define MOE_UNION_MIN_TOKENS_LARGE 8  // W >= 512 MB
#endif
constexpr int kUnionMinTokensLarge = MOE_UNION_MIN_TOKENS_LARGE;
inline int union_min_tokens(double w_bytes) {
  return w_bytes >= 512e6 ? kUnionMinTokensLarge : (w_bytes >= 128e6 ? 32 : 128);
}
// Whether a sparse bf16 call of these shapes takes the packed-rows form.
bool union_form(int T, int E, int top_k, int H, int d_ff);
// Whether a sparse workspace for T tokens carries the packed-rows segments.
bool union_layout_ok(int T, int H, int d_ff, int bf16);
// Whether this sparse call takes the packed-rows down projection.
bool union_down_ok(const FfnArgs &a);
// 32-bit words of that projection's scratch for at most T tokens.
size_t union_scratch_words(int T, int E, int d_ff);

// Counter words of the fused FFN: per expert (each on its own 256-byte
// line: waiting blocks poll them, and pollers of one line all land on one
// memory channel), per (token, 64-column block), and one abort flag.
constexpr int kCounterStride = 64;
// Largest batch of the fused launch (its workspace segments are sized for
// min(T, this) tokens).
constexpr int kFusedMaxTokens = 16;
inline size_t fused_sync_words(int T, int E, int H) {
  return (size_t)E * kCounterStride + (size_t)T * (H / 64) + 1;
}
// Whether the fused single-launch FFN takes a sparse call with these shapes
// (then an earlier kernel of the call may zero its counters).
bool fused_ffn_ok(const FfnArgs &a);

// Device address of the static scratch of moe_layer_sparse_noalloc on the
// current device (looked up once per device).
hipError_t noalloc_scratch(void **out);

hipError_t launch_residual(const void *x_in, const float *y, void *x_out, size_t n, int bf16,
                           hipStream_t stream);
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, int max_blocks,
                              hipStream_t stream);
hipError_t launch_pack_gate_up(const void *src, void *dst, int E, int d_ff, int H, int bf16,
                               int unpack, hipStream_t stream);
hipError_t launch_pack_down(const void *src, void *dst, int E, int d_ff, int H, int unpack,
                            hipStream_t stream);

// Rows of the dense-path down GEMM's partial buffer for calls of at most T tokens.
size_t dense_down_partial_rows(int T, int E, int top_k, int H);
hipError_t launch_ffn_sparse(const FfnArgs &a, hipStream_t stream);
// A whole small-batch layer (moe_route then launch_ffn_sparse, same bits)
// without the router's select-and-group launch: logits, gate/up selecting
// its own expert, then mask and down.  layer_small_ok: whether these shapes
// take it.
bool layer_small_ok(const RouteArgs &r, const FfnArgs &a);
hipError_t launch_layer_small(const RouteArgs &r, const FfnArgs &a, hipStream_t stream);
hipError_t launch_ffn_dense(const FfnArgs &a, hipStream_t stream);
hipError_t launch_ffn_updown(const FfnArgs &a, hipStream_t stream);
bool threshold_supported(int d_ff);
hipError_t launch_ffn_threshold(const FfnArgs &a, const float *tau, int32_t *counts,
                                bool want_counts, bool want_idx, hipStream_t stream);
hipError_t launch_calibrate(const FfnArgs &a, double sparsity, float *tau, float *tau_all,
                            bool gate_only, hipStream_t stream);
hipError_t launch_ffn_updown_threshold(const FfnArgs &a, const float *tau, int32_t *counts,
                                       hipStream_t stream);

}  // namespace moe
