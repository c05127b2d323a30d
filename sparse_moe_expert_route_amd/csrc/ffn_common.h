// Shared by the expert FFN kernel files (ffn.hip: the sparse path and the
// small-batch gate/up; dense.hip: the grouped MFMA GEMMs): the work-item
// enumeration over the routing, SwiGLU's silu, and the host-side view of a
// call's routing.
#pragma once

#include "device_common.h"
#include "internal.h"

namespace moe {


// Work items enumerate, for each active expert in slot order, ceil(n_e / TG)
// groups of at most TG of its tokens.  Every lane of the calling wave gets
// the same answer; returns false for items past the end.
template <int TG>
__device__ __forceinline__ bool find_item(const RouteView &rv, int item, int &e, int &q0,
                                          int &ntok) {
  constexpr int kTokGroup = TG;
  if (rv.implicit) {
    const int ng = (rv.T + kTokGroup - 1) / kTokGroup;
    const int s = item / ng, gi = item - s * ng;
    if (s >= rv.E) return false;
    e = s;
    q0 = s * rv.T + gi * kTokGroup;
    ntok = min(kTokGroup, rv.T - gi * kTokGroup);
    return true;
  }
  const int lane = threadIdx.x & 63;
  const int nact = *rv.n_active;
  int base = 0;
  for (int s0 = 0; s0 < nact; s0 += 64) {
    const int s = s0 + lane;
    int ee = 0, b = 0, n = 0, cnt = 0;
    if (s < nact) {
      ee = rv.active[s];
      b = rv.offsets[ee];
      n = rv.offsets[ee + 1] - b;
      cnt = (n + kTokGroup - 1) / kTokGroup;
    }
    const int incl = wave_incl_scan(cnt);
    const int tot = lane_value(incl, 63);
    if (item < base + tot) {
      const uint64_t m = __ballot(s < nact && item < base + incl);
      const int L = __ffsll((unsigned long long)m) - 1;
      e = lane_value(ee, L);
      const int bb = lane_value(b, L), nn = lane_value(n, L);
      const int before = lane_value(incl - cnt, L);
      const int gi = item - base - before;
      q0 = bb + gi * kTokGroup;
      ntok = min(kTokGroup, nn - gi * kTokGroup);
      return true;
    }
    base += tot;
  }
  return false;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

inline RouteView make_view(const FfnArgs &a) {
  RouteView v;
  v.topk_ids = a.topk_ids;
  v.topk_w = a.topk_w;
  v.offsets = a.offsets;
  v.pair_by_expert = a.pair_by_expert;
  v.active = a.active;
  v.n_active = a.n_active;
  v.implicit = a.implicit;
  v.T = a.T;
  v.top_k = a.top_k;
  v.E = a.E;
  return v;
}

// Upper bound on the work items of a call with token groups of TG: each
// active expert contributes ceil(n_e / TG) <= n_e / TG + 1.
inline int n_items(const FfnArgs &a, int TG) {
  const int P = a.T * a.top_k;
  if (a.implicit) return a.E * ((a.T + TG - 1) / TG);
  return (a.E < P ? a.E : P) + P / TG;
}


// The grouped GEMMs of dense.hip.  launch_gateup_gemm: h (or the gate
// scores alone) for calls past 64 tokens, on the caller's stream, untimed.
// launch_down_dense: the dense-path down projection of bf16 masked rows
// a.hm into per-pair partials, then their combine into y.
void launch_gateup_gemm(const FfnArgs &a, const RouteView &rv, bool gate_only, hipStream_t stream);
hipError_t launch_down_dense(const FfnArgs &a, const RouteView &rv, hipStream_t stream);
// launch_down_union: the sparse path's packed-rows down projection (union
// kernel, gathering down GEMM, combine) from the mask kernel's kept lists
hipError_t launch_down_union(const FfnArgs &a, const RouteView &rv, hipStream_t stream);

}  // namespace moe
