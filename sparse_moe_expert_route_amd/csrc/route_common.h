// Router selection shared by the router kernels and by the fused
// single-token layer's gate/up kernel: one wave selects one token's experts
// from the router's split-K logit partials (roster bias optional).
#pragma once
#include "device_common.h"
#include "internal.h"

namespace moe {

// ---------------------------------------------------------------- roster bias
// The roster rule (Predatory MoE, technical summary, section 2) for one
// sequence's row of expert usage counts, in the wave's lane layout (expert
// lane + 64 i): the roster is the m most-used experts (ties: lower id),
// found by m rounds of a wavefront max over (count, ~id) keys.  Pinned rows
// keep only members selectable (bias 0 / -inf); otherwise no bias while
// fewer than m experts have been used, then +delta for members and -delta
// for the rest.  Negative counts read as 0.
template <int V>
__device__ __forceinline__ void roster_bias_row(const int32_t *__restrict__ usage, int pinned,
                                                int m, float delta, int E, float (&rb)[V]) {
  const int lane = threadIdx.x & 63;
  uint64_t key[V];
  bool member[V];
  float used = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = lane + 64 * i;
    const int c = e < E ? max(usage[e], 0) : 0;
    used += c > 0 ? 1.f : 0.f;
    key[i] = e < E ? ((uint64_t)(uint32_t)c << 32) | (uint32_t)(0xffffffffu - e) : 0ull;
    member[i] = false;
  }
  used = wave_sum(used);
  for (int r = 0; r < m; ++r) {
    uint64_t b = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) b = key[i] > b ? key[i] : b;
    b = wave_max_u64(b);
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (b != 0ull && key[i] == b) { member[i] = true; key[i] = 0ull; }
  }
  const bool explore = used < (float)m;
#pragma unroll
  for (int i = 0; i < V; ++i)
    rb[i] = pinned ? (member[i] ? 0.f : -INFINITY) : explore ? 0.f : (member[i] ? delta : -delta);
}

// ---------------------------------------------------------------- top-k
// One wave selects one token's experts.  Each lane holds V logits (expert
// lane + 64 i) as 64-bit keys (order-preserving float bits, then the
// complement of the expert id so that equal logits favour the lower id);
// top_k rounds of a wavefront max-reduction pick the experts in
// descending-logit order.  Weights are the full softmax over all E experts
// at the picks, optionally renormalised over the picks.  Lane r < top_k
// returns slot r's (expert, weight).
// With RO, token t's roster bias (from its usage row) is added to the
// logits before the softmax and the selection, and each selection adds one
// to the row's usage.
template <int V, bool RO>
__device__ __forceinline__ void wave_topk(const float *__restrict__ part, size_t split_stride,
                                          int nsplit, const float *__restrict__ bias, int E,
                                          int top_k, int norm_topk, const RosterArgs &ro, int t,
                                          int &esel, float &wsel) {
  const int lane = threadIdx.x & 63;
  float v[V];
  uint64_t key[V];
  float rb[V];
  if (RO) roster_bias_row<V>(ro.usage + (size_t)t * E, ro.pinned ? ro.pinned[t] : 0, ro.m, ro.delta,
                             E, rb);
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = lane + 64 * i;
    float l = 0.f;
    if (e < E) {
      // all split partials in flight at once, then added in split order
      float pv[kRouterSplits];
#pragma unroll
      for (int c = 0; c < kRouterSplits; ++c) pv[c] = c < nsplit ? part[c * split_stride + e] : 0.f;
#pragma unroll
      for (int c = 0; c < kRouterSplits; ++c)
        if (c < nsplit) l += pv[c];
      if (bias) l += bias[e];
      if (RO) l += rb[i];
    }
    v[i] = l;
    key[i] = e < E ? ((uint64_t)ordered_key(l) << 32) | (uint32_t)(0xffffffffu - e) : 0ull;
  }
  uint64_t best = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) best = key[i] > best ? key[i] : best;
  best = wave_max_u64(best);
  const float m = key_value(best);
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i)
    if (lane + 64 * i < E) z += expf(v[i] - m);
  z = wave_sum(z);
  float psel = 0.f;
  esel = 0;
  for (int r = 0; r < top_k; ++r) {
    uint64_t b = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) b = key[i] > b ? key[i] : b;
    b = wave_max_u64(b);
    const int e = (int)(0xffffffffu - (uint32_t)b);
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (lane + 64 * i == e) key[i] = 0ull;
    if (lane == r) { esel = e; psel = expf(key_value(b) - m); }
  }
  float denom = z;
  if (norm_topk) denom = wave_sum(lane < top_k ? psel : 0.f);
  wsel = psel / denom;
  // usage update: the row was read above by this wave; distinct experts
  if (RO && lane < top_k) ro.usage[(size_t)t * E + esel] += 1;
}

}  // namespace moe
