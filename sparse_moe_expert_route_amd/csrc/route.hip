// Router: logits, softmax top-k, and the stable token -> expert grouping.
//
// The router itself is the model's unchanged linear router (the intra-expert
// page keeps router logic as is: technical summary, Methodology, vLLM
// implementation).  The grouping lets each expert's tokens run as one batched
// product, as the page's gate projection does.
#include "device_common.h"
#include "internal.h"

namespace moe {

// ---------------------------------------------------------------- logits
// l[t, e] = sum_h x[t, h] * w[e, h] + bias[e].  One wave per expert row,
// TT tokens per block; each lane owns 8-element chunks of H strided by 512
// and accumulates in fp32, then a butterfly sum.  The router matrix row is
// read once per block; the token rows come from L2.
constexpr int kLogitTokens = 8;

template <bool BF16>
__global__ __launch_bounds__(256) void router_logits_kernel(const void *__restrict__ xv,
                                                            const void *__restrict__ wv,
                                                            const float *__restrict__ bias,
                                                            int T, int H, int E,
                                                            float *__restrict__ logits) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int e = blockIdx.x * 4 + wid;
  const int t0 = blockIdx.y * kLogitTokens;
  if (e >= E) return;  // wave-uniform, no barrier below
  const int nt = min(kLogitTokens, T - t0);
  float acc[kLogitTokens];
#pragma unroll
  for (int i = 0; i < kLogitTokens; ++i) acc[i] = 0.f;

  for (int c = lane * 8; c < H; c += 512) {
    float w[8];
    if (BF16) {
      const uint16_t *wr = static_cast<const uint16_t *>(wv) + (size_t)e * H;
      u32x4 q = ld16(wr + c);
#pragma unroll
      for (int j = 0; j < 4; ++j) { w[2 * j] = bf16lo(q[j]); w[2 * j + 1] = bf16hi(q[j]); }
    } else {
      const float *wr = static_cast<const float *>(wv) + (size_t)e * H;
      u32x4 q0 = ld16(wr + c), q1 = ld16(wr + c + 4);
#pragma unroll
      for (int j = 0; j < 4; ++j) { w[j] = __uint_as_float(q0[j]); w[4 + j] = __uint_as_float(q1[j]); }
    }
#pragma unroll
    for (int i = 0; i < kLogitTokens; ++i) {
      if (i < nt) {
        float xs[8];
        if (BF16) {
          u32x4 q = ld16(static_cast<const uint16_t *>(xv) + (size_t)(t0 + i) * H + c);
#pragma unroll
          for (int j = 0; j < 4; ++j) { xs[2 * j] = bf16lo(q[j]); xs[2 * j + 1] = bf16hi(q[j]); }
        } else {
          const float *xr = static_cast<const float *>(xv) + (size_t)(t0 + i) * H + c;
          u32x4 q0 = ld16(xr), q1 = ld16(xr + 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) { xs[j] = __uint_as_float(q0[j]); xs[4 + j] = __uint_as_float(q1[j]); }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i] = fmaf(xs[j], w[j], acc[i]);
      }
    }
  }
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int i = 0; i < kLogitTokens; ++i) {
    float s = wave_sum(acc[i]);
    if (lane == 0 && i < nt) logits[(size_t)(t0 + i) * E + e] = s + b;
  }
}

// ---------------------------------------------------------------- top-k
// One wave per token.  Each lane holds V logits (expert lane + 64 i) as
// 64-bit keys (order-preserving float bits, then the complement of the
// expert id so that equal logits favour the lower id); top_k rounds of a
// wavefront max-reduction pick the experts in descending-logit order.
// Weights are the full softmax over all E experts at the picks, optionally
// renormalised over the picks.
template <int V>
__global__ __launch_bounds__(256) void router_topk_kernel(const float *__restrict__ logits, int T,
                                                          int E, int top_k, int norm_topk,
                                                          int32_t *__restrict__ ids,
                                                          float *__restrict__ wout) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wid;
  if (t >= T) return;
  const float *l = logits + (size_t)t * E;
  float v[V];
  uint64_t key[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = lane + 64 * i;
    v[i] = e < E ? l[e] : 0.f;
    key[i] = e < E ? ((uint64_t)ordered_key(v[i]) << 32) | (uint32_t)(0xffffffffu - e) : 0ull;
  }
  // first pick = the maximum logit m
  uint64_t best = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) best = key[i] > best ? key[i] : best;
  best = wave_max_u64(best);
  const float m = l[0xffffffffu - (uint32_t)best];
  float z = 0.f;
#pragma unroll
  for (int i = 0; i < V; ++i)
    if (lane + 64 * i < E) z += expf(v[i] - m);
  z = wave_sum(z);

  float psel = 0.f;  // this lane's pick (lane r holds round r)
  int esel = 0;
  for (int r = 0; r < top_k; ++r) {
    uint64_t b = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) b = key[i] > b ? key[i] : b;
    b = wave_max_u64(b);
    const int e = (int)(0xffffffffu - (uint32_t)b);
#pragma unroll
    for (int i = 0; i < V; ++i)
      if (lane + 64 * i == e) key[i] = 0ull;
    if (lane == r) { esel = e; psel = expf(l[e] - m); }
  }
  float denom = z;
  if (norm_topk) denom = wave_sum(lane < top_k ? psel : 0.f);
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = esel;
    wout[(size_t)t * top_k + lane] = psel / denom;
  }
}

// ---------------------------------------------------------------- grouping
// Single block, 1024 threads.  Counts pairs per expert, scans them into CSR
// offsets and the ascending active-expert list, then places pairs chunk by
// chunk: inside a wave, lanes with the same expert are matched by ballots on
// the expert id bits; across the 16 waves of a chunk, per-(wave, expert)
// counts give each wave its base.  The result is a stable sort by (expert,
// pair id), i.e. ascending token order within an expert.
__global__ __launch_bounds__(1024) void route_group_kernel(const int32_t *__restrict__ ids, int P,
                                                           int E, int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ pair_by_expert,
                                                           int32_t *__restrict__ active,
                                                           int32_t *__restrict__ n_active) {
  __shared__ int cursor[1024];
  __shared__ uint8_t wcnt[16][1024];
  __shared__ int tmp[16];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  cursor[tid] = 0;
  __syncthreads();
  for (int p = tid; p < P; p += 1024) atomicAdd(&cursor[ids[p]], 1);
  __syncthreads();
  const int c = tid < E ? cursor[tid] : 0;
  int total = 0;
  const int incl = block_incl_scan<1024>(c, tmp, &total);
  if (tid < E) offsets[tid] = incl - c;
  if (tid == 0) offsets[E] = total;
  const int flag = (tid < E && c > 0) ? 1 : 0;
  int nact = 0;
  const int aincl = block_incl_scan<1024>(flag, tmp, &nact);
  if (flag) active[aincl - 1] = tid;
  if (tid == 0) *n_active = nact;
  cursor[tid] = incl - c;
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  __syncthreads();

  for (int base = 0; base < P; base += 1024) {
    const int p = base + tid;
    const bool valid = p < P;
    const int e = valid ? ids[p] : 0;
    if (tid < E) {
#pragma unroll
      for (int w = 0; w < 16; ++w) wcnt[w][tid] = 0;
    }
    __syncthreads();
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const int bit = (e >> b) & 1;
      const uint64_t m = __ballot(valid && bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    if (valid && rank == 0) wcnt[wid][e] = (uint8_t)__popcll(peers);
    __syncthreads();
    if (valid) {
      int pos = cursor[e] + rank;
      for (int w = 0; w < wid; ++w) pos += wcnt[w][e];
      pair_by_expert[pos] = p;
    }
    __syncthreads();
    if (tid < E) {
      int add = 0;
#pragma unroll
      for (int w = 0; w < 16; ++w) add += wcnt[w][tid];
      cursor[tid] += add;
    }
    __syncthreads();
  }
}

hipError_t launch_route(const RouteArgs &a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  dim3 g1((a.E + 3) / 4, (a.T + kLogitTokens - 1) / kLogitTokens);
  timer_begin(kStageLogits, stream);
  if (a.bf16)
    router_logits_kernel<true><<<g1, 256, 0, stream>>>(a.x, a.w_router, a.bias, a.T, a.H, a.E, a.logits);
  else
    router_logits_kernel<false><<<g1, 256, 0, stream>>>(a.x, a.w_router, a.bias, a.T, a.H, a.E, a.logits);
  timer_end(stream);
  dim3 g2((a.T + 3) / 4);
  timer_begin(kStageTopk, stream);
  if (a.E <= 64)
    router_topk_kernel<1><<<g2, 256, 0, stream>>>(a.logits, a.T, a.E, a.top_k, a.norm_topk, a.topk_ids, a.topk_w);
  else if (a.E <= 128)
    router_topk_kernel<2><<<g2, 256, 0, stream>>>(a.logits, a.T, a.E, a.top_k, a.norm_topk, a.topk_ids, a.topk_w);
  else if (a.E <= 256)
    router_topk_kernel<4><<<g2, 256, 0, stream>>>(a.logits, a.T, a.E, a.top_k, a.norm_topk, a.topk_ids, a.topk_w);
  else
    router_topk_kernel<16><<<g2, 256, 0, stream>>>(a.logits, a.T, a.E, a.top_k, a.norm_topk, a.topk_ids, a.topk_w);
  timer_end(stream);
  timer_begin(kStageGroup, stream);
  route_group_kernel<<<1, 1024, 0, stream>>>(a.topk_ids, a.T * a.top_k, a.E, a.offsets,
                                             a.pair_by_expert, a.active, a.n_active);
  timer_end(stream);
  return hipGetLastError();
}

}  // namespace moe
