// Router: logits, softmax top-k, and the stable token -> expert grouping.
//
// The router itself is the model's unchanged linear router (the intra-expert
// page keeps router logic as is: technical summary, Methodology, vLLM
// implementation).  The grouping lets each expert's tokens run as one batched
// product, as the page's gate projection does.
#include "device_common.h"
#include "internal.h"
#include "route_common.h"

namespace moe {

// ---------------------------------------------------------------- logits
// l[t, e] = sum_h x[t, h] * w[e, h] (+ bias[e], added by the selection) as a
// small GEMM on MFMA.  Block = 16 experts x up to 16 * MT tokens x one of
// gridDim.z contiguous K ranges (split-K, so that even one token spreads the
// router matrix over many CUs); the 4 waves split the block's K range in
// interleaved steps and meet in LDS.  Each split writes its own partial
// [split][t][e]; the selection adds the splits in order.
template <bool BF16, int MT>
__global__ __launch_bounds__(256) void router_logits_kernel(const void *__restrict__ xv,
                                                            const void *__restrict__ wv, int T,
                                                            int H, int E,
                                                            float *__restrict__ partial,
                                                            int32_t *__restrict__ zero = nullptr,
                                                            int nzero = 0) {
  __shared__ float red[4][MT][4][64];
  // the fused FFN kernel that follows on this stream counts into these words
  if (zero && blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0)
    for (int i = threadIdx.x; i < nzero; i += 256) zero[i] = 0;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int r = lane & 15, g = lane >> 4;
  const int e0 = blockIdx.x * 16, t0 = blockIdx.y * 16 * MT;
  const int ntok = min(16 * MT, T - t0);
  const int ntiles = (ntok + 15) >> 4;
  const bool rv = e0 + r < E;
  f32x4 acc[MT];
  bool xval[MT];
  size_t xoff[MT];
#pragma unroll
  for (int tl = 0; tl < MT; ++tl) {
    acc[tl] = f32x4{0, 0, 0, 0};
    xval[tl] = tl * 16 + r < ntok;
    xoff[tl] = xval[tl] ? (size_t)(t0 + tl * 16 + r) * H : 0;
  }
  constexpr int U = 8;
  const int KS = BF16 ? 32 : 16;  // K elements per step
  const int nall = H / KS;
  const int per = (nall + gridDim.z - 1) / gridDim.z;  // k-steps of this split
  const int kbeg = blockIdx.z * per;
  const int nsteps = min(nall, kbeg + per);
  const size_t wrow = (size_t)(rv ? e0 + r : 0) * H;
  for (int s = kbeg + wid; s < nsteps; s += 4 * U) {
    u32x4 a[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = s + 4 * u;
      const int k = ks * KS + g * (KS / 4);
      a[u] = (ks < nsteps && rv)
                 ? (BF16 ? ld16(static_cast<const uint16_t *>(wv) + wrow + k)
                         : ld16(static_cast<const float *>(wv) + wrow + k))
                 : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ks = s + 4 * u;
      if (ks < nsteps) {
        const int k = ks * KS + g * (KS / 4);
#pragma unroll
        for (int tl = 0; tl < MT; ++tl) {
          if (tl < ntiles) {
            const u32x4 b = xval[tl] ? (BF16 ? ld16(static_cast<const uint16_t *>(xv) + xoff[tl] + k)
                                             : ld16(static_cast<const float *>(xv) + xoff[tl] + k))
                                     : u32x4{0, 0, 0, 0};
            if (BF16) {
              acc[tl] = mfma_bf16(a[u], b, acc[tl]);
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j)
                acc[tl] = mfma_f32(__uint_as_float(a[u][j]), __uint_as_float(b[j]), acc[tl]);
            }
          }
        }
      }
    }
  }
#pragma unroll
  for (int tl = 0; tl < MT; ++tl)
    if (tl < ntiles) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) red[wid][tl][rr][lane] = acc[tl][rr];
    }
  __syncthreads();
  for (int o = threadIdx.x; o < ntiles * 256; o += 256) {
    const int tl = o >> 8, rr = (o >> 6) & 3, ln = o & 63;
    const int c = tl * 16 + (ln & 15);           // token within the block
    const int e = e0 + 4 * (ln >> 4) + rr;       // expert row of the tile
    if (c < ntok && e < E) {
      const float v = red[0][tl][rr][ln] + red[1][tl][rr][ln] + red[2][tl][rr][ln] + red[3][tl][rr][ln];
      partial[((size_t)blockIdx.z * T + t0 + c) * E + e] = v;
    }
  }
}

template <int V, bool RO>
__global__ __launch_bounds__(256) void router_topk_kernel(const float *__restrict__ part,
                                                          int nsplit, const float *__restrict__ bias,
                                                          int T, int E, int top_k, int norm_topk,
                                                          RosterArgs ro,
                                                          int32_t *__restrict__ ids,
                                                          float *__restrict__ wout) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int t = blockIdx.x * 4 + wid;
  if (t >= T) return;
  int e;
  float w;
  wave_topk<V, RO>(part + (size_t)t * E, (size_t)T * E, nsplit, bias, E, top_k, norm_topk, ro, t,
                   e, w);
  if (lane < top_k) {
    ids[(size_t)t * top_k + lane] = e;
    wout[(size_t)t * top_k + lane] = w;
  }
}

// ---------------------------------------------------------------- grouping
// Block of 1024 threads.  Counts pairs per expert, scans them into CSR
// offsets and the ascending active-expert list, then places pairs chunk by
// chunk: inside a wave, lanes with the same expert are matched by ballots on
// the expert id bits; across the 16 waves of a chunk, per-(wave, expert)
// counts give each wave its base.  The result is a stable sort by (expert,
// pair id), i.e. ascending token order within an expert.  `ids` may live in
// LDS or global memory.
__device__ __forceinline__ void block_group(const int32_t *ids, int P, int E,
                                            int32_t *__restrict__ offsets,
                                            int32_t *__restrict__ pair_by_expert,
                                            int32_t *__restrict__ active,
                                            int32_t *__restrict__ n_active, int *cursor,
                                            uint8_t (*wcnt)[1024], int *tmp) {
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

// The same grouping by one wave, for the few pairs of a decode batch: no
// block barriers (they dominated the block version at T <= 16).  Counts by
// LDS atomics, offsets and the active list by wave scans over 64 experts at
// a time, then placement 64 pairs at a time with ballot matching on the
// expert id bits; `cur` (LDS, >= E ints) holds the per-expert cursors.
// Same result as block_group: a stable sort by (expert, pair id).
__device__ __forceinline__ void wave_group(const int32_t *ids, int P, int E,
                                           int32_t *__restrict__ offsets,
                                           int32_t *__restrict__ pair_by_expert,
                                           int32_t *__restrict__ active,
                                           int32_t *__restrict__ n_active, int *cur) {
  const int lane = threadIdx.x & 63;
  for (int e = lane; e < E; e += 64) cur[e] = 0;
  for (int p = lane; p < P; p += 64) atomicAdd(&cur[ids[p]], 1);
  int base = 0, abase = 0;
  for (int e0 = 0; e0 < E; e0 += 64) {
    const int e = e0 + lane;
    const int c = e < E ? cur[e] : 0;
    const int incl = wave_incl_scan(c);
    const int flag = c > 0 ? 1 : 0;
    const int aincl = wave_incl_scan(flag);
    if (e < E) {
      offsets[e] = base + incl - c;
      cur[e] = base + incl - c;  // the expert's cursor starts at its offset
    }
    if (flag) active[abase + aincl - 1] = e;
    base += lane_value(incl, 63);
    abase += lane_value(aincl, 63);
  }
  if (lane == 0) {
    offsets[E] = base;
    *n_active = abase;
  }
  const int nbits = E > 1 ? 32 - __clz(E - 1) : 0;
  const uint64_t lt_mask = (1ull << lane) - 1ull;
  for (int p0 = 0; p0 < P; p0 += 64) {
    const int p = p0 + lane;
    const bool valid = p < P;
    const int e = valid ? ids[p] : 0;
    uint64_t peers = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const int bit = (e >> b) & 1;
      const uint64_t m = __ballot(valid && bit);
      peers &= bit ? m : ~m;
    }
    const int rank = __popcll(peers & lt_mask);
    const int at = valid ? cur[e] : 0;  // every lane reads before the leader writes
    if (valid) pair_by_expert[at + rank] = p;
    if (valid && rank == 0) cur[e] = at + __popcll(peers);
  }
}

__global__ __launch_bounds__(1024) void route_group_kernel(const int32_t *__restrict__ ids, int P,
                                                           int E, int32_t *__restrict__ offsets,
                                                           int32_t *__restrict__ pair_by_expert,
                                                           int32_t *__restrict__ active,
                                                           int32_t *__restrict__ n_active) {
  __shared__ int cursor[1024];
  __shared__ uint8_t wcnt[16][1024];
  __shared__ int tmp[16];
  block_group(ids, P, E, offsets, pair_by_expert, active, n_active, cursor, wcnt, tmp);
}

// Decode batches (T <= 16): one block selects every token's experts (16
// waves, one token each) into LDS and global memory, then groups the pairs.
// Past one round of 16 tokens the selection is better spread over many
// blocks (router_topk_kernel) ahead of the grouping kernel: at T = 256 the
// one-block form took 56 us against ~10 us for the two kernels.
constexpr int kFusedMaxPairs = 2048;
template <int V, bool RO>
__global__ __launch_bounds__(1024) void route_select_group_kernel(
    const float *__restrict__ part, int nsplit, const float *__restrict__ bias, int T, int E,
    int top_k, int norm_topk, RosterArgs ro,
    int32_t *__restrict__ ids, float *__restrict__ wout, int32_t *__restrict__ offsets,
    int32_t *__restrict__ pair_by_expert, int32_t *__restrict__ active,
    int32_t *__restrict__ n_active) {
  __shared__ int sids[kFusedMaxPairs];
  __shared__ int cursor[1024];
  __shared__ uint8_t wcnt[16][1024];
  __shared__ int tmp[16];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  for (int t = wid; t < T; t += 16) {
    int e;
    float w;
    wave_topk<V, RO>(part + (size_t)t * E, (size_t)T * E, nsplit, bias, E, top_k, norm_topk, ro,
                     t, e, w);
    if (lane < top_k) {
      sids[t * top_k + lane] = e;
      ids[(size_t)t * top_k + lane] = e;
      wout[(size_t)t * top_k + lane] = w;
    }
  }
  __syncthreads();
  if (T * top_k <= 256) {
    if (threadIdx.x < 64) wave_group(sids, T * top_k, E, offsets, pair_by_expert, active, n_active, cursor);
  } else {
    block_group(sids, T * top_k, E, offsets, pair_by_expert, active, n_active, cursor, wcnt, tmp);
  }
}

template <int V, bool RO>
static void launch_select_ro(const RouteArgs &a, int nsplit, hipStream_t stream) {
  const int P = a.T * a.top_k;
  if (a.T <= 16 && P <= kFusedMaxPairs) {
    timer_begin(kStageTopk, stream);
    route_select_group_kernel<V, RO><<<1, 1024, 0, stream>>>(
        a.logits, nsplit, a.bias, a.T, a.E, a.top_k, a.norm_topk, a.roster, a.topk_ids, a.topk_w,
        a.offsets, a.pair_by_expert, a.active, a.n_active);
    timer_end(stream);
    return;
  }
  timer_begin(kStageTopk, stream);
  router_topk_kernel<V, RO><<<(a.T + 3) / 4, 256, 0, stream>>>(a.logits, nsplit, a.bias, a.T, a.E,
                                                               a.top_k, a.norm_topk, a.roster,
                                                               a.topk_ids, a.topk_w);
  timer_end(stream);
  timer_begin(kStageGroup, stream);
  route_group_kernel<<<1, 1024, 0, stream>>>(a.topk_ids, P, a.E, a.offsets, a.pair_by_expert,
                                             a.active, a.n_active);
  timer_end(stream);
}

template <int V>
static void launch_select(const RouteArgs &a, int nsplit, hipStream_t stream) {
  if (a.roster.usage) launch_select_ro<V, true>(a, nsplit, stream);
  else launch_select_ro<V, false>(a, nsplit, stream);
}

// Tokens per logits block: 16, or 64 once 64-token blocks (with the full
// split) still give two blocks per CU; fewer, larger blocks are slower
// (the 16-expert Llama-4-like router on 8 of them at T = 64: 14.7 against
// 5.8 us; the 64-expert OLMoE-like one at T = 64: 7.8 against 4.3 us).
static int router_token_group(int T, int E) {
  const long tiles64 = (long)((E + 15) / 16) * ((T + 63) / 64);
  return T > 16 && tiles64 * kRouterSplits >= 512 ? 64 : 16;
}

// Split-K factor of the router GEMM: enough blocks to spread the router
// matrix over many CUs (64 at decode batches; past one tile of tokens, two
// rounds of the chip's 256 CUs, since each block's K loop is a serial
// latency chain), at least 4 k-steps per split, at most kRouterSplits.
int router_splits(int T, int H, int E, int bf16) {
  const int tg = router_token_group(T, E);
  const int blocks = ((E + 15) / 16) * ((T + tg - 1) / tg);
  const int nsteps = H / (bf16 ? 32 : 16);
  const int target = T <= 16 ? 64 : 512;
  int sp = (target + blocks - 1) / blocks;
  sp = sp < nsteps / 4 ? sp : nsteps / 4;
  sp = sp < kRouterSplits ? sp : kRouterSplits;
  return sp < 1 ? 1 : sp;
}

int launch_router_logits(const RouteArgs &a, hipStream_t stream) {
  const bool one = router_token_group(a.T, a.E) == 16;
  const int nsplit = router_splits(a.T, a.H, a.E, a.bf16);
  dim3 g1((a.E + 15) / 16, (a.T + (one ? 16 : 64) - 1) / (one ? 16 : 64), nsplit);
  timer_begin(kStageLogits, stream);
  if (a.bf16) {
    if (one) router_logits_kernel<true, 1><<<g1, 256, 0, stream>>>(a.x, a.w_router, a.T, a.H, a.E, a.logits, a.zero, a.nzero);
    else router_logits_kernel<true, 4><<<g1, 256, 0, stream>>>(a.x, a.w_router, a.T, a.H, a.E, a.logits, a.zero, a.nzero);
  } else {
    if (one) router_logits_kernel<false, 1><<<g1, 256, 0, stream>>>(a.x, a.w_router, a.T, a.H, a.E, a.logits, a.zero, a.nzero);
    else router_logits_kernel<false, 4><<<g1, 256, 0, stream>>>(a.x, a.w_router, a.T, a.H, a.E, a.logits, a.zero, a.nzero);
  }
  timer_end(stream);
  return nsplit;
}

hipError_t launch_route(const RouteArgs &a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const int nsplit = launch_router_logits(a, stream);
  if (a.E <= 64) launch_select<1>(a, nsplit, stream);
  else if (a.E <= 128) launch_select<2>(a, nsplit, stream);
  else if (a.E <= 256) launch_select<4>(a, nsplit, stream);
  else launch_select<16>(a, nsplit, stream);
  return hipGetLastError();
}

}  // namespace moe
