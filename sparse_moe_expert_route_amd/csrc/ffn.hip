// Expert FFN kernels of the intra-expert-sparse MoE layer (gfx950).
//
//   gateup_swiglu   h = silu(W_g x) * (W_u x), dense, MFMA, per (expert, <=64 tokens)
//   neuron_topk     exact top-k of |h| per pair (radix select + one threshold pass),
//                   compacted ascending kept-neuron list, weights folded in
//   down_rows       y_p = sum over kept rows j of hact_j * W_d[j, :], streaming
//                   only those rows (the sparse down projection)
//   down_dense      dense-path down GEMM (MFMA) over every row of W_d
//   combine         y[t] (+)= sum of a token's partials in fixed order
//
// Method: the page "Uncovering Intra-expert Activation Sparsity for
// Efficient Mixture-of-Expert Model Execution", technical summary,
// Methodology (vLLM implementation): gate projection run densely for the
// activation scores; activation masking in one O(n) threshold pass; a
// sparse projection that gathers only the active neurons' weights; a
// batch-size switch to the dense path.
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
    const int tot = __shfl(incl, 63, 64);
    if (item < base + tot) {
      const uint64_t m = __ballot(s < nact && item < base + incl);
      const int L = __ffsll((unsigned long long)m) - 1;
      e = __shfl(ee, L, 64);
      const int bb = __shfl(b, L, 64), nn = __shfl(n, L, 64);
      const int before = __shfl(incl - cnt, L, 64);
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

// ---------------------------------------------------------------- gate / up
// Block = one work item (an expert and up to 16 * MT of its tokens) x 16
// neurons; 4 waves split K (H) by interleaved steps so that at any moment
// the block reads contiguous 256-byte runs of each weight row.  Each wave
// keeps 16x16 MFMA accumulators for gate and up for MT token tiles; weights
// are loaded once, token rows (16 B per lane) come from L2.  The wave
// partials meet in LDS, where h = silu(g) * u is formed and written per pair.
template <bool BF16, int MT>
__global__ __launch_bounds__(256) void gateup_swiglu_kernel(const void *__restrict__ xv,
                                                            const void *__restrict__ wgv,
                                                            const void *__restrict__ wuv,
                                                            RouteView rv, int H, int d_ff,
                                                            float *__restrict__ hout) {
  __shared__ float red[4][2][MT][4][64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int e, q0, ntok;
  if (!find_item<16 * MT>(rv, blockIdx.x, e, q0, ntok)) return;  // block-uniform
  const int ntiles = (ntok + 15) >> 4;
  const int r = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.y * 16;
  const size_t wrow = ((size_t)e * d_ff + row0 + r) * (size_t)H;

  size_t xoff[MT];
  bool xval[MT];
#pragma unroll
  for (int tl = 0; tl < MT; ++tl) {
    const int c = tl * 16 + r;
    xval[tl] = c < ntok;
    const int t = xval[tl] ? rv.pair_at(q0 + c) / rv.top_k : 0;
    xoff[tl] = (size_t)t * H;
  }
  f32x4 accg[MT], accu[MT];
#pragma unroll
  for (int tl = 0; tl < MT; ++tl) { accg[tl] = f32x4{0, 0, 0, 0}; accu[tl] = f32x4{0, 0, 0, 0}; }

  constexpr int U = 4;
  if (BF16) {
    const uint16_t *wg = static_cast<const uint16_t *>(wgv) + wrow;
    const uint16_t *wu = static_cast<const uint16_t *>(wuv) + wrow;
    const uint16_t *x = static_cast<const uint16_t *>(xv);
    const int nsteps = H / 32;
    for (int s = wid; s < nsteps; s += 4 * U) {
      u32x4 ag[U], au[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ks = s + 4 * u;
        if (ks < nsteps) {
          const int k = ks * 32 + g * 8;
          ag[u] = ld16(wg + k);
          au[u] = ld16(wu + k);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ks = s + 4 * u;
        if (ks < nsteps) {
          const int k = ks * 32 + g * 8;
#pragma unroll
          for (int tl = 0; tl < MT; ++tl) {
            if (tl < ntiles) {
              const u32x4 b = xval[tl] ? ld16(x + xoff[tl] + k) : u32x4{0, 0, 0, 0};
              accg[tl] = mfma_bf16(ag[u], b, accg[tl]);
              accu[tl] = mfma_bf16(au[u], b, accu[tl]);
            }
          }
        }
      }
    }
  } else {
    const float *wg = static_cast<const float *>(wgv) + wrow;
    const float *wu = static_cast<const float *>(wuv) + wrow;
    const float *x = static_cast<const float *>(xv);
    const int nsteps = H / 16;
    for (int s = wid; s < nsteps; s += 4 * U) {
      u32x4 ag[U], au[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ks = s + 4 * u;
        if (ks < nsteps) {
          const int k = ks * 16 + g * 4;
          ag[u] = ld16(wg + k);
          au[u] = ld16(wu + k);
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ks = s + 4 * u;
        if (ks < nsteps) {
          const int k = ks * 16 + g * 4;
#pragma unroll
          for (int tl = 0; tl < MT; ++tl) {
            if (tl < ntiles) {
              const u32x4 b = xval[tl] ? ld16(x + xoff[tl] + k) : u32x4{0, 0, 0, 0};
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                accg[tl] = mfma_f32(__uint_as_float(ag[u][j]), __uint_as_float(b[j]), accg[tl]);
                accu[tl] = mfma_f32(__uint_as_float(au[u][j]), __uint_as_float(b[j]), accu[tl]);
              }
            }
          }
        }
      }
    }
  }

#pragma unroll
  for (int tl = 0; tl < MT; ++tl) {
    if (tl < ntiles) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        red[wid][0][tl][rr][lane] = accg[tl][rr];
        red[wid][1][tl][rr][lane] = accu[tl][rr];
      }
    }
  }
  __syncthreads();
  for (int o = threadIdx.x; o < ntiles * 256; o += 256) {
    const int tl = o >> 8, rr = (o >> 6) & 3, ln = o & 63;
    const int c = tl * 16 + (ln & 15);
    if (c < ntok) {
      const float gs = red[0][0][tl][rr][ln] + red[1][0][tl][rr][ln] + red[2][0][tl][rr][ln] +
                       red[3][0][tl][rr][ln];
      const float us = red[0][1][tl][rr][ln] + red[1][1][tl][rr][ln] + red[2][1][tl][rr][ln] +
                       red[3][1][tl][rr][ln];
      const int neuron = row0 + 4 * (ln >> 4) + rr;
      const int p = rv.pair_at(q0 + c);
      hout[(size_t)p * d_ff + neuron] = silu(gs) * us;
    }
  }
}

// ---------------------------------------------------------------- neuron mask
// One block per pair.  The pair's d_ff activations sit in LDS as raw fp32
// bits; the score key is the bit pattern of |h| (an order-preserving uint32
// for non-negative floats, -0 == +0).  Four 8-bit MSB-first radix passes
// find the exact key tau of the k-th largest score and how many tau-equal
// neurons must be kept; one pass in index order then keeps key > tau plus
// the first tau-equal ones.  Outputs: ascending kept ids, w * h at them,
// and optionally the dense masked row hm (dense path).
__global__ __launch_bounds__(256) void neuron_topk_kernel(const float *__restrict__ h, RouteView rv,
                                                          int d_ff, int k,
                                                          int32_t *__restrict__ idx,
                                                          float *__restrict__ hact,
                                                          void *__restrict__ hm, int hm_bf16) {
  extern __shared__ uint32_t sbits[];
  __shared__ int hist[256];
  __shared__ int tmp[4];
  __shared__ int sel[2];
  const int tid = threadIdx.x;
  const int p = blockIdx.x;
  const float w = rv.weight(p);
  const float *hp = h + (size_t)p * d_ff;
  for (int j = tid; j < d_ff; j += 256) sbits[j] = __float_as_uint(hp[j]);
  __syncthreads();

  const bool keep_all = k >= d_ff;
  uint32_t tau = 0, pmask = 0;
  int krem = k;
  if (!keep_all && k > 0) {
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = 24 - 8 * pass;
      hist[tid] = 0;
      __syncthreads();
      for (int j = tid; j < d_ff; j += 256) {
        const uint32_t key = sbits[j] & 0x7fffffffu;
        if ((key & pmask) == tau) atomicAdd(&hist[(key >> shift) & 255u], 1);
      }
      __syncthreads();
      // thread tid owns digit 255 - tid: inclusive scan = keys with digit >= it
      const int cnt = hist[255 - tid];
      const int incl = block_incl_scan<256>(cnt, tmp);
      if (incl >= krem && incl - cnt < krem) {
        sel[0] = 255 - tid;
        sel[1] = krem - (incl - cnt);
      }
      __syncthreads();
      tau |= (uint32_t)sel[0] << shift;
      pmask |= 0xffu << shift;
      krem = sel[1];
      __syncthreads();
    }
  }

  // contiguous segment per thread, in index order
  const int C = (d_ff + 255) / 256;
  const int j0 = min(d_ff, tid * C), j1 = min(d_ff, j0 + C);
  int ngt = 0, neq = 0;
  if (!keep_all && k > 0) {
    for (int j = j0; j < j1; ++j) {
      const uint32_t key = sbits[j] & 0x7fffffffu;
      ngt += key > tau;
      neq += key == tau;
    }
  }
  const int gt_before = block_incl_scan<256>(ngt, tmp) - ngt;
  const int eq_before = block_incl_scan<256>(neq, tmp) - neq;
  int pos = keep_all ? j0 : gt_before + min(eq_before, krem);
  int eq_seen = eq_before;
  for (int j = j0; j < j1; ++j) {
    const uint32_t bits = sbits[j];
    const uint32_t key = bits & 0x7fffffffu;
    bool keep;
    if (keep_all) keep = true;
    else if (k == 0) keep = false;
    else if (key > tau) keep = true;
    else if (key == tau) keep = eq_seen++ < krem;
    else keep = false;
    const float v = w * __uint_as_float(bits);
    if (keep) {
      if (pos < k) {  // always true for finite input; keeps NaN input memory-safe
        if (idx) idx[(size_t)p * k + pos] = j;
        if (hact) hact[(size_t)p * k + pos] = v;
      }
      ++pos;
    }
    if (hm) {
      const float mv = keep ? v : 0.0f;
      if (hm_bf16)
        static_cast<uint16_t *>(hm)[(size_t)p * d_ff + j] = (uint16_t)f32_to_bf16_bits(mv);
      else
        static_cast<float *>(hm)[(size_t)p * d_ff + j] = mv;
    }
  }
}

// ---------------------------------------------------------------- sparse down
// Block = (pair, row chunk) x a slice of 64 * VEC output columns.  Each wave
// streams whole row slices (bf16: 1 KB, one 16-byte load per lane; fp32:
// 1 KB) of the kept rows i = chunk start + wave, +4, ..., 4 rows in flight,
// multiplying by the row's coefficient.  With idx == nullptr the rows are
// 0..k-1 (dense rows, coefficient row stride k).  The four wave partials
// are added in fixed order into partial[pair * n_chunks + chunk].
template <bool BF16>
__global__ __launch_bounds__(256) void down_rows_kernel(const void *__restrict__ wdv,
                                                        const int32_t *__restrict__ idx,
                                                        const float *__restrict__ coef,
                                                        RouteView rv, int H, int d_ff, int k,
                                                        int n_chunks, int R,
                                                        float *__restrict__ partial) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int SW = 64 * VEC;
  __shared__ float red[4][SW];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int pc = blockIdx.x;
  const int p = pc / n_chunks, c = pc - p * n_chunks;
  const int e = rv.expert_of_pair(p);
  const int i0 = c * R, i1 = min(k, i0 + R);
  const int col = blockIdx.y * SW + lane * VEC;
  const bool cv = col < H;
  const int32_t *ip = idx ? idx + (size_t)p * k : nullptr;
  const float *cp = coef + (size_t)p * k;
  const size_t ebase = (size_t)e * d_ff * H;
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;

  constexpr int U = 4;
  for (int i = i0 + wid; i < i1; i += 4 * U) {
    u32x4 q[U];
    float hv[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int ii = i + 4 * u;
      hv[u] = 0.f;
      q[u] = u32x4{0, 0, 0, 0};
      if (ii < i1) {
        int j = ip ? ip[ii] : ii;
        j = (unsigned)j < (unsigned)d_ff ? j : 0;  // memory-safe on any index input
        hv[u] = cp[ii];
        if (cv) {
          const size_t off = ebase + (size_t)j * H + col;
          q[u] = BF16 ? ld16(static_cast<const uint16_t *>(wdv) + off)
                      : ld16(static_cast<const float *>(wdv) + off);
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (BF16) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          acc[2 * jj] = fmaf(hv[u], bf16lo(q[u][jj]), acc[2 * jj]);
          acc[2 * jj + 1] = fmaf(hv[u], bf16hi(q[u][jj]), acc[2 * jj + 1]);
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[jj] = fmaf(hv[u], __uint_as_float(q[u][jj]), acc[jj]);
      }
    }
  }
#pragma unroll
  for (int v = 0; v < VEC; ++v) red[wid][lane * VEC + v] = acc[v];
  __syncthreads();
  for (int o = threadIdx.x; o < SW; o += 256) {
    const int cc = blockIdx.y * SW + o;
    if (cc < H)
      partial[(size_t)pc * H + cc] = red[0][o] + red[1][o] + red[2][o] + red[3][o];
  }
}

// ---------------------------------------------------------------- dense down (bf16)
// Dense-path down GEMM for one work item (expert, <=64 tokens) and 64
// output columns: out[tok, col] = sum_j hm[pair(tok), j] * W_d[e][j, col].
// W_d's K (= d_ff) is its row index, so 128-row x 64-col tiles are staged
// through LDS transposed ([col][k]) to give each lane the 8 consecutive k
// the MFMA B operand wants; the next tile is prefetched into registers
// while the current one is consumed.  Wave w owns columns 16w..16w+15 for
// up to 4 token tiles.
constexpr int kDKC = 128;
constexpr int kDenseTokGroup = 64;
__global__ __launch_bounds__(256) void down_dense_bf16_kernel(const uint16_t *__restrict__ wd,
                                                              const uint16_t *__restrict__ hm,
                                                              RouteView rv, int H, int d_ff,
                                                              float *__restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint16_t bt[64][kDKC + 8];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int e, q0, ntok;
  if (!find_item<kDenseTokGroup>(rv, blockIdx.x, e, q0, ntok)) return;
  const int ntiles = (ntok + 15) >> 4;
  const int r = lane & 15, g = lane >> 4;
  const int col0 = blockIdx.y * 64;

  size_t aoff[4];
  bool aval[4];
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) {
    const int c = tl * 16 + r;
    aval[tl] = c < ntok;
    aoff[tl] = aval[tl] ? (size_t)rv.pair_at(q0 + c) * d_ff : 0;
  }
  f32x4 acc[4];
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) acc[tl] = f32x4{0, 0, 0, 0};

  // staging map: 128 rows x 64 cols = 4 rows per thread, 8 columns each
  const int srow = tid >> 3, scol = (tid & 7) * 8;
  const uint16_t *wbase = wd + (size_t)e * d_ff * H + col0 + scol;
  u32x4 pf[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    pf[i] = srow + 32 * i < d_ff ? ld16(wbase + (size_t)(srow + 32 * i) * H) : u32x4{0, 0, 0, 0};

  for (int kb = 0; kb < d_ff; kb += kDKC) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = srow + 32 * i;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        bt[scol + 2 * j][kr] = (uint16_t)(pf[i][j] & 0xffffu);
        bt[scol + 2 * j + 1][kr] = (uint16_t)(pf[i][j] >> 16);
      }
    }
    __syncthreads();
    if (kb + kDKC < d_ff) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int kr = kb + kDKC + srow + 32 * i;
        pf[i] = kr < d_ff ? ld16(wbase + (size_t)kr * H) : u32x4{0, 0, 0, 0};
      }
    }
#pragma unroll
    for (int ks = 0; ks < kDKC / 32; ++ks) {
      if (kb + ks * 32 >= d_ff) break;  // d_ff is a multiple of 64, not of 128
      const u32x4 b = *reinterpret_cast<const u32x4 *>(&bt[16 * wid + r][ks * 32 + 8 * g]);
#pragma unroll
      for (int tl = 0; tl < 4; ++tl) {
        if (tl < ntiles) {
          const u32x4 a = aval[tl] ? ld16(hm + aoff[tl] + kb + ks * 32 + 8 * g) : u32x4{0, 0, 0, 0};
          acc[tl] = mfma_bf16(a, b, acc[tl]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int tl = 0; tl < 4; ++tl) {
    if (tl < ntiles) {
#pragma unroll
      for (int rr = 0; rr < 4; ++rr) {
        const int c = tl * 16 + 4 * g + rr;
        if (c < ntok) {
          const int p = rv.pair_at(q0 + c);
          partial[(size_t)p * H + col0 + 16 * wid + r] = acc[tl][rr];
        }
      }
    }
  }
}

// ---------------------------------------------------------------- combine
// y[t, :] = (accumulate ? y[t, :] : 0) + sum over slots, then chunks, of
// the token's partial rows: a fixed order, so reruns are bitwise equal.
__global__ __launch_bounds__(256) void combine_kernel(const float *__restrict__ partial, int H,
                                                      int top_k, int n_chunks, int accumulate,
                                                      float *__restrict__ y) {
  const int t = blockIdx.x;
  const int col = (blockIdx.y * 256 + threadIdx.x) * 4;
  if (col >= H) return;
  f32x4 s = accumulate ? *reinterpret_cast<const f32x4 *>(y + (size_t)t * H + col)
                       : f32x4{0, 0, 0, 0};
  const size_t rows = (size_t)top_k * n_chunks;
  const float *pp = partial + (size_t)t * rows * H + col;
  for (size_t i = 0; i < rows; ++i) s += *reinterpret_cast<const f32x4 *>(pp + i * H);
  *reinterpret_cast<f32x4 *>(y + (size_t)t * H + col) = s;
}

__global__ __launch_bounds__(256) void zero_kernel(float *__restrict__ y, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = 0.f;
}

// ---------------------------------------------------------------- host side

static RouteView make_view(const FfnArgs &a) {
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
static int n_items(const FfnArgs &a, int TG) {
  const int P = a.T * a.top_k;
  if (a.implicit) return a.E * ((a.T + TG - 1) / TG);
  return (a.E < P ? a.E : P) + P / TG;
}

static constexpr int kDownTargetBlocks = 2048;
static constexpr int kDownMinRows = 8;

static int slice_width(int bf16) { return bf16 ? 512 : 256; }

DownPlan plan_down(int P, int k, int H, int bf16) {
  DownPlan d{1, k > 0 ? k : 1};
  if (P <= 0 || k <= 0) return d;
  const int slices = (H + slice_width(bf16) - 1) / slice_width(bf16);
  long long want = (kDownTargetBlocks + (long long)P * slices - 1) / ((long long)P * slices);
  int maxc = k / kDownMinRows;
  if (maxc < 1) maxc = 1;
  int nc = (int)(want < maxc ? want : maxc);
  if (nc < 1) nc = 1;
  const int R = (k + nc - 1) / nc;
  d.rows_per_chunk = R;
  d.n_chunks = (k + R - 1) / R;
  return d;
}

size_t max_partial_rows(int P, int k, int H, int bf16) {
  const int slices = (H + slice_width(bf16) - 1) / slice_width(bf16);
  return (size_t)P + (size_t)(kDownTargetBlocks + slices - 1) / slices + 1;
}

static void launch_mask(const FfnArgs &a, const RouteView &rv, int32_t *idx, float *hact, void *hm,
                        int hm_bf16, hipStream_t stream) {
  const int P = a.T * a.top_k;
  timer_begin(kStageMask, stream);
  neuron_topk_kernel<<<P, 256, (size_t)a.d_ff * 4, stream>>>(a.h, rv, a.d_ff, a.k_keep, idx, hact,
                                                              hm, hm_bf16);
  timer_end(stream);
}

// A routed expert never holds more than T tokens, so at T <= 16 one token
// tile per item suffices (and keeps the kernel at high occupancy).
static void launch_gateup(const FfnArgs &a, const RouteView &rv, hipStream_t stream) {
  const bool one = a.T <= 16;
  dim3 grid(n_items(a, one ? 16 : 64), a.d_ff / 16);
  timer_begin(kStageGateup, stream);
  if (a.bf16) {
    if (one) gateup_swiglu_kernel<true, 1><<<grid, 256, 0, stream>>>(a.x, a.w_gate, a.w_up, rv, a.H, a.d_ff, a.h);
    else gateup_swiglu_kernel<true, 4><<<grid, 256, 0, stream>>>(a.x, a.w_gate, a.w_up, rv, a.H, a.d_ff, a.h);
  } else {
    if (one) gateup_swiglu_kernel<false, 1><<<grid, 256, 0, stream>>>(a.x, a.w_gate, a.w_up, rv, a.H, a.d_ff, a.h);
    else gateup_swiglu_kernel<false, 4><<<grid, 256, 0, stream>>>(a.x, a.w_gate, a.w_up, rv, a.H, a.d_ff, a.h);
  }
  timer_end(stream);
}

static void launch_combine(const FfnArgs &a, int n_chunks, hipStream_t stream) {
  dim3 grid(a.T, (a.H + 1023) / 1024);
  timer_begin(kStageCombine, stream);
  combine_kernel<<<grid, 256, 0, stream>>>(a.partial, a.H, a.top_k, n_chunks, a.accumulate, a.y);
  timer_end(stream);
}

static bool zero_contribution(const FfnArgs &a, hipStream_t stream) {
  if (a.k_keep > 0) return false;
  if (!a.accumulate) {
    const size_t n = (size_t)a.T * a.H;
    timer_begin(kStageZero, stream);
    zero_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(a.y, n);
    timer_end(stream);
  }
  return true;
}

static void launch_down_rows(const FfnArgs &a, const RouteView &rv, const int32_t *idx,
                             const float *coef, int k, const DownPlan &dp, hipStream_t stream) {
  const int P = a.T * a.top_k;
  dim3 grid(P * dp.n_chunks, (a.H + slice_width(a.bf16) - 1) / slice_width(a.bf16));
  timer_begin(kStageDownRows, stream);
  if (a.bf16)
    down_rows_kernel<true><<<grid, 256, 0, stream>>>(a.w_down, idx, coef, rv, a.H, a.d_ff, k,
                                                     dp.n_chunks, dp.rows_per_chunk, a.partial);
  else
    down_rows_kernel<false><<<grid, 256, 0, stream>>>(a.w_down, idx, coef, rv, a.H, a.d_ff, k,
                                                      dp.n_chunks, dp.rows_per_chunk, a.partial);
  timer_end(stream);
}

hipError_t launch_ffn_sparse(const FfnArgs &a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  if (zero_contribution(a, stream)) return hipGetLastError();
  const RouteView rv = make_view(a);
  const int P = a.T * a.top_k;
  launch_gateup(a, rv, stream);
  launch_mask(a, rv, a.idx, a.hact, nullptr, 0, stream);
  const DownPlan dp = plan_down(P, a.k_keep, a.H, a.bf16);
  launch_down_rows(a, rv, a.idx, a.hact, a.k_keep, dp, stream);
  launch_combine(a, dp.n_chunks, stream);
  return hipGetLastError();
}

hipError_t launch_ffn_dense(const FfnArgs &a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  if (zero_contribution(a, stream)) return hipGetLastError();
  const RouteView rv = make_view(a);
  const int P = a.T * a.top_k;
  launch_gateup(a, rv, stream);
  launch_mask(a, rv, a.idx, nullptr, a.hm, a.bf16, stream);
  if (a.bf16) {
    dim3 grid(n_items(a, kDenseTokGroup), a.H / 64);
    timer_begin(kStageDownDense, stream);
    down_dense_bf16_kernel<<<grid, 256, 0, stream>>>(static_cast<const uint16_t *>(a.w_down),
                                                     static_cast<const uint16_t *>(a.hm), rv, a.H,
                                                     a.d_ff, a.partial);
    timer_end(stream);
    launch_combine(a, 1, stream);
  } else {
    // fp32: every row of W_d against the dense masked row, on the row kernel
    const DownPlan dp = plan_down(P, a.d_ff, a.H, 0);
    launch_down_rows(a, rv, nullptr, static_cast<const float *>(a.hm), a.d_ff, dp, stream);
    launch_combine(a, dp.n_chunks, stream);
  }
  return hipGetLastError();
}

}  // namespace moe
