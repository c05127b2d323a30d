// Dense-path grouped GEMMs of the MoE expert FFN (gfx950, MFMA), for
// batches where an expert holds many tokens and the contraction is dense:
//
//   gateup_gemm   h = silu(W_g x) * (W_u x) per (expert, <= 128 tokens) item,
//                 weights in the packed fragment layout, tokens staged in LDS
//   down_dense    partial[pair, chunk] = hm . W_d over one K chunk (MFMA)
//   combine       y[t] (+)= the token's partials in a fixed order
//
// Method: the page "Uncovering Intra-expert Activation Sparsity for
// Efficient Mixture-of-Expert Model Execution", technical summary,
// Methodology (vLLM implementation): past a batch-size threshold the layer
// runs dense kernels instead of gathering kept rows.
#include "ffn_common.h"

namespace moe {


// ---------------------------------------------------------------- XCD-aware block order
// Workgroups go to the chip's 8 XCDs in turn (linear block id mod 8), and
// each XCD has its own L2.  This returns a logical linear index (x fastest,
// then y, then z) such that each XCD runs one contiguous range of it: the
// token items that share a weight tile (same y, z; x differs) then run on
// one XCD at about the same time and meet in its L2, instead of every XCD
// streaming every weight tile.  A bijection for any grid size.
__device__ __forceinline__ unsigned xcd_logical_block() {
  const unsigned nx = gridDim.x, nxy = nx * gridDim.y, total = nxy * gridDim.z;
  const unsigned L = blockIdx.x + nx * blockIdx.y + nxy * blockIdx.z;
  const unsigned xcd = L & 7u, slot = L >> 3, per = total >> 3, rem = total & 7u;
  return xcd * per + (xcd < rem ? xcd : rem) + slot;
}

// ---------------------------------------------------------------- gate / up GEMM
// Grouped GEMM for batches where an expert holds many tokens: work item =
// one expert and up to 128 of its tokens, block = 4 waves x 64 neurons
// (wave w owns neuron tile 4 * blockIdx.y + w for all 8 token tiles).  Per
// stage of two k-steps (128 bytes of every token row) the block gathers the
// item's token rows into an LDS tile (double-buffered, rows padded to avoid
// bank conflicts), while each wave streams its own packed gate and up
// fragments from HBM one stage ahead.  Each weight byte thus feeds up to 128
// tokens and each staged token row 4 neuron tiles; x is read from L2 once
// per 64 neurons instead of once per 16.  Epilogue: h = silu(g) * u, four
// consecutive neurons per lane, one 16-byte store per token.
// NTW = 2 gives each wave two neuron tiles (block = 128 neurons): every
// token fragment read from LDS then feeds twice the MFMAs, which halves the
// LDS traffic per flop where the contraction is MFMA-bound (many tokens
// per expert), and doubles the weight bytes each wave has in flight.
constexpr int kGemmTok = 128;               // tokens per work item (8 MFMA token tiles)
constexpr int kGemmRowB = 128 + 16;         // LDS bytes per staged token row (+ pad)

template <bool BF16, bool GO = false, int NTW = 1>
__global__ __launch_bounds__(256, 2) void gateup_gemm_kernel(const void *__restrict__ xv,
                                                             const void *__restrict__ wgv,
                                                             const void *__restrict__ wuv,
                                                             RouteView rv, int H, int d_ff,
                                                             float *__restrict__ hout) {
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][kGemmTok * kGemmRowB];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int e, q0, ntok;
  const unsigned qb = xcd_logical_block();
  const int bx = (int)(qb % gridDim.x), by = (int)(qb / gridDim.x);
  if (!find_item<kGemmTok>(rv, bx, e, q0, ntok)) return;  // block-uniform
  const int ntiles = (ntok + 15) >> 4;
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int KS = BF16 ? 32 : 16;        // elements per k-step (64 bytes of a row)
  const int nsteps = H / KS;                // even: H is a multiple of 64
  const int nit = nsteps / 2;               // stages of two k-steps

  // staging map: token rows tid / 8 + 32 i (i < 4), 16-byte chunk tid % 8
  const int srow = tid >> 3, schunk = tid & 7;
  const uint8_t *xrow[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = srow + 32 * i;
    xrow[i] = c < ntok ? static_cast<const uint8_t *>(xv) +
                             (size_t)(rv.pair_at(q0 + c) / rv.top_k) * H * EB + schunk * 16
                       : nullptr;
  }
  const int nt = (by * 4 + wid) * NTW;     // this wave's first neuron tile
  const size_t tstride = (size_t)nsteps * 1024;   // bytes of one neuron tile
  const size_t fbase = ((size_t)e * (d_ff / 16) + nt) * tstride + lane * 16;
  const uint8_t *wg = static_cast<const uint8_t *>(wgv) + fbase;
  const uint8_t *wu = static_cast<const uint8_t *>(wuv) + fbase;

  f32x4 accg[NTW][8], accu[NTW][8];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int tl = 0; tl < 8; ++tl) { accg[j][tl] = f32x4{0, 0, 0, 0}; accu[j][tl] = f32x4{0, 0, 0, 0}; }

  u32x4 stg[4], ag[NTW][2], au[NTW][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) stg[i] = xrow[i] ? ld16(xrow[i]) : u32x4{0, 0, 0, 0};
#pragma unroll
  for (int i = 0; i < 4; ++i)
    *reinterpret_cast<u32x4 *>(&xs[0][(srow + 32 * i) * kGemmRowB + schunk * 16]) = stg[i];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      ag[j][k] = ld16_nt(wg + j * tstride + (size_t)k * 1024);
      if (!GO) au[j][k] = ld16_nt(wu + j * tstride + (size_t)k * 1024);
    }
  __syncthreads();

  const int r = lane & 15, g = lane >> 4;
  for (int it = 0; it < nit; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < nit;
    u32x4 ng[NTW][2], nu[NTW][2];
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        stg[i] = xrow[i] ? ld16(xrow[i] + (size_t)(it + 1) * 128) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int k = 0; k < 2; ++k) {
          ng[j][k] = ld16_nt(wg + j * tstride + (size_t)(2 * it + 2 + k) * 1024);
          if (!GO) nu[j][k] = ld16_nt(wu + j * tstride + (size_t)(2 * it + 2 + k) * 1024);
        }
    }
    auto bfrag = [&](int k, int tl) {
      return *reinterpret_cast<const u32x4 *>(
          &xs[cur][(tl * 16 + r) * kGemmRowB + k * 64 + g * 16]);
    };
    auto tile = [&](int k, int tl, const u32x4 &b) {
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        if (BF16) {
          accg[j][tl] = mfma_bf16(ag[j][k], b, accg[j][tl]);
          if (!GO) accu[j][tl] = mfma_bf16(au[j][k], b, accu[j][tl]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            accg[j][tl] = mfma_f32(__uint_as_float(ag[j][k][q]), __uint_as_float(b[q]),
                                   accg[j][tl]);
            if (!GO)
              accu[j][tl] = mfma_f32(__uint_as_float(au[j][k][q]), __uint_as_float(b[q]),
                                     accu[j][tl]);
          }
        }
      }
    };
    // Each token fragment is read from LDS one tile ahead of its MFMAs, so
    // the LDS latency overlaps the matrix work instead of stalling it (rows
    // past the item's tokens hold zeros, so the read ahead is harmless).
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      u32x4 b = bfrag(k, 0);
#pragma unroll
      for (int tl = 0; tl < 8; ++tl) {
        if (tl < ntiles) {  // block-uniform
          const u32x4 bn = bfrag(k, tl < 7 ? tl + 1 : 7);
          tile(k, tl, b);
          b = bn;
        }
      }
    }
    if (more) {
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<u32x4 *>(&xs[cur ^ 1][(srow + 32 * i) * kGemmRowB + schunk * 16]) = stg[i];
#pragma unroll
      for (int j = 0; j < NTW; ++j)
#pragma unroll
        for (int k = 0; k < 2; ++k) { ag[j][k] = ng[j][k]; if (!GO) au[j][k] = nu[j][k]; }
    }
    __syncthreads();
  }

#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int neuron0 = (nt + j) * 16 + 4 * g;
#pragma unroll
    for (int tl = 0; tl < 8; ++tl) {
      const int c = tl * 16 + r;
      if (tl < ntiles && c < ntok) {
        const int p = rv.pair_at(q0 + c);
        f32x4 hv;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          hv[rr] = GO ? silu(accg[j][tl][rr]) : silu(accg[j][tl][rr]) * accu[j][tl][rr];
        *reinterpret_cast<f32x4 *>(hout + (size_t)p * d_ff + neuron0) = hv;
      }
    }
  }
}

// ---------------------------------------------------------------- dense down (bf16)
// Dense-path down GEMM: partial[pair, chunk, col] = sum over the chunk's k of
// hm[pair, k] * W_d[e][k, col], for a work item (expert, <= 128 of its
// tokens) x 64 output columns x one K chunk (blockIdx.z).  MFMA A = the
// masked h rows (k-contiguous, staged through LDS in padded rows); MFMA B
// needs k-contiguous columns of the row-major W_d, so each stage of 64 rows
// is packed into bf16 k-pairs and written transposed ([col][k]) into LDS.
// The k-pair slot is XOR-swizzled by the column, so the transposing writes
// and the 16-byte fragment reads both reach the 2-way minimum of bank
// conflicts.  Waves form a 2 x 2 grid: each owns 4 token tiles x 2 column
// tiles.  Both LDS tiles are double-buffered with one register stage.
constexpr int kDnTok = 128;                 // tokens per work item
constexpr int kDnCols = 64;                 // output columns per block
constexpr int kDnK = 64;                    // k per stage
constexpr int kDnArow = kDnK * 2 + 16;      // LDS bytes per staged hm row (+ pad)
constexpr int kDnBrow = kDnK * 2;           // LDS bytes per transposed W_d column

__device__ __forceinline__ int dn_swz(int col) { return 4 * ((col & 7) ^ ((col >> 3) & 7)); }

__global__ __launch_bounds__(256, 2) void down_dense_gemm_kernel(const uint16_t *__restrict__ wd,
                                                                 const uint16_t *__restrict__ hm,
                                                                 RouteView rv, int H, int d_ff,
                                                                 int kchunk,
                                                                 float *__restrict__ partial) {
  __shared__ __attribute__((aligned(16))) uint8_t as[2][kDnTok * kDnArow];
  __shared__ __attribute__((aligned(16))) uint32_t bs[2][kDnCols * kDnBrow / 4];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int e, q0, ntok;
  const unsigned qb = xcd_logical_block();
  const int bx = (int)(qb % gridDim.x), by = (int)(qb / gridDim.x % gridDim.y);
  if (!find_item<kDnTok>(rv, bx, e, q0, ntok)) return;  // block-uniform
  const int col0 = by * kDnCols;
  const int S = gridDim.z, sidx = (int)(qb / (gridDim.x * gridDim.y));
  const int k0 = sidx * kchunk;
  const int nit = (min(d_ff, k0 + kchunk) - k0) / kDnK;
  const int ntiles = (ntok + 15) >> 4;

  // A staging: rows tid / 8 + 32 i (i < 4), 16-byte chunk tid % 8 (8 k)
  const int arow = tid >> 3, achunk = tid & 7;
  const uint16_t *ap[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = arow + 32 * i;
    ap[i] = c < ntok ? hm + (size_t)rv.pair_at(q0 + c) * d_ff + k0 + achunk * 8 : nullptr;
  }
  // B staging: k-pair kp = tid / 8 (rows 2 kp, 2 kp + 1), columns 8 cg .. 8 cg + 7
  const int kp = tid >> 3, cg = tid & 7;
  const uint16_t *bp = wd + ((size_t)e * d_ff + k0 + 2 * kp) * H + col0 + 8 * cg;

  u32x4 sa[4], sb[2];
  auto load_stage = [&](int it) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[i] = ap[i] ? ld16(ap[i] + it * kDnK) : u32x4{0, 0, 0, 0};
    sb[0] = ld16_nt(bp + (size_t)it * kDnK * H);
    sb[1] = ld16_nt(bp + (size_t)it * kDnK * H + H);
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4 *>(&as[buf][(arow + 32 * i) * kDnArow + achunk * 16]) = sa[i];
#pragma unroll
    for (int c = 0; c < 8; ++c) {  // column 8 cg + c gets the pair (row 2 kp, row 2 kp + 1)
      const uint32_t lo = (sb[0][c >> 1] >> (16 * (c & 1))) & 0xffffu;
      const uint32_t hi = (sb[1][c >> 1] >> (16 * (c & 1))) & 0xffffu;
      const int col = 8 * cg + c;
      bs[buf][col * (kDnBrow / 4) + (kp ^ dn_swz(col))] = lo | (hi << 16);
    }
  };

  const int r = lane & 15, g = lane >> 4;
  const int wt = wid >> 1, wc = wid & 1;  // token tiles 4 wt .. 4 wt + 3, column tiles 2 wc, 2 wc + 1
  f32x4 acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i) { acc[i][0] = f32x4{0, 0, 0, 0}; acc[i][1] = f32x4{0, 0, 0, 0}; }

  if (nit > 0) {
    load_stage(0);
    store_stage(0);
  }
  __syncthreads();
  for (int it = 0; it < nit; ++it) {
    const int cur = it & 1;
    const bool more = it + 1 < nit;
    if (more) load_stage(it + 1);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 b[2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int col = (2 * wc + j) * 16 + r;
        const int w0 = (ks * 16 + 4 * g) ^ dn_swz(col);  // 4 k-pairs = this lane's 8 k
        b[j] = *reinterpret_cast<const u32x4 *>(&bs[cur][col * (kDnBrow / 4) + w0]);
      }
      auto afrag = [&](int i) {
        return *reinterpret_cast<const u32x4 *>(
            &as[cur][((4 * wt + i) * 16 + r) * kDnArow + ks * 64 + g * 16]);
      };
      // A fragments read one tile ahead of their MFMAs (rows past the
      // item's tokens hold zeros, so the read ahead is harmless)
      u32x4 av = afrag(0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * wt + i < ntiles) {  // wave-uniform
          const u32x4 an = afrag(i < 3 ? i + 1 : 3);
          acc[i][0] = mfma_bf16(av, b[0], acc[i][0]);
          acc[i][1] = mfma_bf16(av, b[1], acc[i][1]);
          av = an;
        }
      }
    }
    if (more) store_stage(cur ^ 1);
    __syncthreads();
  }
  // D: lane holds column r of each column tile, token rows 4 g + rr of each token tile
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tl = 4 * wt + i;
    if (tl >= ntiles) continue;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int c = tl * 16 + 4 * g + rr;
      if (c < ntok) {
        const size_t row = (size_t)rv.pair_at(q0 + c) * S + sidx;
#pragma unroll
        for (int j = 0; j < 2; ++j)
          partial[row * H + col0 + (2 * wc + j) * 16 + r] = acc[i][j][rr];
      }
    }
  }
}

// K chunks of the dense down GEMM: enough blocks to fill the chip when few
// work items exist (small batches), each chunk a multiple of 64 rows and at
// least 256.  A function of the shape only, so the workspace size and the
// launch agree.
static int dense_down_kchunk(int T, int E, int top_k, int H, int d_ff) {
  const long P = (long)T * top_k;
  const long items = (E < P ? E : P) + P / kDnTok;
  const long base = items * (H / kDnCols);
  long S = (1024 + base - 1) / base;
  const long smax = d_ff / 256 > 0 ? d_ff / 256 : 1;
  if (S > smax) S = smax;
  if (S < 1) S = 1;
  const long per = (d_ff + S - 1) / S;
  return (int)((per + kDnK - 1) / kDnK * kDnK);
}

// Partial rows the dense down GEMM may write at most T tokens: P * chunks
// <= P + 65536 P / (items H) with items >= min(E, P), so this bound holds for
// every smaller T too (a workspace sized for T serves any shorter call).
size_t dense_down_partial_rows(int T, int E, int top_k, int H) {
  const size_t P = (size_t)T * top_k;
  const size_t per_item = P > (size_t)E ? (P + E - 1) / E : 1;
  return P + (size_t)((65536 + H - 1) / H) * per_item;
}

// ---------------------------------------------------------------- combine
// y[t, :] = (accumulate ? y[t, :] : 0) + sum over slots, then chunks, of
// the token's partial rows: a fixed order, so reruns are bitwise equal.
__global__ __launch_bounds__(64) void combine_kernel(const float *__restrict__ partial, int H,
                                                      int top_k, int n_chunks, int accumulate,
                                                      float *__restrict__ y) {
  const int t = blockIdx.x;
  const int col = (blockIdx.y * 64 + threadIdx.x) * 4;
  if (col >= H) return;
  f32x4 s = accumulate ? *reinterpret_cast<const f32x4 *>(y + (size_t)t * H + col)
                       : f32x4{0, 0, 0, 0};
  const int rows = top_k * n_chunks;
  const float *pp = partial + (size_t)t * rows * H + col;
  int i = 0;
  for (; i + 8 <= rows; i += 8) {  // 8 loads in flight, added in row order
    f32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const f32x4 *>(pp + (size_t)(i + u) * H);
#pragma unroll
    for (int u = 0; u < 8; ++u) s += v[u];
  }
  for (; i < rows; ++i) s += *reinterpret_cast<const f32x4 *>(pp + (size_t)i * H);
  *reinterpret_cast<f32x4 *>(y + (size_t)t * H + col) = s;
}

// ---------------------------------------------------------------- host side

void launch_gateup_gemm(const FfnArgs &a, const RouteView &rv, bool gate_only, hipStream_t stream) {
  // two neuron tiles per wave for the bf16 SwiGLU contraction when d_ff
  // allows (a multiple of 128) and the grid still has >= 2 blocks per CU
  // (few items, e.g. a shared expert at T = 256, keep the narrow blocks)
  const int items = n_items(a, kGemmTok);
  const bool wide = a.bf16 && !gate_only && a.d_ff % 128 == 0 &&
                    (long)items * (a.d_ff / 128) >= 512;
  dim3 grid(items, a.d_ff / (wide ? 128 : 64));
#define MOE_GG(BF, GOV, N) \
  gateup_gemm_kernel<BF, GOV, N><<<grid, 256, 0, stream>>>(a.x, a.w_gate, a.w_up, rv, a.H, a.d_ff, a.h)
  if (a.bf16) {
    if (gate_only) MOE_GG(true, true, 1);
    else if (wide) MOE_GG(true, false, 2);
    else MOE_GG(true, false, 1);
  } else {
    if (gate_only) MOE_GG(false, true, 1); else MOE_GG(false, false, 1);
  }
#undef MOE_GG
}

hipError_t launch_down_dense(const FfnArgs &a, const RouteView &rv, hipStream_t stream) {
  const int kc = dense_down_kchunk(a.T, a.E, a.top_k, a.H, a.d_ff);
  const int S = (a.d_ff + kc - 1) / kc;
  if ((size_t)a.T * a.top_k * S > dense_down_partial_rows(a.T, a.E, a.top_k, a.H))
    return hipErrorInvalidValue;  // cannot happen: the bound covers every split count
  dim3 grid(n_items(a, kDnTok), a.H / kDnCols, S);
  timer_begin(kStageDownDense, stream);
  down_dense_gemm_kernel<<<grid, 256, 0, stream>>>(static_cast<const uint16_t *>(a.w_down),
                                                   static_cast<const uint16_t *>(a.hm), rv, a.H,
                                                   a.d_ff, kc, a.partial);
  timer_end(stream);
  dim3 cgrid(a.T, (a.H + 255) / 256);
  timer_begin(kStageCombine, stream);
  combine_kernel<<<cgrid, 64, 0, stream>>>(a.partial, a.H, a.top_k, S, a.accumulate, a.y);
  timer_end(stream);
  return hipGetLastError();
}

}  // namespace moe
