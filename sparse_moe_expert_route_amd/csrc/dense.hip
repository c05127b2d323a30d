// Grouped GEMMs of the MoE expert FFN (gfx950, MFMA), for batches where
// experts hold several tokens:
//
//   gateup_gemm   h = silu(W_g x) * (W_u x) per (expert, <= 128 tokens) item,
//                 weights in the packed fragment layout, tokens staged in LDS
//   down_skinny   partial[pair, chunk] = hm . W_d over one K chunk, items of
//                 <= 32 or 64 tokens (HBM-bound)
//   down_wide     the same for items of <= 128 tokens
//   down_packed   the same over a W_d copy packed in MFMA fragment order
//                 (moe_pack_down): weights straight into registers, items of
//                 32, 64 or 128 tokens
//   union_*       the sparse path's packed-rows form: each active expert's
//                 union of kept rows, for the two down GEMMs to gather
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

// The GEMMs that feed MFMAs straight from weight registers (gate/up, the
// packed down) raise their wave priority over each stage's MFMA run, so
// that of two waves sharing a SIMD the one with matrix work ready keeps
// issuing it (1024-token Llama-4-like shared expert, alternating runs:
// gate/up 187-190 -> 175 us, packed down 109-110 -> 103-104 us; the
// row-major down GEMMs, which stage weights through LDS, gained <= 1 %).
#ifndef MOE_GEMM_SETPRIO
#define MOE_GEMM_SETPRIO 1
#endif

// A compile-time int for the kernels' step lambdas.
template <int V>
struct SkIc {
  static constexpr int value = V;
};

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

// DEPTH > 1 (one neuron tile per wave, grids of few items): the weights
// stream DEPTH stages ahead through a ring of DEPTH + 1 register sets, so
// that a grid of a few hundred waves still keeps enough bytes in flight
// (three stages, always-on experts at 256 tokens: Llama-4-like 90.0 -> 81.3
// us, the DeepSeek-V2-like pair 85.3 -> 76.6 us).
// MT = token tiles per work item (8: 128 tokens).  The few-item SwiGLU grids
// take MT = 4 (64-token items): an expert past 64 tokens then streams its
// weight tile once per 64 tokens, but such a grid (under 2 blocks per CU)
// gains more from the extra blocks in flight.
template <bool BF16, bool GO = false, int NTW = 1, int DEPTH = 1, int MT = 8>
__global__ __launch_bounds__(256, 2) void gateup_gemm_kernel(const void *__restrict__ xv,
                                                             const void *__restrict__ wgv,
                                                             const void *__restrict__ wuv,
                                                             RouteView rv, int H, int d_ff,
                                                             float *__restrict__ hout) {
  constexpr int TOK = 16 * MT;  // tokens per work item
  constexpr int SR = MT / 2;     // staged 16-byte chunks per thread
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][TOK * kGemmRowB];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int e, q0, ntok;
  const unsigned qb = xcd_logical_block();
  const int bx = (int)(qb % gridDim.x), by = (int)(qb / gridDim.x);
  if (!find_item<TOK>(rv, bx, e, q0, ntok)) return;  // block-uniform
  const int ntiles = (ntok + 15) >> 4;
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int KS = BF16 ? 32 : 16;        // elements per k-step (64 bytes of a row)
  const int nsteps = H / KS;                // even: H is a multiple of 64
  const int nit = nsteps / 2;               // stages of two k-steps

  // staging map: token rows tid / 8 + 32 i (i < SR), 16-byte chunk tid % 8.
  // Rows past the item's tokens stage the first token's row (every load is
  // issued unconditionally, so that the compiler's waits count the loads in
  // flight); they only feed accumulator rows that are never stored.
  const int srow = tid >> 3, schunk = tid & 7;
  const uint8_t *xrow[SR];
#pragma unroll
  for (int i = 0; i < SR; ++i) {
    const int c = srow + 32 * i;
    xrow[i] = static_cast<const uint8_t *>(xv) +
              (size_t)(rv.pair_at(q0 + (c < ntok ? c : 0)) / rv.top_k) * H * EB + schunk * 16;
  }
  const int nt = (by * 4 + wid) * NTW;     // this wave's first neuron tile
  const size_t tstride = (size_t)nsteps * 1024;   // bytes of one neuron tile
  const size_t fbase = ((size_t)e * (d_ff / 16) + nt) * tstride + lane * 16;
  const uint8_t *wg = static_cast<const uint8_t *>(wgv) + fbase;
  const uint8_t *wu = static_cast<const uint8_t *>(wuv) + fbase;

  f32x4 accg[NTW][MT], accu[NTW][MT];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int tl = 0; tl < MT; ++tl) { accg[j][tl] = f32x4{0, 0, 0, 0}; accu[j][tl] = f32x4{0, 0, 0, 0}; }

  constexpr int R = DEPTH == 1 ? 1 : DEPTH + 1;  // weight register sets
  u32x4 stg[SR], ag[R][NTW][2], au[R][NTW][2];
  auto load_w = [&](int it, u32x4 (&g)[NTW][2], u32x4 (&u)[NTW][2]) {
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        g[j][k] = ld16_nt(wg + j * tstride + (size_t)(2 * it + k) * 1024);
        if (!GO) u[j][k] = ld16_nt(wu + j * tstride + (size_t)(2 * it + k) * 1024);
      }
  };
#pragma unroll
  for (int i = 0; i < SR; ++i) stg[i] = ld16(xrow[i]);
#pragma unroll
  for (int i = 0; i < SR; ++i)
    *reinterpret_cast<u32x4 *>(&xs[0][(srow + 32 * i) * kGemmRowB + schunk * 16]) = stg[i];
  load_w(0, ag[0], au[0]);
#pragma unroll
  for (int d = 1; d < DEPTH; ++d)
    if (d < nit) load_w(d, ag[d], au[d]);
  __syncthreads();

  const int r = lane & 15, g = lane >> 4;
  // Step it reads weight set SL = it % R.  STEADY: stage it + DEPTH exists
  // (no branch around the loads); DEPTH = 1 loads into a temporary set that
  // replaces set 0 after the MFMAs
  auto step = [&](int it, auto slc, auto steadyc) {
    constexpr int SL = decltype(slc)::value;
    constexpr bool STEADY = decltype(steadyc)::value;
    const bool more = STEADY || it + 1 < nit;
    const int cur = it & 1;
    u32x4 ng[NTW][2], nu[NTW][2];
    if (more) {
#pragma unroll
      for (int i = 0; i < SR; ++i) stg[i] = ld16(xrow[i] + (size_t)(it + 1) * 128);
      if (DEPTH == 1) load_w(it + 1, ng, nu);
    }
    if (DEPTH > 1 && (STEADY || it + DEPTH < nit))
      load_w(it + DEPTH, ag[(SL + DEPTH) % R], au[(SL + DEPTH) % R]);
    auto bfrag = [&](int k, int tl) {
      return *reinterpret_cast<const u32x4 *>(
          &xs[cur][(tl * 16 + r) * kGemmRowB + k * 64 + g * 16]);
    };
    auto tile = [&](int k, int tl, const u32x4 &b) {
#pragma unroll
      for (int j = 0; j < NTW; ++j) {
        if (BF16) {
          accg[j][tl] = mfma_bf16(ag[SL][j][k], b, accg[j][tl]);
          if (!GO) accu[j][tl] = mfma_bf16(au[SL][j][k], b, accu[j][tl]);
        } else {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            accg[j][tl] = mfma_f32(__uint_as_float(ag[SL][j][k][q]), __uint_as_float(b[q]),
                                   accg[j][tl]);
            if (!GO)
              accu[j][tl] = mfma_f32(__uint_as_float(au[SL][j][k][q]), __uint_as_float(b[q]),
                                     accu[j][tl]);
          }
        }
      }
    };
    // Each token fragment is read from LDS one tile ahead of its MFMAs, so
    // the LDS latency overlaps the matrix work instead of stalling it (a
    // read past the item's last tile feeds no MFMA).
    if (MOE_GEMM_SETPRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      u32x4 b = bfrag(k, 0);
#pragma unroll
      for (int tl = 0; tl < MT; ++tl) {
        if (tl < ntiles) {  // block-uniform
          const u32x4 bn = bfrag(k, tl < MT - 1 ? tl + 1 : MT - 1);
          tile(k, tl, b);
          b = bn;
        }
      }
    }
    if (MOE_GEMM_SETPRIO) __builtin_amdgcn_s_setprio(0);
    if (more) {
#pragma unroll
      for (int i = 0; i < SR; ++i)
        *reinterpret_cast<u32x4 *>(&xs[cur ^ 1][(srow + 32 * i) * kGemmRowB + schunk * 16]) = stg[i];
      if (DEPTH == 1) {
#pragma unroll
        for (int j = 0; j < NTW; ++j)
#pragma unroll
          for (int k = 0; k < 2; ++k) { ag[0][j][k] = ng[j][k]; if (!GO) au[0][j][k] = nu[j][k]; }
      }
    }
    __syncthreads();
  };
  if constexpr (DEPTH == 1) {
    for (int it = 0; it + 1 < nit; ++it) step(it, SkIc<0>{}, SkIc<1>{});
    if (nit > 0) step(nit - 1, SkIc<0>{}, SkIc<0>{});
  } else {
    static_assert(R <= 5, "the ring's steps are unrolled up to 5 sets");
    int it = 0;
    for (; it + R - 1 + DEPTH < nit; it += R) {
      step(it, SkIc<0>{}, SkIc<1>{});
      step(it + 1, SkIc<1 % R>{}, SkIc<1>{});
      if (R > 2) step(it + 2, SkIc<2 % R>{}, SkIc<1>{});
      if (R > 3) step(it + 3, SkIc<3 % R>{}, SkIc<1>{});
      if (R > 4) step(it + 4, SkIc<4 % R>{}, SkIc<1>{});
    }
    for (; it < nit; it += R) {
      step(it, SkIc<0>{}, SkIc<0>{});
      if (it + 1 < nit) step(it + 1, SkIc<1 % R>{}, SkIc<0>{});
      if (R > 2 && it + 2 < nit) step(it + 2, SkIc<2 % R>{}, SkIc<0>{});
      if (R > 3 && it + 3 < nit) step(it + 3, SkIc<3 % R>{}, SkIc<0>{});
      if (R > 4 && it + 4 < nit) step(it + 4, SkIc<4 % R>{}, SkIc<0>{});
    }
  }

  // the pair ids of the lane's MT token columns, all read before the stores
  int prow[MT];
#pragma unroll
  for (int tl = 0; tl < MT; ++tl) {
    const int c = tl * 16 + r;
    prow[tl] = rv.pair_at(q0 + (c < ntok ? c : 0));
  }
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int neuron0 = (nt + j) * 16 + 4 * g;
#pragma unroll
    for (int tl = 0; tl < MT; ++tl) {
      const int c = tl * 16 + r;
      if (tl < ntiles && c < ntok) {
        const int p = prow[tl];
        f32x4 hv;
#pragma unroll
        for (int rr = 0; rr < 4; ++rr)
          hv[rr] = GO ? silu(accg[j][tl][rr]) : silu(accg[j][tl][rr]) * accu[j][tl][rr];
        *reinterpret_cast<f32x4 *>(hout + (size_t)p * d_ff + neuron0) = hv;
      }
    }
  }
}

// ---------------------------------------------------------------- packed down GEMM
// The dense path's down product when the caller passes W_d packed
// (moe_pack_down): the gate/up GEMM's structure with W_d^T as the MFMA A
// operand, so the weights stream straight from memory in fragment order and
// no weight tile passes through LDS.  Work item = one expert and up to
// 16 * MT of its tokens; block = 4 waves x NTW column tiles of 16 each;
// blockIdx.z = one chunk of d_ff.  Per stage of two k-steps the block
// stages the item's coefficient rows (masked, weighted h, bf16,
// k-contiguous) into a double-buffered LDS tile, read one tile ahead of the
// MFMAs as in the gate/up GEMM; each wave streams its own W_d fragments
// DEPTH stages ahead: DEPTH = 2 through a ring of 3 register sets (the set
// a stage's MFMAs read is never a load target meanwhile), DEPTH = 1 into a
// temporary set that replaces the current one after the stage's MFMAs.
// Items of 128 tokens are bound by the matrix work and keep one stage in
// flight (their accumulators fill the registers); items of 32 or 64 tokens
// stream W_d at a few flops per byte, where two stages in flight keep more
// bytes moving.
// Epilogue: 4 consecutive columns per lane, one 16-byte store per token.
// CW (always-on experts): W_d through ordinary cached loads instead of the
// streaming hint.  Every item of such a group reads the same W_d tiles, and
// their blocks run on one XCD at about the same time (xcd_logical_block),
// so the tiles are worth keeping (1024-token Llama-4-like shared expert
// 98.4 -> 95.9 us, 256 tokens 44.3 -> 38.0 us; on routed experts, whose
// items mostly belong to different experts, the hint stays: 262 -> 310 us
// without it).
template <int NTW, int MT, int DEPTH, bool CW = false>
__global__ __launch_bounds__(256, 2) void down_packed_kernel(const uint8_t *__restrict__ wdp,
                                                             const uint16_t *__restrict__ hm,
                                                             RouteView rv, int H, int d_ff,
                                                             int kchunk,
                                                             float *__restrict__ partial) {
  constexpr int TOK = 16 * MT;       // tokens per item
  constexpr int SR = MT / 2;         // staged 16-byte chunks per thread (rows tid / 8 + 32 i)
  // W_d register sets (DEPTH = 1: a two-set ring unrolled by two spilled
  // at 128 tokens x 64 columns, or, with the loads held at the stage's top,
  // ran slower; the temporary set is renamed by the compiler instead)
  constexpr int R = DEPTH == 1 ? 1 : DEPTH + 1;
  __shared__ __attribute__((aligned(16))) uint8_t xs[2][TOK * kGemmRowB];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int e, q0, ntok;
  const unsigned qb = xcd_logical_block();
  const int bx = (int)(qb % gridDim.x), by = (int)(qb / gridDim.x % gridDim.y);
  if (!find_item<TOK>(rv, bx, e, q0, ntok)) return;  // block-uniform
  const int S = gridDim.z, sidx = (int)(qb / (gridDim.x * gridDim.y));
  const int ntiles = (ntok + 15) >> 4;
  const int k0 = sidx * kchunk;                                  // a multiple of 64
  const int nit = max(0, (min(d_ff, k0 + kchunk) - k0) / 64);    // stages of two k-steps

  // staging map: coefficient rows tid / 8 + 32 i (i < SR), 16-byte chunk
  // tid % 8; rows past the item's tokens stage the first token's row (they
  // only feed accumulator columns that are never stored)
  const int srow = tid >> 3, schunk = tid & 7;
  const uint8_t *xrow[SR];
#pragma unroll
  for (int i = 0; i < SR; ++i) {
    const int c = srow + 32 * i;
    xrow[i] = reinterpret_cast<const uint8_t *>(
                  hm + (size_t)rv.pair_at(q0 + (c < ntok ? c : 0)) * d_ff + k0) + schunk * 16;
  }
  const int nt = (by * 4 + wid) * NTW;             // this wave's first column tile
  const size_t tstride = (size_t)(d_ff / 32) * 1024;  // bytes of one column tile
  const uint8_t *wa = wdp + ((size_t)e * (H / 16) + nt) * tstride + (size_t)(k0 / 32) * 1024 + lane * 16;

  f32x4 acc[NTW][MT];
#pragma unroll
  for (int j = 0; j < NTW; ++j)
#pragma unroll
    for (int tl = 0; tl < MT; ++tl) acc[j][tl] = f32x4{0, 0, 0, 0};

  u32x4 stg[SR], aw[R][NTW][2];
  auto load_w = [&](int it, u32x4 (&dst)[NTW][2]) {
#pragma unroll
    for (int j = 0; j < NTW; ++j)
#pragma unroll
      for (int k = 0; k < 2; ++k) {
        const uint8_t *p = wa + j * tstride + (size_t)(2 * it + k) * 1024;
        dst[j][k] = CW ? ld16(p) : ld16_nt(p);
      }
  };
  if (nit > 0) {
#pragma unroll
    for (int i = 0; i < SR; ++i) stg[i] = ld16(xrow[i]);
#pragma unroll
    for (int i = 0; i < SR; ++i)
      *reinterpret_cast<u32x4 *>(&xs[0][(srow + 32 * i) * kGemmRowB + schunk * 16]) = stg[i];
    load_w(0, aw[0]);
    if (DEPTH > 1 && nit > 1) load_w(1, aw[1]);
  }
  __syncthreads();

  const int r = lane & 15, g = lane >> 4;
  // Step it reads W_d set SL = it % R; STEADY: stage it + DEPTH exists (so
  // every load is issued unconditionally and the compiler's waits count
  // the loads in flight instead of draining them)
  auto step = [&](int it, auto slc, auto steadyc) {
    constexpr int SL = decltype(slc)::value;
    constexpr bool STEADY = decltype(steadyc)::value;
    const int cur = it & 1;
    const bool more = STEADY || it + 1 < nit;
    if (more) {
#pragma unroll
      for (int i = 0; i < SR; ++i) stg[i] = ld16(xrow[i] + (size_t)(it + 1) * 128);
    }
    u32x4 nw[NTW][2];
    if (STEADY || it + DEPTH < nit) load_w(it + DEPTH, DEPTH == 1 ? nw : aw[(SL + DEPTH) % R]);
    auto bfrag = [&](int k, int tl) {
      return *reinterpret_cast<const u32x4 *>(&xs[cur][(tl * 16 + r) * kGemmRowB + k * 64 + g * 16]);
    };
    if (MOE_GEMM_SETPRIO) __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      u32x4 b = bfrag(k, 0);
#pragma unroll
      for (int tl = 0; tl < MT; ++tl) {
        if (tl < ntiles) {  // block-uniform
          const u32x4 bn = bfrag(k, tl < MT - 1 ? tl + 1 : MT - 1);
#pragma unroll
          for (int j = 0; j < NTW; ++j) acc[j][tl] = mfma_bf16(aw[SL][j][k], b, acc[j][tl]);
          b = bn;
        }
      }
    }
    if (MOE_GEMM_SETPRIO) __builtin_amdgcn_s_setprio(0);
    if (more) {
#pragma unroll
      for (int i = 0; i < SR; ++i)
        *reinterpret_cast<u32x4 *>(&xs[cur ^ 1][(srow + 32 * i) * kGemmRowB + schunk * 16]) = stg[i];
      if (DEPTH == 1) {
#pragma unroll
        for (int j = 0; j < NTW; ++j) { aw[0][j][0] = nw[j][0]; aw[0][j][1] = nw[j][1]; }
      }
    }
    __syncthreads();
  };
  int it = 0;
  for (; it + R - 1 + DEPTH < nit; it += R) {
    step(it, SkIc<0>{}, SkIc<1>{});
    if (R > 1) step(it + 1, SkIc<1 % R>{}, SkIc<1>{});
    if (R > 2) step(it + 2, SkIc<2 % R>{}, SkIc<1>{});
  }
  for (; it < nit; it += R) {
    step(it, SkIc<0>{}, SkIc<0>{});
    if (R > 1 && it + 1 < nit) step(it + 1, SkIc<1 % R>{}, SkIc<0>{});
    if (R > 2 && it + 2 < nit) step(it + 2, SkIc<2 % R>{}, SkIc<0>{});
  }

  // D: lane holds token column r of each token tile, output columns 4 g ..
  // 4 g + 3 of each column tile; the pair ids are all read before the stores
  int prow[MT];
#pragma unroll
  for (int tl = 0; tl < MT; ++tl) {
    const int c = tl * 16 + r;
    prow[tl] = rv.pair_at(q0 + (c < ntok ? c : 0));
  }
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int col = (nt + j) * 16 + 4 * g;
#pragma unroll
    for (int tl = 0; tl < MT; ++tl) {
      const int c = tl * 16 + r;
      if (tl < ntiles && c < ntok)
        *reinterpret_cast<f32x4 *>(partial + ((size_t)prow[tl] * S + sidx) * H + col) = acc[j][tl];
    }
  }
}

// ---------------------------------------------------------------- skinny down GEMM
// The down product for items of at most 16 * MT tokens of one expert (a few
// tokens per expert: HBM-bound on W_d).  Block = 4 waves x 256 output
// columns x one K chunk; stage = 64 W_d rows x 256 columns (32 KB).  Each
// thread loads 8 rows x 8 columns (8 x 16 B, one stage ahead in registers,
// so a block keeps 32 KB in flight), transposes them in registers into 8
// k-contiguous 16-byte column fragments (the MFMA B layout) and writes
// those to LDS: column stride 144 B, 16-byte slot = k-chunk ^ ((col >> 4) &
// 7), which keeps both the writes and the fragment reads free of bank
// conflicts.  The coefficients (A: token rows, k-contiguous) come straight
// from global memory in the MFMA layout, also one stage ahead.  Wave w
// owns columns 64 w .. 64 w + 63 (4 column tiles) for all MT token tiles.
// UNION (the sparse path's packed-rows form): k runs over the expert's
// union of kept rows (urow[e * d_ff ..], ascending, ucnt[e] of them), whose
// row ids each thread fetches two stages ahead, and hm is then the
// coefficients compacted to the same positions (hmu, zero-padded to a
// multiple of 64).  Rows past the union are never read.
constexpr int kSkCols = 256;   // output columns per block
constexpr int kSkK = 64;       // k per stage
constexpr int kSkColB = 144;   // LDS bytes per staged column (128 + 16 pad)
#ifndef MOE_SKINNY_DEPTH
#define MOE_SKINNY_DEPTH 2
#endif
// W_d stages in flight per thread (one where two would spill registers)
template <int MT, bool UNION>
constexpr int sk_depth() { return MT == 4 && UNION ? 1 : MOE_SKINNY_DEPTH; }

__device__ __forceinline__ int sk_off(int col, int chunk) {
  return col * kSkColB + ((chunk ^ ((col >> 4) & 7)) << 4);
}

template <int MT, bool UNION, int DEPTH>
__global__ __launch_bounds__(256, 2) void down_skinny_kernel(const uint16_t *__restrict__ wd,
                                                             const uint16_t *__restrict__ hm,
                                                             RouteView rv, int H, int d_ff,
                                                             int kchunk,
                                                             float *__restrict__ partial,
                                                             const int32_t *__restrict__ urow,
                                                             const int32_t *__restrict__ ucnt) {
  __shared__ __attribute__((aligned(16))) uint8_t bs[2][kSkCols * kSkColB];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int e, q0, ntok;
  const unsigned qb = xcd_logical_block();
  const int bx = (int)(qb % gridDim.x), by = (int)(qb / gridDim.x % gridDim.y);
  if (!find_item<16 * MT>(rv, bx, e, q0, ntok)) return;  // block-uniform
  const int col0 = by * kSkCols;
  const int S = gridDim.z, sidx = (int)(qb / (gridDim.x * gridDim.y));
  int uc = d_ff, kend = d_ff;
  if (UNION) {  // the chunks split the union, whose size only the device knows
    uc = ucnt[e];
    uc = uc < 0 ? 0 : (uc > d_ff ? d_ff : uc);
    kend = (uc + kSkK - 1) / kSkK * kSkK;  // hm is zero past uc up to here
    kchunk = ((uc + S - 1) / S + kSkK - 1) / kSkK * kSkK;
  }
  const int k0 = sidx * kchunk;
  const int nit = max(0, (min(kend, k0 + kchunk) - k0) / kSkK);

  // B: rows 8 rg .. 8 rg + 7 of a stage, columns col0 + 8 cg .. + 7
  const int rg = tid >> 5, cg = tid & 31;
  // Every load below is issued unconditionally (lanes without work read a
  // valid stand-in address), so that the compiler's waits can count the
  // loads still in flight instead of draining them all.  Columns past H
  // (H is a multiple of 64) read column block col0 and only feed output
  // columns that are never stored; token rows past the item read the first
  // token's row and only feed accumulator rows that are never stored.
  const bool colok = col0 + 8 * cg < H;
  const uint16_t *bcol = wd + (size_t)e * d_ff * H + (colok ? col0 + 8 * cg : col0);
  // A: token 16 mt + r of the item, k = 8 g .. 8 g + 7 of each 32-k step
  const int r = lane & 15, g = lane >> 4;
  const uint16_t *ap[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int c = 16 * mt + r;
    ap[mt] = hm + (size_t)rv.pair_at(q0 + (c < ntok ? c : 0)) * d_ff + k0 + 8 * g;
  }
  // UNION: positions past the union count (up to the 64-row stage) read the
  // union's first row, and their W_d values are replaced by zeros
  const int32_t *ur = UNION ? urow + (size_t)e * d_ff : nullptr;
  int row0 = 0;
  if (UNION && uc > 0) row0 = min(max(ur[0], 0), d_ff - 1);
  int rows[8];           // UNION: row ids of the stage to load next
  uint32_t rvalid = 0u;  // UNION: bit i: rows[i] lies inside the union
  u32x4 rn[2];      // UNION: row ids of the stage after that, in flight
  auto fetch_rows = [&](int it) {  // q + 8 <= kend <= d_ff: inside e's list
    const int q = k0 + it * kSkK + 8 * rg;
    rn[0] = ld16(ur + q);
    rn[1] = ld16(ur + q + 4);
  };
  auto take_rows = [&](int it) {
    const int q = k0 + it * kSkK + 8 * rg;
    rvalid = 0u;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int v = (int)rn[i >> 2][i & 3];
      const bool ok = q + i < uc && (unsigned)v < (unsigned)d_ff;
      rows[i] = ok ? v : row0;
      rvalid |= ok ? 1u << i : 0u;
    }
  };

  // W_d stages in flight: DEPTH register sets (stage it + DEPTH is issued
  // while stage it is multiplied); coefficients one stage ahead
  u32x4 sb[DEPTH][8], sa[MT][2];
  auto load_b = [&](int it, u32x4 (&dst)[8]) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = UNION ? rows[i] : k0 + it * kSkK + 8 * rg + i;
      dst[i] = ld16_nt(bcol + (size_t)row * H);
    }
  };
  auto load_a = [&](int it) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks)
        sa[mt][ks] = ld16(ap[mt] + it * kSkK + 32 * ks);
  };
  // column 8 cg + c gets rows 8 rg .. 8 rg + 7 as one k-contiguous fragment
  // (UNION: zeros for rows outside the union, valid = that stage's rvalid)
  auto store_b = [&](int buf, const u32x4 (&src)[8], uint32_t valid) {
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const int j = c >> 1;
      u32x4 o;
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        uint32_t lo = src[2 * w][j], hi = src[2 * w + 1][j];
        if (UNION) {
          lo = (valid >> (2 * w)) & 1u ? lo : 0u;
          hi = (valid >> (2 * w + 1)) & 1u ? hi : 0u;
        }
        o[w] = (c & 1) ? ((lo >> 16) | (hi & 0xffff0000u)) : ((lo & 0xffffu) | (hi << 16));
      }
      *reinterpret_cast<u32x4 *>(&bs[buf][sk_off(8 * cg + c, rg)]) = o;
    }
  };

  f32x4 acc[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) acc[mt][ct] = f32x4{0, 0, 0, 0};

  u32x4 a_cur[MT][2];
  uint32_t vb[DEPTH];  // UNION: rvalid of the stage in each register set
  if (nit > 0) {
    if (UNION) {
      fetch_rows(0);
      take_rows(0);
      fetch_rows(min(1, nit - 1));
    }
    vb[0] = rvalid;
    load_b(0, sb[0]);
    load_a(0);
    if (DEPTH == 2 && nit > 1) {
      if (UNION) {
        take_rows(1);
        fetch_rows(min(2, nit - 1));
      }
      vb[DEPTH - 1] = rvalid;
      load_b(1, sb[DEPTH - 1]);
    }
    store_b(0, sb[0], vb[0]);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) { a_cur[mt][0] = sa[mt][0]; a_cur[mt][1] = sa[mt][1]; }
  }
  __syncthreads();
  // One step: multiply stage it (LDS buffer it & 1, coefficients a_cur),
  // with stage it + 1's coefficients and stage it + DEPTH's W_d rows (into
  // register set SL = it % DEPTH, whose stage is already in LDS) issued
  // first, then stage it + 1 written from its register set to the other
  // buffer.  STEADY: every load and store is in range (no branch around a
  // load, so the compiler's waits count the loads in flight exactly).
  auto step = [&](int it, auto slc, auto steadyc) {
    constexpr int SL = decltype(slc)::value;
    constexpr bool STEADY = decltype(steadyc)::value;
    const int cur = it & 1;
    const int ahead = it + DEPTH;
    if (STEADY || it + 1 < nit) load_a(it + 1);
    if (STEADY || ahead < nit) {
      if (UNION) {
        take_rows(ahead);
        fetch_rows(min(ahead + 1, nit - 1));
      }
      vb[SL] = rvalid;
      load_b(ahead, sb[SL]);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 b[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
        b[ct] = *reinterpret_cast<const u32x4 *>(&bs[cur][sk_off(64 * wid + 16 * ct + r, 4 * ks + g)]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        if (16 * mt < ntok)  // block-uniform
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) acc[mt][ct] = mfma_bf16(a_cur[mt][ks], b[ct], acc[mt][ct]);
    }
    if (STEADY || it + 1 < nit) {
      store_b(cur ^ 1, sb[(SL + 1) % DEPTH], vb[(SL + 1) % DEPTH]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) { a_cur[mt][0] = sa[mt][0]; a_cur[mt][1] = sa[mt][1]; }
    }
    __syncthreads();
  };
  int it = 0;
  for (; it + DEPTH + 1 < nit; it += DEPTH) {
    step(it, SkIc<0>{}, SkIc<1>{});
    if (DEPTH == 2) step(it + 1, SkIc<1 % DEPTH>{}, SkIc<1>{});
  }
  for (; it < nit; it += DEPTH) {
    step(it, SkIc<0>{}, SkIc<0>{});
    if (DEPTH == 2 && it + 1 < nit) step(it + 1, SkIc<1 % DEPTH>{}, SkIc<0>{});
  }
  // D: lane holds column r of each column tile, token rows 4 g + rr of each
  // token tile; the rows' pair ids are all read before the first store
  int prow[MT][4];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int c = 16 * mt + 4 * g + rr;
      prow[mt][rr] = rv.pair_at(q0 + (c < ntok ? c : 0));
    }
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int c = 16 * mt + 4 * g + rr;
      if (c < ntok) {
        const size_t row = (size_t)prow[mt][rr] * S + sidx;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int col = col0 + 64 * wid + 16 * ct + r;
          if (col < H) partial[row * H + col] = acc[mt][ct][rr];
        }
      }
    }
  }
}

// Token tiles per skinny item for this call (0: the 128-token GEMM instead).
// An expert with more tokens than one item holds is split over items that
// each stream its rows again, so the tiles cover well past the average
// count n (the busiest expert of a routed batch holds about n + 3 sqrt(n):
// 28 at n = 16); tiles past an item's tokens cost no MFMA.
#ifndef MOE_SKINNY_MT2_MAX
#define MOE_SKINNY_MT2_MAX 16  // routed: average tokens per expert for 2 tiles
#endif
#ifndef MOE_SKINNY_MT4_MAX
#define MOE_SKINNY_MT4_MAX 40  // routed: ... for 4 tiles
#endif
static int skinny_tiles(int T, int E, int top_k, int implicit) {
  const long P = (long)T * top_k;
  const long per_expert = implicit ? T : P / (E < P ? E : P);
  if (implicit) return per_expert <= 32 ? 2 : (per_expert <= 64 ? 4 : 0);
  return per_expert <= MOE_SKINNY_MT2_MAX ? 2 : (per_expert <= MOE_SKINNY_MT4_MAX ? 4 : 0);
}

// K chunks of the skinny GEMM: enough for ~2048 blocks (a lone shared
// expert at a few tokens has only H / 256 column blocks), each chunk >= 256
// rows, at most 16, and at most max(4, 1024 / P) (dense_down_partial_rows
// bounds the partial rows this gives).
static int skinny_splits(int T, int E, int top_k, int implicit, int H, int d_ff, int mt) {
  const long P = (long)T * top_k;
  const long items = implicit ? (long)E * ((T + 16 * mt - 1) / (16 * mt))
                              : (E < P ? E : P) + P / (16 * mt);
  const long base = items * ((H + kSkCols - 1) / kSkCols);
  long S = (2048 + base - 1) / base;
  const long smax = d_ff / 256 > 0 ? d_ff / 256 : 1;
  if (S > smax) S = smax;
  if (S > 16) S = 16;
  const long pmax = P > 0 && 1024 / P > 4 ? 1024 / P : 4;
  if (S > pmax) S = pmax;
  return S < 1 ? 1 : (int)S;
}

// ---------------------------------------------------------------- wide down GEMM
// The down product for items of up to 128 tokens of one expert (many
// tokens per expert: the MFMA-bound shared expert at large batches, routed
// experts past the skinny GEMM's range).  Block = 4 waves in a 2 x 2 grid x
// 128 output columns x one K chunk; wave (wt, wc) owns tokens 64 wt ..
// 64 wt + 63 (4 token tiles) x columns 64 wc .. 64 wc + 63 (4 column
// tiles), so each k-step reads 4 + 4 fragments for 16 MFMAs.  Stage = 64
// k: the coefficient rows (A, k-contiguous) are staged to LDS as they are
// (rows padded to 144 bytes); the W_d rows (B) are transposed in registers,
// each thread holding 4 rows x 8 columns, into 8-byte k-runs written to a
// column-major LDS tile (column stride 144 bytes, 16-byte slot = k-chunk ^
// ((col >> 4) & 7): no bank conflicts for the writes or the fragment reads).
// Both tiles are double-buffered; DEPTH register stages are in flight (the
// k loop is latency-bound with one); every load is issued unconditionally
// (see down_skinny_kernel).  UNION as there.
constexpr int kWdTok = 128;   // tokens per work item
constexpr int kWdCols = 128;  // output columns per block
constexpr int kWdK = 64;      // k per stage
constexpr int kWdRowB = 144;  // LDS bytes per staged coefficient row / W_d column
// Register stages in flight.  Measured at Llama-4-like T = 1024 (shared
// expert / routed experts): one stage 159 / 317 us, two 156 / 318 us, two
// with cached instead of non-temporal W_d loads 152 / 331 us; the stage
// is not latency-bound, so one it is.
constexpr int kWdDepth = 1;

template <bool UNION, int DEPTH>
__global__ __launch_bounds__(256, 2) void down_wide_kernel(const uint16_t *__restrict__ wd,
                                                           const uint16_t *__restrict__ hm,
                                                           RouteView rv, int H, int d_ff,
                                                           int kchunk,
                                                           float *__restrict__ partial,
                                                           const int32_t *__restrict__ urow,
                                                           const int32_t *__restrict__ ucnt) {
  __shared__ __attribute__((aligned(16))) uint8_t as[2][kWdTok * kWdRowB];
  __shared__ __attribute__((aligned(16))) uint8_t bs[2][kWdCols * kWdRowB];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  int e, q0, ntok;
  const unsigned qb = xcd_logical_block();
  const int bx = (int)(qb % gridDim.x), by = (int)(qb / gridDim.x % gridDim.y);
  if (!find_item<kWdTok>(rv, bx, e, q0, ntok)) return;  // block-uniform
  const int col0 = by * kWdCols;
  const int S = gridDim.z, sidx = (int)(qb / (gridDim.x * gridDim.y));
  int uc = d_ff, kend = d_ff;
  if (UNION) {  // the chunks split the union, whose size only the device knows
    uc = ucnt[e];
    uc = uc < 0 ? 0 : (uc > d_ff ? d_ff : uc);
    kend = (uc + kWdK - 1) / kWdK * kWdK;  // hm is zero past uc up to here
    kchunk = ((uc + S - 1) / S + kWdK - 1) / kWdK * kWdK;
  }
  const int k0 = sidx * kchunk;
  const int nit = max(0, (min(kend, k0 + kchunk) - k0) / kWdK);
  const int ntiles = (ntok + 15) >> 4;

  // A staging: rows tid / 8 + 32 i (i < 4), 16-byte chunk tid % 8; rows past
  // the item's tokens stage the first token's row (never-stored accumulators)
  const int arow = tid >> 3, achunk = tid & 7;
  const uint16_t *ap[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int c = arow + 32 * i;
    ap[i] = hm + (size_t)rv.pair_at(q0 + (c < ntok ? c : 0)) * d_ff + k0 + achunk * 8;
  }
  // B staging: rows 4 rg .. 4 rg + 3 of a stage, columns col0 + 8 cg .. + 7
  // (columns past H, a multiple of 64, read column block col0 and feed only
  // never-stored outputs)
  const int rg = tid >> 4, cg = tid & 15;
  const bool colok = col0 + 8 * cg < H;
  const uint16_t *bcol = wd + (size_t)e * d_ff * H + (colok ? col0 + 8 * cg : col0);
  const int32_t *ur = UNION ? urow + (size_t)e * d_ff : nullptr;
  int row0 = 0;
  if (UNION && uc > 0) row0 = min(max(ur[0], 0), d_ff - 1);
  int rows[4];
  uint32_t rvalid = 0u;
  u32x4 rn = u32x4{0, 0, 0, 0};  // UNION: row ids of the next stage, in flight
  auto fetch_rows = [&](int it) {  // q + 4 <= kend <= d_ff: inside e's list
    rn = ld16(ur + k0 + it * kWdK + 4 * rg);
  };
  auto take_rows = [&](int it) {
    const int q = k0 + it * kWdK + 4 * rg;
    rvalid = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int v = (int)rn[i];
      const bool ok = q + i < uc && (unsigned)v < (unsigned)d_ff;
      rows[i] = ok ? v : row0;
      rvalid |= ok ? 1u << i : 0u;
    }
  };

  // DEPTH register sets of staged loads: stage it + DEPTH is issued while
  // stage it is multiplied
  u32x4 sa[DEPTH][4], sb[DEPTH][4];
  uint32_t svalid[DEPTH];
  auto load_stage = [&](int it, u32x4 (&da)[4], u32x4 (&db)[4], uint32_t &dv) {
#pragma unroll
    for (int i = 0; i < 4; ++i) da[i] = ld16(ap[i] + it * kWdK);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = UNION ? rows[i] : k0 + it * kWdK + 4 * rg + i;
      db[i] = ld16_nt(bcol + (size_t)row * H);
    }
    dv = rvalid;
  };
  auto store_stage = [&](int buf, const u32x4 (&ra)[4], const u32x4 (&rb)[4], uint32_t vv) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<u32x4 *>(&as[buf][(arow + 32 * i) * kWdRowB + achunk * 16]) = ra[i];
#pragma unroll
    for (int c = 0; c < 8; ++c) {  // column 8 cg + c gets rows 4 rg .. 4 rg + 3 (one 8-byte k-run)
      const int j = c >> 1;
      uint32_t v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint32_t w = rb[i][j];
        v[i] = (c & 1) ? (w >> 16) : (w & 0xffffu);
        if (UNION) v[i] = (vv >> i) & 1u ? v[i] : 0u;
      }
      const int col = 8 * cg + c;
      const int off = col * kWdRowB + ((((rg >> 1) ^ ((col >> 4) & 7))) << 4) + (rg & 1) * 8;
      uint2 o;
      o.x = v[0] | (v[1] << 16);
      o.y = v[2] | (v[3] << 16);
      *reinterpret_cast<uint2 *>(&bs[buf][off]) = o;
    }
  };

  const int r = lane & 15, g = lane >> 4;
  const int wt = wid >> 1, wc = wid & 1;
  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0, 0, 0, 0};

  if (nit > 0) {
    if (UNION) {
      fetch_rows(0);
      take_rows(0);
      fetch_rows(min(1, nit - 1));
    }
    load_stage(0, sa[0], sb[0], svalid[0]);
    if (DEPTH == 2 && nit > 1) {
      if (UNION) {
        take_rows(1);
        fetch_rows(min(2, nit - 1));
      }
      load_stage(1, sa[DEPTH - 1], sb[DEPTH - 1], svalid[DEPTH - 1]);
    }
    store_stage(0, sa[0], sb[0], svalid[0]);
  }
  __syncthreads();
  // One step: stage it + DEPTH into register set SL = it % DEPTH (whose
  // stage is already in LDS), multiply stage it, write stage it + 1 from
  // its register set to the other buffer.  STEADY: all of it in range, no
  // branch around a load.
  auto step = [&](int it, auto slc, auto steadyc) {
    constexpr int SL = decltype(slc)::value;
    constexpr bool STEADY = decltype(steadyc)::value;
    const int cur = it & 1;
    const int ahead = it + DEPTH;
    if (STEADY || ahead < nit) {
      if (UNION) {
        take_rows(ahead);
        fetch_rows(min(ahead + 1, nit - 1));
      }
      load_stage(ahead, sa[SL], sb[SL], svalid[SL]);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      u32x4 b[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int col = 64 * wc + 16 * j + r;
        b[j] = *reinterpret_cast<const u32x4 *>(
            &bs[cur][col * kWdRowB + (((4 * ks + g) ^ ((col >> 4) & 7)) << 4)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (4 * wt + i < ntiles) {  // wave-uniform
          const u32x4 a = *reinterpret_cast<const u32x4 *>(
              &as[cur][((4 * wt + i) * 16 + r) * kWdRowB + ks * 64 + g * 16]);
#pragma unroll
          for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(a, b[j], acc[i][j]);
        }
      }
    }
    if (STEADY || it + 1 < nit) {
      constexpr int NX = (SL + 1) % DEPTH;
      store_stage(cur ^ 1, sa[NX], sb[NX], svalid[NX]);
    }
    __syncthreads();
  };
  int it = 0;
  for (; it + DEPTH + 1 < nit; it += DEPTH) {
    step(it, SkIc<0>{}, SkIc<1>{});
    if (DEPTH == 2) step(it + 1, SkIc<1 % DEPTH>{}, SkIc<1>{});
  }
  for (; it < nit; it += DEPTH) {
    step(it, SkIc<0>{}, SkIc<0>{});
    if (DEPTH == 2 && it + 1 < nit) step(it + 1, SkIc<1 % DEPTH>{}, SkIc<0>{});
  }

  // D: lane holds column r of each column tile, token rows 4 g + rr of each
  // token tile; the rows' pair ids are all read before the first store
  int prow[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int c = (4 * wt + i) * 16 + 4 * g + rr;
      prow[i][rr] = rv.pair_at(q0 + (c < ntok ? c : 0));
    }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (4 * wt + i >= ntiles) continue;
#pragma unroll
    for (int rr = 0; rr < 4; ++rr) {
      const int c = (4 * wt + i) * 16 + 4 * g + rr;
      if (c < ntok) {
        const size_t row = (size_t)prow[i][rr] * S + sidx;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int col = col0 + 64 * wc + 16 * j + r;
          if (col < H) partial[row * H + col] = acc[i][j][rr];
        }
      }
    }
  }
}

// K chunks of the wide down GEMM: enough for ~1024 blocks, each chunk >= 256
// rows, and P * chunks within dense_down_partial_rows.
static int wide_splits(int T, int E, int top_k, int implicit, int H, int d_ff) {
  const long P = (long)T * top_k;
  const long items = implicit ? (long)E * ((T + kWdTok - 1) / kWdTok)
                              : (E < P ? E : P) + P / kWdTok;
  const long base = items * ((H + kWdCols - 1) / kWdCols);
  long S = (1024 + base - 1) / base;
  const long smax = d_ff / 256 > 0 ? d_ff / 256 : 1;
  if (S > smax) S = smax;
  const long bound = P > 0 ? (long)(dense_down_partial_rows(T, E, top_k, H) / P) : 1;
  if (S > bound) S = bound;
  return S < 1 ? 1 : (int)S;
}

// Partial rows the down GEMMs may write for at most T tokens (P pairs).
// Wide: chunks = ceil(1024 / base), base = items * cb (cb = ceil(H / 128)
// column blocks) with items >= max(1, P / 128), so P * chunks <= P + 1024 *
// min(P, 128) / cb.  Skinny: chunks = ceil(2048 / base), base = items * cs
// (cs = ceil(H / 256)) with items >= max(1, P / 64), and at most
// max(4, 1024 / P) chunks, so P * chunks <= min(max(4 P, 1024), P + 2048 *
// min(P, 64) / cs).  Each grows with T, so a workspace sized for T serves
// any shorter call.
size_t dense_down_partial_rows(int T, int E, int top_k, int H) {
  (void)E;
  const size_t P = (size_t)T * top_k;
  if (P == 0) return 0;
  const size_t cb = ((size_t)H + kWdCols - 1) / kWdCols;
  const size_t wide = P + (1024 * (P < kWdTok ? P : (size_t)kWdTok) + cb - 1) / cb;
  const size_t cs = ((size_t)H + kSkCols - 1) / kSkCols;
  const size_t sk_a = 4 * P > 1024 ? 4 * P : 1024;
  const size_t sk_b = P + (2048 * (P < 64 ? P : (size_t)64) + cs - 1) / cs;
  const size_t skinny = sk_a < sk_b ? sk_a : sk_b;
  return wide > skinny ? wide : skinny;
}

// ---------------------------------------------------------------- union of kept rows
// The sparse path's packed-rows form, for experts that hold several tokens
// (the page's fused projection gathers the active neurons' down weights
// once into a dense matrix and runs a dense product over them).  Two short
// launches build, from the mask kernel's kept lists:
//   union_bits   slot s (expert e), group g of 8 of its pairs: the OR of
//                their kept ids as a d_ff-bit map, pbits[e, g] (only where
//                experts hold over 8 tokens on average)
//   union_coef   pair p (expert e): the OR of e's group maps (or of all its
//                pairs' kept ids) and its prefix
//                counts per 32-bit word; e's first pair writes the
//                ascending union urow[e, 0 .. ucnt[e]); every pair writes
//                its coefficients (w * h at its kept ids, fp32) at their
//                union positions (prefix + popcount within the word),
//                rounded to bf16, as hmu[p, 0 .. upad) with zeros elsewhere
//                (upad = the union count rounded up to 64)
// for the gathering down GEMM.
constexpr int kUnionMaxDff = 8192;
constexpr int kUnionGroup = 8;  // pairs per union_bits block

__global__ __launch_bounds__(256) void union_bits_kernel(const int32_t *__restrict__ idx, int k,
                                                         RouteView rv, int d_ff, int G,
                                                         uint32_t *__restrict__ pbits) {
  __shared__ uint32_t bits[kUnionMaxDff / 32];
  const int tid = threadIdx.x;
  const int s = blockIdx.x, g = blockIdx.y;
  if (s >= rv.nact()) return;  // block-uniform
  const int e = rv.expert(s);
  const int q0 = rv.begin(e), np = rv.end(e) - q0;
  if (g * kUnionGroup >= np) return;
  const int ng = min(kUnionGroup, np - g * kUnionGroup);
  const int nw = d_ff / 32;
  for (int w = tid; w < nw; w += 256) bits[w] = 0u;
  __syncthreads();
  // pair pi's ids are read by the threads of sub-group pi % 8 (32 threads
  // each), 4 loads in flight per thread before their LDS updates
  const int sg = tid >> 5, st = tid & 31;
  if (sg < ng) {
    const int32_t *ip = idx + (size_t)rv.pair_at(q0 + g * kUnionGroup + sg) * k;
    for (int i0 = st; i0 < k; i0 += 128) {
      int v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = i0 + 32 * u < k ? ip[i0 + 32 * u] : -1;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        if ((unsigned)v[u] < (unsigned)d_ff) atomicOr(&bits[v[u] >> 5], 1u << (v[u] & 31));
    }
  }
  __syncthreads();
  uint32_t *o = pbits + ((size_t)e * G + g) * nw;
  for (int w = tid; w < nw; w += 256) o[w] = bits[w];
}

__global__ __launch_bounds__(256) void union_coef_kernel(const int32_t *__restrict__ idx,
                                                         const float *__restrict__ hact, int k,
                                                         RouteView rv, int d_ff, int G,
                                                         const uint32_t *__restrict__ pbits,
                                                         int32_t *__restrict__ urow,
                                                         int32_t *__restrict__ ucnt,
                                                         uint16_t *__restrict__ hmu) {
  __shared__ uint32_t bits[kUnionMaxDff / 32];
  __shared__ int pre[kUnionMaxDff / 32];
  __shared__ int wtot[4];
  __shared__ __attribute__((aligned(16))) uint16_t crow[kUnionMaxDff];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int p = blockIdx.x;
  const int e = rv.expert_of_pair(p);
  const int q0 = rv.begin(e), np = rv.end(e) - q0;
  const bool first = rv.pair_at(q0) == p;
  // the expert's map (thread w owns word w, nw <= 256): the OR of its
  // groups' maps (8 loads in flight), or, without union_bits (G == 0), of
  // its pairs' kept ids straight from the lists
  const int nw = d_ff / 32;
  uint32_t wb = 0u;
  if (G > 0) {
    const int ngr = (np + kUnionGroup - 1) / kUnionGroup;
    if (tid < nw) {
      const uint32_t *pb = pbits + (size_t)e * G * nw + tid;
      for (int g0 = 0; g0 < ngr; g0 += 8) {
        uint32_t v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = g0 + u < ngr ? pb[(size_t)(g0 + u) * nw] : 0u;
#pragma unroll
        for (int u = 0; u < 8; ++u) wb |= v[u];
      }
    }
  } else {
    for (int w = tid; w < nw; w += 256) bits[w] = 0u;
    __syncthreads();
    // pair pi's ids are read by the threads of sub-group pi % 8 (32 each)
    const int sg = tid >> 5, st = tid & 31;
    for (int pi = sg; pi < np; pi += 8) {
      const int32_t *ip = idx + (size_t)rv.pair_at(q0 + pi) * k;
      for (int i0 = st; i0 < k; i0 += 128) {
        int v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = i0 + 32 * u < k ? ip[i0 + 32 * u] : -1;
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if ((unsigned)v[u] < (unsigned)d_ff) atomicOr(&bits[v[u] >> 5], 1u << (v[u] & 31));
      }
    }
    __syncthreads();
    if (tid < nw) wb = bits[tid];
    __syncthreads();  // bits is rewritten below
  }
  const int c = __popc(wb);
  const int incl = wave_incl_scan(c);
  if (lane == 63) wtot[wid] = incl;
  __syncthreads();
  int base = incl - c;
  for (int ww = 0; ww < wid; ++ww) base += wtot[ww];
  const int uc = wtot[0] + wtot[1] + wtot[2] + wtot[3];
  if (tid < nw) {
    bits[tid] = wb;
    pre[tid] = base;
  }
  if (first) {  // the expert's first pair writes its union list
    int32_t *ur = urow + (size_t)e * d_ff;
    uint32_t m = wb;
    int o = base;
    while (m) {
      const int b = __ffs(m) - 1;
      m &= m - 1;
      ur[o++] = tid * 32 + b;
    }
    if (tid == 0) ucnt[e] = uc;
  }
  const int upad = (uc + kWdK - 1) / kWdK * kWdK;
  for (int q = tid; q < upad; q += 256) crow[q] = 0;
  __syncthreads();
  for (int i = tid; i < k; i += 256) {
    const int j = idx[(size_t)p * k + i];
    if ((unsigned)j < (unsigned)d_ff) {
      const int pos = pre[j >> 5] + __popc(bits[j >> 5] & ((1u << (j & 31)) - 1u));
      if (pos < upad) crow[pos] = (uint16_t)f32_to_bf16_bits(hact[(size_t)p * k + i]);
    }
  }
  __syncthreads();
  uint16_t *o = hmu + (size_t)p * d_ff;
  for (int q = 8 * tid; q < upad; q += 8 * 256)
    *reinterpret_cast<u32x4 *>(o + q) = *reinterpret_cast<const u32x4 *>(&crow[q]);
}

// Words of the union build's scratch (the groups' maps) for at most T
// tokens on E experts (at most E active slots).
size_t union_scratch_words(int T, int E, int d_ff) {
  const size_t G = (T + kUnionGroup - 1) / kUnionGroup;
  return (size_t)E * G * (d_ff / 32);
}

// ---------------------------------------------------------------- combine
// y[t, :] = (accumulate ? y[t, :] : 0) + sum over slots, then chunks, of
// the token's partial rows: a fixed order, so reruns are bitwise equal.
// With xnext: also x_next = x_res + y, rounded to the layer dtype (bf16
// when BF16), as the sparse path's residual epilogue.
template <bool BF16 = true>
__global__ __launch_bounds__(64) void combine_kernel(const float *__restrict__ partial, int H,
                                                      int top_k, int n_chunks, int accumulate,
                                                      float *__restrict__ y,
                                                      const void *__restrict__ xres = nullptr,
                                                      void *__restrict__ xnext = nullptr) {
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
  if (xnext) {
    const size_t o = (size_t)t * H + col;
    if (BF16) {
      const uint2 xb = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(xres) + o);
      uint2 ob;
      ob.x = f32_to_bf16_bits(bf16lo(xb.x) + s[0]) | (f32_to_bf16_bits(bf16hi(xb.x) + s[1]) << 16);
      ob.y = f32_to_bf16_bits(bf16lo(xb.y) + s[2]) | (f32_to_bf16_bits(bf16hi(xb.y) + s[3]) << 16);
      *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(xnext) + o) = ob;
    } else {
      const f32x4 xv = *reinterpret_cast<const f32x4 *>(static_cast<const float *>(xres) + o);
      *reinterpret_cast<f32x4 *>(static_cast<float *>(xnext) + o) = xv + s;
    }
  }
}

// ---------------------------------------------------------------- host side

#ifndef MOE_GEMM_DEEP
#define MOE_GEMM_DEEP 3
#endif
void launch_gateup_gemm(const FfnArgs &a, const RouteView &rv, bool gate_only, hipStream_t stream) {
  // two neuron tiles per wave for the bf16 SwiGLU contraction when d_ff
  // allows (a multiple of 128) and the grid still has >= 2 blocks per CU
  // (few items, e.g. a shared expert at T = 256, keep the narrow blocks)
  const int items = n_items(a, kGemmTok);
  const bool wide = a.bf16 && !gate_only && a.d_ff % 128 == 0 &&
                    (long)items * (a.d_ff / 128) >= 512;
  // a grid of under 2 blocks per CU keeps more weight stages in flight
  const bool deep = a.bf16 && !wide && (long)items * (a.d_ff / 64) < 512;
#ifndef MOE_GEMM_HALF_ITEMS
#define MOE_GEMM_HALF_ITEMS 1
#endif
  const bool half = MOE_GEMM_HALF_ITEMS && deep && !gate_only;
  dim3 grid(half ? n_items(a, kGemmTok / 2) : items, a.d_ff / (wide ? 128 : 64));
#define MOE_GG(BF, GOV, N, D) \
  gateup_gemm_kernel<BF, GOV, N, D><<<grid, 256, 0, stream>>>(a.x, a.w_gate, a.w_up, rv, a.H, a.d_ff, a.h)
  if (a.bf16) {
    if (gate_only) { if (deep) MOE_GG(true, true, 1, MOE_GEMM_DEEP); else MOE_GG(true, true, 1, 1); }
    else if (wide) MOE_GG(true, false, 2, 1);
    else if (half)
      gateup_gemm_kernel<true, false, 1, MOE_GEMM_DEEP, 4><<<grid, 256, 0, stream>>>(a.x, a.w_gate, a.w_up,
                                                                                  rv, a.H, a.d_ff, a.h);
    else if (deep) MOE_GG(true, false, 1, MOE_GEMM_DEEP);
    else MOE_GG(true, false, 1, 1);
  } else {
    if (gate_only) MOE_GG(false, true, 1, 1); else MOE_GG(false, false, 1, 1);
  }
#undef MOE_GG
}

bool union_form(int T, int E, int top_k, int H, int d_ff) {
  if (T <= 0 || E <= 0 || top_k <= 0) return false;
  const long P = (long)T * top_k;
  const long per_expert = P / (E < P ? E : P);  // T for a shared group (top_k == E)
  const double active = E * (1.0 - pow(1.0 - (double)top_k / E, (double)T));
  const double bytes = active * d_ff * H * 2.0;  // the active experts' W_d
  return per_expert >= union_min_tokens(bytes);
}

bool union_layout_ok(int T, int H, int d_ff, int bf16) {
  return bf16 && H % 64 == 0 && d_ff % kWdK == 0 && d_ff <= kUnionMaxDff &&
         T >= kUnionMinTokensLarge;
}

bool union_down_ok(const FfnArgs &a) {
  if (!a.hmu || !a.urow || !a.ucnt || !a.ubuf || a.k_keep <= 0) return false;
  if (!union_layout_ok(a.T, a.H, a.d_ff, a.bf16)) return false;
  return union_form(a.T, a.E, a.top_k, a.H, a.d_ff);
}

// The sparse path's packed-rows form (bf16): the union kernel, then the down
// GEMM over each expert's union of kept rows, then the combine.  a.idx and
// a.hact hold the mask kernel's kept lists; a.hmu, a.urow and a.ucnt receive
// the union.
hipError_t launch_down_union(const FfnArgs &a, const RouteView &rv, hipStream_t stream) {
  const int P = a.T * a.top_k;
  const int slots = a.implicit ? a.E : (a.E < P ? a.E : P);
  const int G = (a.T + kUnionGroup - 1) / kUnionGroup;
  uint32_t *pbits = a.ubuf;
  timer_begin(kStageUnionRows, stream);
  // experts of a few tokens: each pair's block ORs its expert's lists itself
  // (one launch; measured 11.3 -> 7.9 us at 8 tokens per expert, but 35 ->
  // 40 us at 16); past 8 tokens per expert on average, per-group maps first
  const long per_expert = a.implicit ? a.T : P / slots;
  const int Gl = per_expert > 8 ? G : 0;
  if (Gl > 0)
    union_bits_kernel<<<dim3(slots, G), 256, 0, stream>>>(a.idx, a.k_keep, rv, a.d_ff, G, pbits);
  union_coef_kernel<<<P, 256, 0, stream>>>(a.idx, a.hact, a.k_keep, rv, a.d_ff, Gl, pbits, a.urow,
                                           a.ucnt, a.hmu);
  timer_end(stream);
  const int mt = skinny_tiles(a.T, a.E, a.top_k, a.implicit);
  int S;
  timer_begin(kStageDownUnion, stream);
  if (mt > 0) {
    S = skinny_splits(a.T, a.E, a.top_k, a.implicit, a.H, a.d_ff, mt);
    if ((size_t)P * S > dense_down_partial_rows(a.T, a.E, a.top_k, a.H)) return hipErrorInvalidValue;
    dim3 grid(n_items(a, 16 * mt), (a.H + kSkCols - 1) / kSkCols, S);
    const uint16_t *wd = static_cast<const uint16_t *>(a.w_down);
    if (mt == 2)
      down_skinny_kernel<2, true, sk_depth<2, true>()><<<grid, 256, 0, stream>>>(wd, a.hmu, rv, a.H, a.d_ff, 0, a.partial,
                                                            a.urow, a.ucnt);
    else
      down_skinny_kernel<4, true, sk_depth<4, true>()><<<grid, 256, 0, stream>>>(wd, a.hmu, rv, a.H, a.d_ff, 0, a.partial,
                                                            a.urow, a.ucnt);
  } else {
    S = wide_splits(a.T, a.E, a.top_k, a.implicit, a.H, a.d_ff);
    if ((size_t)P * S > dense_down_partial_rows(a.T, a.E, a.top_k, a.H)) return hipErrorInvalidValue;
    dim3 grid(n_items(a, kWdTok), (a.H + kWdCols - 1) / kWdCols, S);
    down_wide_kernel<true, kWdDepth><<<grid, 256, 0, stream>>>(
        static_cast<const uint16_t *>(a.w_down), a.hmu, rv, a.H, a.d_ff, 0, a.partial, a.urow, a.ucnt);
  }
  timer_end(stream);
  dim3 cgrid(a.T, (a.H + 255) / 256);
  timer_begin(kStageCombine, stream);
  combine_kernel<true><<<cgrid, 64, 0, stream>>>(a.partial, a.H, a.top_k, S, a.accumulate, a.y,
                                                 a.xres, a.xnext);
  timer_end(stream);
  return hipGetLastError();
}

#ifndef MOE_PACKED_NTW_MAX
#define MOE_PACKED_NTW_MAX 4
#endif
// The dense down GEMM over a packed W_d.  Item size: 32, 64 or 128 tokens,
// the skinny GEMM's token tiles (routed experts: 2 or 4 tiles up to 16 or
// 40 tokens per expert on average, so the busiest expert still fits one
// item; always-on experts: T <= 32, <= 64); 64-token items at 64 tokens
// per expert split the busier experts in two and read their W_d twice (381
// us against 268 us with 128-token items on the 1024-token Llama-4-like
// routed experts).  16 * NTW columns per wave, NTW the largest of 4, 2, 1
// that divides H / 64.  K chunks S:
//  - always-on experts of 128-token items (the matrix-bound shape, item
//    counts exact): the grid runs in rounds of `slots` resident blocks (2,
//    3 or 4 per CU as NTW = 4, 2, 1 allow: registers, LDS) and each block
//    takes kc / 64 stages, so S minimises rounds x stages (the smallest
//    such S, which also writes the fewest partial rows).  A partial last
//    round costs a whole one: on the 1024-token Llama-4-like shared expert,
//    640 blocks (1.25 rounds of 32 stages) took 139.5 us, 480 blocks (one
//    round of 43 stages) 103.2 us.
//  - otherwise (streaming W_d at a few flops per byte): ~1024 blocks to keep
//    bytes in flight (~2048 for a lone always-on item of <= 64 tokens);
//    fewer lost (24 x 20 x 1 blocks: 296 us against 268 us at S = 3 on the
//    routed experts of the same layer at 1024 tokens), and so did more,
//    whose partial rows cost more than they gained (routed experts at 16
//    tokens each: 251.5 us at S = 5 against 237.1 us at S = 3).
// Chunks are >= 256 rows and a multiple of 64, P * S within
// dense_down_partial_rows.
static hipError_t launch_down_packed(const FfnArgs &a, const RouteView &rv, hipStream_t stream) {
  const int ntw = (a.H % 256 == 0 && MOE_PACKED_NTW_MAX >= 4) ? 4
                  : (a.H % 128 == 0 && MOE_PACKED_NTW_MAX >= 2) ? 2 : 1;
  const size_t P = (size_t)a.T * a.top_k;
  const int skt = skinny_tiles(a.T, a.E, a.top_k, a.implicit);
  const int mt = skt > 0 ? skt : 8;
  const int items = n_items(a, 16 * mt);
  const long base = (long)items * (a.H / (64 * ntw));
  long smax = a.d_ff / 256 > 0 ? a.d_ff / 256 : 1;
  const long bound = (long)(dense_down_partial_rows(a.T, a.E, a.top_k, a.H) / P);
  if (smax > bound) smax = bound;
  auto chunk = [&](long S) { return (int)((a.d_ff + S - 1) / S + 63) / 64 * 64; };
  int kc;
  if (a.implicit && mt == 8) {
    const long slots = 256L * (ntw == 4 ? 2 : ntw == 2 ? 3 : 4);
    long best = -1;
    kc = a.d_ff;
    for (long S = 1; S <= smax; ++S) {
      const int k = chunk(S);
      const long n = (a.d_ff + k - 1) / k;
      const long est = (base * n + slots - 1) / slots * (k / 64);
      if (best < 0 || est < best) { best = est; kc = k; }
    }
  } else {
    const long target = a.implicit && mt < 8 ? 2048 : 1024;
    long S = (target + base - 1) / base;
    if (S > smax) S = smax;
    if (S > 16) S = 16;
    kc = chunk(S < 1 ? 1 : S);
  }
  const int Sc = (a.d_ff + kc - 1) / kc;
  if (P * Sc > dense_down_partial_rows(a.T, a.E, a.top_k, a.H)) return hipErrorInvalidValue;
  const uint8_t *wdp = static_cast<const uint8_t *>(a.w_down);
  const uint16_t *hm = static_cast<const uint16_t *>(a.hm);
  dim3 grid(items, a.H / (64 * ntw), Sc);
  timer_begin(kStageDownDense, stream);
#define MOE_PK(N, M, D) \
  down_packed_kernel<N, M, D><<<grid, 256, 0, stream>>>(wdp, hm, rv, a.H, a.d_ff, kc, a.partial)
#define MOE_PKC(N) \
  down_packed_kernel<N, 8, 1, true><<<grid, 256, 0, stream>>>(wdp, hm, rv, a.H, a.d_ff, kc, a.partial)
  if (mt == 8 && a.implicit) {
    if (ntw == 4) MOE_PKC(4); else if (ntw == 2) MOE_PKC(2); else MOE_PKC(1);
  } else if (mt == 8) {
    if (ntw == 4) MOE_PK(4, 8, 1); else if (ntw == 2) MOE_PK(2, 8, 1); else MOE_PK(1, 8, 1);
  } else if (mt == 4) {
    if (ntw == 4) MOE_PK(4, 4, 2); else if (ntw == 2) MOE_PK(2, 4, 2); else MOE_PK(1, 4, 2);
  } else {
    if (ntw == 4) MOE_PK(4, 2, 2); else if (ntw == 2) MOE_PK(2, 2, 2); else MOE_PK(1, 2, 2);
  }
#undef MOE_PK
#undef MOE_PKC
  timer_end(stream);
  dim3 cgrid(a.T, (a.H + 255) / 256);
  timer_begin(kStageCombine, stream);
  combine_kernel<true><<<cgrid, 64, 0, stream>>>(a.partial, a.H, a.top_k, Sc, a.accumulate, a.y);
  timer_end(stream);
  return hipGetLastError();
}

hipError_t launch_down_dense(const FfnArgs &a, const RouteView &rv, hipStream_t stream) {
  if (a.down_packed) return launch_down_packed(a, rv, stream);
  const int mt = skinny_tiles(a.T, a.E, a.top_k, a.implicit);
  const size_t P = (size_t)a.T * a.top_k;
  const uint16_t *wd = static_cast<const uint16_t *>(a.w_down);
  const uint16_t *hm = static_cast<const uint16_t *>(a.hm);
  int S;
  timer_begin(kStageDownDense, stream);
  if (mt > 0) {  // few tokens per expert: the skinny GEMM over all d_ff rows
    S = skinny_splits(a.T, a.E, a.top_k, a.implicit, a.H, a.d_ff, mt);
    const int per = (a.d_ff + S - 1) / S;
    const int kc = (per + kSkK - 1) / kSkK * kSkK;
    if (P * S > dense_down_partial_rows(a.T, a.E, a.top_k, a.H)) return hipErrorInvalidValue;
    dim3 grid(n_items(a, 16 * mt), (a.H + kSkCols - 1) / kSkCols, S);
    if (mt == 2)
      down_skinny_kernel<2, false, sk_depth<2, false>()><<<grid, 256, 0, stream>>>(wd, hm, rv, a.H, a.d_ff, kc, a.partial,
                                                             nullptr, nullptr);
    else
      down_skinny_kernel<4, false, sk_depth<4, false>()><<<grid, 256, 0, stream>>>(wd, hm, rv, a.H, a.d_ff, kc, a.partial,
                                                             nullptr, nullptr);
  } else {  // many tokens per expert: the 128 x 128 GEMM over all d_ff rows
    S = wide_splits(a.T, a.E, a.top_k, a.implicit, a.H, a.d_ff);
    const int per = (a.d_ff + S - 1) / S;
    const int kc = (per + kWdK - 1) / kWdK * kWdK;
    S = (a.d_ff + kc - 1) / kc;
    if (P * S > dense_down_partial_rows(a.T, a.E, a.top_k, a.H)) return hipErrorInvalidValue;
    dim3 grid(n_items(a, kWdTok), (a.H + kWdCols - 1) / kWdCols, S);
    down_wide_kernel<false, kWdDepth><<<grid, 256, 0, stream>>>(wd, hm, rv, a.H, a.d_ff, kc,
                                                                a.partial, nullptr, nullptr);
  }
  timer_end(stream);
  dim3 cgrid(a.T, (a.H + 255) / 256);
  timer_begin(kStageCombine, stream);
  combine_kernel<true><<<cgrid, 64, 0, stream>>>(a.partial, a.H, a.top_k, S, a.accumulate, a.y);
  timer_end(stream);
  return hipGetLastError();
}

}  // namespace moe
