// Expert FFN kernels of the intra-expert-sparse MoE layer (gfx950).
//
//   gateup_swiglu   h = silu(W_g x) * (W_u x), dense, MFMA, per active-expert
//                   slot (T <= 16) or per expert and 16 of its tokens (T <= 64);
//                   past that the grouped GEMM of dense.hip
//   neuron_topk     exact top-k of |h| per pair (radix select + one threshold pass),
//                   compacted ascending kept-neuron list, weights folded in
//   down_token      y_t = sum over the token's pairs and kept rows j of
//                   hact_j * W_d[j, :], streaming only those rows (the sparse
//                   down projection, with the combine in a fixed order)
//   up_rows         the split's sparse up projection: u_j = W_u[j] . x for
//                   kept j only (gate-only scores from gateup_swiglu)
//   neuron_threshold / down_var_token / down_thr_token
//                   threshold masking (a kept count per pair) and the down
//                   projection over variable-length lists; calibrate_kernel
//                   sets the per-expert thresholds offline
//
// Method: the page "Uncovering Intra-expert Activation Sparsity for
// Efficient Mixture-of-Expert Model Execution", technical summary,
// Methodology (vLLM implementation): gate projection run densely for the
// activation scores; activation masking in one O(n) threshold pass; a
// sparse projection that gathers only the active neurons' weights; a
// batch-size switch to the dense path.
#include <cmath>

#include "ffn_common.h"
#include "route_common.h"

namespace moe {

// ---------------------------------------------------------------- sparse down rows
// The down kernels share one inner loop: a block of NWV (kDownWaves) waves
// streams n staged rows (srow[q] = expert * d_ff + row, scoef[q] its
// coefficient, both in LDS) of W_d, each row contributing one SW-element run
// at column colo.  Wave wid takes row groups wid, wid + kDownWaves, ...
// (RPI rows per group, one per LPR-lane slice) and issues U groups' 16-byte
// loads before folding any of them into acc, so a lane has up to U loads in
// flight.  U = 4: deeper rounds (8) measured no faster at decode batches
// and raise the kernels to ~78 VGPRs, which halves the blocks a CU holds
// at large batches (Llama-4-like T = 256 sparse: 1082 -> 1156 us).
constexpr int kDownWaves = 16;
constexpr int kDownStage = 4096;     // row-list entries staged in LDS

// The residual stream's element o of the next layer's input: x_res + y
// summed in fp32, rounded to the layer dtype (as residual_kernel does).
template <bool BF16>
__device__ __forceinline__ void residual_store(const void *xres, void *xnext, size_t o, float y) {
  if (BF16) {
    const uint32_t xb = static_cast<const uint16_t *>(xres)[o];
    static_cast<uint16_t *>(xnext)[o] = (uint16_t)f32_to_bf16_bits(bf16lo(xb) + y);
  } else {
    static_cast<float *>(xnext)[o] = static_cast<const float *>(xres)[o] + y;
  }
}

template <bool BF16, int SW, int U, int NWV = kDownWaves>
__device__ __forceinline__ void stream_rows_u(const void *__restrict__ wdv,
                                              const uint32_t *srow, const float *scoef, int n,
                                              int H, size_t colo, int wid, int rsel,
                                              float (&acc)[BF16 ? 8 : 4]) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int RPI = 64 / (SW / VEC);
  for (int b0 = wid; b0 * RPI < n; b0 += NWV * U) {
    u32x4 qv[U];
    float cf[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int qq = (b0 + NWV * u) * RPI + rsel;
      cf[u] = 0.f;
      qv[u] = u32x4{0, 0, 0, 0};
      if (qq < n) {
        const size_t off = (size_t)srow[qq] * H + colo;
        cf[u] = scoef[qq];
        qv[u] = BF16 ? ld16(static_cast<const uint16_t *>(wdv) + off)
                     : ld16(static_cast<const float *>(wdv) + off);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (BF16) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          acc[2 * jj] = fmaf(cf[u], bf16lo(qv[u][jj]), acc[2 * jj]);
          acc[2 * jj + 1] = fmaf(cf[u], bf16hi(qv[u][jj]), acc[2 * jj + 1]);
        }
      } else {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) acc[jj] = fmaf(cf[u], __uint_as_float(qv[u][jj]), acc[jj]);
      }
    }
  }
}

template <bool BF16, int SW>
__device__ __forceinline__ void stream_rows(const void *__restrict__ wdv, const uint32_t *srow,
                                            const float *scoef, int n, int H, size_t colo,
                                            int wid, int rsel, float (&acc)[BF16 ? 8 : 4]) {
  stream_rows_u<BF16, SW, 4>(wdv, srow, scoef, n, H, colo, wid, rsel, acc);
}

struct LayerSel {
  const float *part;       // [nsplit, T, E] logit partials
  int nsplit, norm_topk;
  const float *bias;       // [E] or null
};

// Position of the n-th (0-based) set bit of w; w has more than n set bits.
__device__ __forceinline__ int nth_set_bit(uint64_t w, int n) {
  for (int i = 0; i < n; ++i) w &= w - 1;
  return __ffsll((unsigned long long)w) - 1;
}

// ---------------------------------------------------------------- fused layer tail
// The single-launch sparse FFN of decode batches (T <= 16): the gate/up
// kernel's grid gets extra rows of "down units" (launch_ffn_fused), and the
// two kinds of block meet through device-coherent memory instead of a
// kernel boundary:
//
//   gate/up block (slot s, neuron tile)  writes its h tile with agent-scope
//       stores, waits for them, then adds one to cnt_e[e] (e = the slot's
//       expert); d_ff / 16 arrivals mean the expert's h is complete;
//   down unit (pair p, column block c)   finds p's expert e, waits (bounded)
//       for cnt_e[e] == d_ff / 16, selects the pair's k largest |h| with one
//       wave (the exact radix select of the mask kernels), stages those rows
//       in LDS, streams SW columns of each kept W_d row, and writes the
//       weighted partial sum part[p, cols]; it then adds one to
//       cnt_tc[t, c], and the unit that completes the token's top_k pairs
//       sums their partials in slot order into y[t, cols] (+ the residual).
//
// Every wait is on blocks with lower linear ids (the first n_active grid
// rows are the gate/up blocks of the active slots, the down units follow
// directly), and each XCD dispatches its blocks in id order, so every waited
// tile is dispatched ahead of its waiters and never waits itself: no
// deadlock at any occupancy.  Waits are bounded anyway (wait_count).  The
// counters are zeroed by the kernel before this launch on the same stream.
// Down units run in pair order (routing from an earlier kernel: grouped by
// expert, so the earliest experts' rows stream while later experts' gate/up
// tiles still run; selection inside gate/up (VSEL): token-major).
struct FusedArgs {
  int gu_rows;           // grid rows for gate/up blocks, min(E, P); the first
                         // n_active of them run gate/up, the rest down units
  int ncb;               // column blocks per pair (H / SW)
  int npairs;            // T * top_k
  int k;                 // kept neurons per pair (0 < k < d_ff, k <= kFusedMaxK)
  const void *wd;        // W_d [E, d_ff, H]
  float *part;           // [P, H] per-pair partial outputs (agent-coherent)
  int32_t *cnt_e;        // [E * kCounterStride] finished gate/up tiles per expert
  int32_t *cnt_tc;       // [T * ncb] finished pairs per (token, column block)
  int32_t *abort_flag;   // [1] set when a bounded wait gives up
  float *y;
  int accumulate;
  const void *xres;
  void *xnext;
  int32_t *idx_out;      // optional kept ids [P, k]
};
constexpr int kFusedMaxK = 1024;

// Pass 0 of the one-wave exact select (the exponent digit, bits 30..23 of
// |h|) from registers instead of the LDS histogram: each lane counts its
// keys in the eight binades at and below the wave's largest exponent in
// packed 8-bit fields (at most V <= 32 per field), the wave adds them as
// 16-bit fields with DPP, and the digit of the krem-th largest key follows
// from the eight totals, as the histogram pass would find it.  Returns
// false, with nothing written, when that key lies below those binades; the
// histogram pass then runs.  (The histogram pass's LDS atomics cost ~1.3 us
// per pass with eight selecting waves per block, in a stand-alone timing
// copy, much the same however few lanes are active.)
template <int V>
__device__ __forceinline__ bool exp_digit_regs(const uint32_t (&bits)[V], int krem, uint32_t &tau,
                                               uint32_t &pmask, int &krem_out, bool &whole) {
  static_assert(V <= 32, "per-lane counts must fit 8 bits");
  uint32_t emax = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) emax = max(emax, (bits[i] & 0x7fffffffu) >> 23);
  emax = wave_max_u32(emax);
  uint32_t a = 0, b = 0;  // binades emax - 0 .. 3 and emax - 4 .. 7, a byte each
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const uint32_t d = emax - ((bits[i] & 0x7fffffffu) >> 23);  // >= 0
    const uint32_t one = 1u << (8 * (d & 3u));
    a += d < 4u ? one : 0u;
    b += d - 4u < 4u ? one : 0u;  // d in 4 .. 7
  }
  const uint32_t w[4] = {(a & 0xffu) | ((a & 0xff00u) << 8), ((a >> 16) & 0xffu) | ((a >> 8) & 0xff0000u),
                         (b & 0xffu) | ((b & 0xff00u) << 8), ((b >> 16) & 0xffu) | ((b >> 8) & 0xff0000u)};
  int run = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t tot = (uint32_t)lane_value(wave_incl_scan((int)w[q]), 63);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = (int)((tot >> (16 * h)) & 0xffffu);
      if (run + c >= krem) {  // wave-uniform; run < krem here
        tau = (emax - (uint32_t)(2 * q + h)) << 23;
        pmask = 0xffu << 23;
        krem_out = krem - run;
        whole = c == krem_out && tau != 0u;
        return true;
      }
      run += c;
    }
  }
  return false;
}

// The kept list of one lane's V activations (the exact select's tau, krem
// and the lane's position and equal-key count before it), written to LDS at
// base + position without a branch per value: every value is stored, a
// dropped one (or one past k, which finite input never produces) to the
// lane's spare slot.  The
// per-value branches this replaces cost about 1 us per select (timing of
// the d_ff = 1024 and 8192 selects, 1.9 -> 0.8 us).
template <int V>
__device__ __forceinline__ void keep_list_lds(const uint32_t (&bits)[V], uint32_t tau, int krem,
                                              int eq_seen, int pos, int k, int seg, uint32_t rbase,
                                              float w, uint32_t *srow, float *scoef, int base,
                                              int spare) {
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const uint32_t key = bits[i] & 0x7fffffffu;
    const int eq = key == tau ? 1 : 0;
    const bool keep = key > tau || (eq != 0 && eq_seen < krem);
    eq_seen += eq;
    const int slot = keep && pos < k ? base + pos : spare;
    srow[slot] = rbase + (uint32_t)(seg + i);
    scoef[slot] = w * __uint_as_float(bits[i]);
    pos += keep ? 1 : 0;
  }
}

template <bool BF16, int SW, int V, int NWV>
__device__ __forceinline__ void fused_down_unit(const FusedArgs &fa, const RouteView &rv,
                                                const float *h, int H, int d_ff, int unit) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int LPR = SW / VEC;
  static_assert(LPR <= 64 && 64 % LPR == 0, "a row run must fit one wave");
  static_assert(V <= 16, "up to 16 activations per lane (d_ff <= 1024)");
  __shared__ uint32_t srow[kFusedMaxK + 64];  // + one spare slot per lane
  __shared__ float scoef[kFusedMaxK + 64];
  __shared__ int hist[256];
  __shared__ float red[NWV][SW];
  __shared__ int s_ok, s_last;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  if (unit >= fa.npairs * fa.ncb) return;  // block-uniform
  const int q = unit / fa.ncb, c = unit - q * fa.ncb;
  const int K = rv.top_k, k = fa.k;
  const int col0 = c * SW;
  if (wid == 0) {
    // the pair (routing from an earlier kernel, pairs grouped by expert), its
    // expert and routing weight
    int p = rv.pair_at(q);
    p = (unsigned)p < (unsigned)fa.npairs ? p : 0;  // a corrupt routing stays in bounds
    int e = rv.expert_of_pair(p);
    e = (unsigned)e < (unsigned)rv.E ? e : 0;
    const float w = rv.weight(p);
    bool ok = true;
    if (lane == 0) ok = wait_count(fa.cnt_e + (size_t)e * kCounterStride, d_ff / 16, fa.abort_flag);
    ok = __shfl(ok ? 1 : 0, 0, 64) != 0;
    compiler_barrier();
    if (lane == 0) s_ok = ok ? p : -1;
    if (ok) {
      // the pair's activations, read coherently: lane holds V consecutive
      const __amdgpu_buffer_rsrc_t rh = buf_rsrc(h + (size_t)p * d_ff, (uint32_t)d_ff * 4);
      uint32_t bits[V];
#pragma unroll
      for (int i = 0; i < V; i += 4) {
        const u32x4 qv = buf_ld16_agent(rh, (uint32_t)lane * V * 4, (uint32_t)i * 4);
        bits[i] = qv[0]; bits[i + 1] = qv[1]; bits[i + 2] = qv[2]; bits[i + 3] = qv[3];
      }
      // exact k-th |h| by MSB-first radix passes over the float fields
      uint32_t tau = 0, pmask = 0;
      int krem = k;
      bool whole = false;
      const bool p0 = exp_digit_regs<V>(bits, k, tau, pmask, krem, whole);
#pragma unroll
      for (int pass = 0; pass < 4; ++pass) {
        if (whole || (pass == 0 && p0)) continue;  // wave-uniform
        const int shift = pass == 0 ? 23 : pass == 1 ? 15 : pass == 2 ? 7 : 0;
        const uint32_t dmask = pass == 3 ? 0x7fu : 0xffu;
#pragma unroll
        for (int b = 0; b < 4; ++b) hist[lane * 4 + b] = 0;
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const uint32_t key = bits[i] & 0x7fffffffu;
          if ((key & pmask) == tau) atomicAdd(&hist[(key >> shift) & dmask], 1);
        }
        int cb[4], local = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          cb[b] = hist[255 - 4 * lane - b];
          local += cb[b];
        }
        int run = wave_incl_scan(local) - local;
        int dsel = -1, knew = 0, csel = 0;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          if (dsel < 0 && run + cb[b] >= krem && run < krem) {
            dsel = 255 - 4 * lane - b;
            knew = krem - run;
            csel = cb[b];
          }
          run += cb[b];
        }
        const uint64_t m = __ballot(dsel >= 0);
        const int L = __ffsll((unsigned long long)m) - 1;  // exactly one lane
        dsel = lane_value(dsel, L);
        knew = lane_value(knew, L);
        csel = lane_value(csel, L);
        tau |= (uint32_t)dsel << shift;
        pmask |= dmask << shift;
        krem = knew;
        whole = csel == knew && tau != 0u;
      }
      if (whole) {  // keep key >= tau: key > tau - 1, no equal ones
        tau -= 1u;
        krem = 0;
      }
      int ngt = 0, neq = 0;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const uint32_t key = bits[i] & 0x7fffffffu;
        ngt += key > tau;
        neq += key == tau;
      }
      const int eq_before = wave_incl_scan(neq) - neq;
      int pos = wave_incl_scan(ngt) - ngt + min(eq_before, krem);
      int eq_seen = eq_before;
      const uint32_t rbase = (uint32_t)e * (uint32_t)d_ff;
      int32_t *io = (fa.idx_out && c == 0) ? fa.idx_out + (size_t)p * k : nullptr;
      const int seg = lane * V;
      if (io) {
#pragma unroll
        for (int i = 0; i < V; ++i) {
          const uint32_t key = bits[i] & 0x7fffffffu;
          const bool keep = key > tau || (key == tau && eq_seen++ < krem);
          if (keep) {
            if (pos < k) {  // always: exactly k keys are kept
              srow[pos] = rbase + (uint32_t)(seg + i);
              scoef[pos] = w * __uint_as_float(bits[i]);
              if (io) io[pos] = seg + i;
            }
            ++pos;
          }
        }
      } else {
        keep_list_lds(bits, tau, krem, eq_seen, pos, k, seg, rbase, w, srow, scoef, 0,
                      kFusedMaxK + lane);
      }
    }
  }
  __syncthreads();
  const int p = s_ok;
  if (p < 0) return;  // block-uniform: a bounded wait gave up
  const int sub = lane % LPR, rsel = lane / LPR;
  const size_t colo = (size_t)col0 + sub * VEC;
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
  stream_rows_u<BF16, SW, 4, NWV>(fa.wd, srow, scoef, k, H, colo, wid, rsel, acc);
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] += __shfl_xor(acc[v], o, 64);
  }
  if (rsel == 0) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) red[wid][sub * VEC + v] = acc[v];
  }
  __syncthreads();
  const int t = p / K;
  if (tid < SW) {
    float v = 0.f;
#pragma unroll
    for (int ww = 0; ww < NWV; ++ww) v += red[ww][tid];
    st_agent(fa.part + (size_t)p * H + col0 + tid, v);
    wait_stores();
  }
  __syncthreads();
  if (tid == 0) s_last = atomicAdd(fa.cnt_tc + (size_t)t * fa.ncb + c, 1) == K - 1;
  __syncthreads();
  if (!s_last) return;  // block-uniform
  // the token's last pair for these columns: its top_k partials in slot order
  compiler_barrier();
  if (tid < SW) {
    const size_t col = (size_t)col0 + tid;
    float pv[16];  // top_k <= 16: every load in flight, then summed in slot order
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2)
      pv[s2] = s2 < K ? ld_agent(fa.part + ((size_t)t * K + s2) * H + col) : 0.f;
    float v = 0.f;
#pragma unroll
    for (int s2 = 0; s2 < 16; ++s2)
      if (s2 < K) v += pv[s2];
    const size_t o = (size_t)t * H + col;
    const float out = fa.accumulate ? fa.y[o] + v : v;
    fa.y[o] = out;
    if (fa.xnext) residual_store<BF16>(fa.xres, fa.xnext, o, out);
  }
}

// ---------------------------------------------------------------- gate / up
// Block = one work item (an expert and up to 16 * MT of its tokens) x 16
// neurons; W waves split K (H) by interleaved steps so that at any moment
// the block reads contiguous runs of each weight row.  Each wave keeps
// 16x16 MFMA accumulators for gate and up for MT token tiles; weights are
// loaded once, token rows (16 B per lane) come from L2.  The wave partials
// meet in LDS, where h = silu(g) * u is formed and written per pair.
// Grid: x = neuron tile, y = item.  Blocks dispatch x-fastest, so every
// tile of the occupied items starts first and the grid's unoccupied item
// slots (sized from shapes, not from the routing) trail behind them.
// The weight stream depends only on the item's expert, so a wave issues
// its first round of weight loads before it resolves the item's tokens
// (expert offsets, then the pair list): those dependent lookups overlap
// the first HBM round trip instead of preceding it.
// PF (single-token calls, where an item holds one token and 15 of 16
// tile lanes are padding): loads go through buffer resources -- a
// wave-uniform base and range, one shared per-lane offset register and a
// scalar offset per k-step -- which frees the registers to fetch a round's
// token fragments together with its weights (one wait per round, where the
// plain form waits on each fragment's L2 round trip in turn).  Padding
// lanes then read the item's first token (in range; their MFMA columns are
// never stored).  Measured per layer call (OLMoE-like): 36.4 -> 35.6 us at
// one token; the plain form stays 1 us faster at two tokens and 0.5 us at
// 4 and 16.
// VSEL > 0 (calls of T <= W tokens): the block selects its own expert.
// Wave t < T runs the router's top-k selection for token t on the logit
// partials (V = VSEL logits per lane, the router's own device function, so
// the same bits); the picks meet in LDS as per-token lists, a bitmask of
// the picked experts and per-expert counts.  Block slot s takes the s-th
// smallest picked expert id and its tokens in ascending order; block
// (0, 0) writes the routing outputs (ids and weights in slot order, the
// grouping sorted by (expert, pair)).  The routing arrays in rv are then
// written, not read, by this kernel.
// FU (the fused tail above, FSW output columns per down unit, FV = d_ff / 64
// activations per lane in its select): grid rows past the active-expert
// count are down units; the gate/up blocks write h coherently and count
// their tiles.
template <bool BF16, int MT, int W, bool GO = false, bool PF = false, int VSEL = 0, bool FU = false,
          int FSW = 64, int FV = 16>
__global__ __launch_bounds__(64 * W, MT == 1 ? 8 : 1) void gateup_swiglu_kernel(const void *__restrict__ xv,
                                                            const void *__restrict__ wgv,
                                                            const void *__restrict__ wuv,
                                                            RouteView rv, int H, int d_ff,
                                                            float *__restrict__ hout,
                                                            LayerSel sel = LayerSel{},
                                                            FusedArgs fa = FusedArgs{}) {
  static_assert(VSEL == 0 || (MT == 1 && !GO), "selection runs in the one-tile form");
  static_assert(!FU || (MT == 1 && !GO && VSEL == 0), "the fused tail follows the one-tile SwiGLU form");
  if constexpr (FU) {
    // rows below the active-expert count are gate/up blocks, the rows after
    // them down units (no row of inactive slots between the two)
    const int nrows = min(rv.nact(), fa.gu_rows);
    if ((int)blockIdx.y >= nrows) {  // block-uniform: a down unit
      fused_down_unit<BF16, FSW, FV, W>(fa, rv, hout, H, d_ff,
                                        ((int)blockIdx.y - nrows) * (int)gridDim.x +
                                            (int)blockIdx.x);
      return;
    }
  }
  __shared__ float red[W][2][MT][4][64];
  __shared__ int32_t s_pairc[16];  // VSEL: the pair of each tile column
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const bool slot = MT == 1 && rv.T <= 16;  // uniform
  int e = 0, q0 = 0, ntok = 0;
  int xtok = 0;  // VSEL: the token of tile column lane & 15
  if constexpr (VSEL > 0) {
    __shared__ int32_t s_pick[W][16];
    __shared__ uint32_t s_mask[8];
    __shared__ int32_t s_cnt[256 + 1];
    const int T = rv.T, K = rv.top_k, E = rv.E;
    const bool writer = blockIdx.x == 0 && blockIdx.y == 0;  // uniform
    if (threadIdx.x < 8) s_mask[threadIdx.x] = 0u;
    if (writer)
      for (int i = threadIdx.x; i < E; i += 64 * W) s_cnt[i] = 0;
    __syncthreads();
    if (wid < T) {  // wave-uniform
      int esel;
      float wsel;
      wave_topk<VSEL, false>(sel.part + (size_t)wid * E, (size_t)T * E, sel.nsplit, sel.bias, E, K,
                             sel.norm_topk, RosterArgs{}, wid, esel, wsel);
      if (lane < K) {
        s_pick[wid][lane] = esel;
        atomicOr(&s_mask[esel >> 5], 1u << (esel & 31));
        if (writer) {
          atomicAdd(&s_cnt[esel], 1);
          const_cast<int32_t *>(rv.topk_ids)[wid * K + lane] = esel;
          const_cast<float *>(rv.topk_w)[wid * K + lane] = wsel;
        }
      }
    }
    __syncthreads();
    // the slot's expert: the s-th smallest picked id (lanes 0..7 hold the mask words)
    const int s = blockIdx.y;
    const uint32_t mw = lane < 8 ? s_mask[lane] : 0u;
    const int cw = __popc(mw);
    const int incl = wave_incl_scan(cw);
    const int nact = lane_value(incl, 63);
    if (s >= nact) return;  // block-uniform
    const uint64_t wsel_m = __ballot(lane < 8 && incl > s && incl - cw <= s);
    const int L = __ffsll((unsigned long long)wsel_m) - 1;
    e = 32 * L + nth_set_bit(lane_value((int)mw, L), s - (lane_value(incl, L) - lane_value(cw, L)));
    // its tokens, ascending: lane t < T holds the slot of e in token t's picks
    int my_slot = -1;
    if (lane < T)
      for (int r2 = 0; r2 < K; ++r2) my_slot = s_pick[lane][r2] == e ? r2 : my_slot;
    const uint64_t tm = __ballot(lane < T && my_slot >= 0);
    ntok = __popcll(tm);
    const int c = lane & 15;
    const int tc = nth_set_bit(tm, c < ntok ? c : 0);
    xtok = tc;
    const int pc = tc * K + __shfl(my_slot, tc, 64);  // tc varies by lane: a permute, not a readlane
    if (wid == 0 && lane < 16) s_pairc[lane] = pc;  // read after the reduction barrier
    if (writer && wid == 0) {
      // grouping: CSR offsets, ascending active list, pairs by (expert, pair id)
      int32_t *off = const_cast<int32_t *>(rv.offsets);
      int32_t *act = const_cast<int32_t *>(rv.active);
      int32_t *pbe = const_cast<int32_t *>(rv.pair_by_expert);
      int base = 0, abase = 0;
      for (int e0 = 0; e0 < E; e0 += 64) {
        const int ee = e0 + lane;
        const int cnt = ee < E ? s_cnt[ee] : 0;
        const int ci = wave_incl_scan(cnt);
        const int fi = wave_incl_scan(cnt > 0 ? 1 : 0);
        if (ee < E) {
          off[ee] = base + ci - cnt;
          s_cnt[ee] = base + ci - cnt;  // becomes the expert's cursor
        }
        if (cnt > 0) act[abase + fi - 1] = ee;
        base += lane_value(ci, 63);
        abase += lane_value(fi, 63);
      }
      if (lane == 0) {
        off[E] = base;
        *const_cast<int32_t *>(rv.n_active) = abase;
      }
      for (int t = 0; t < T; ++t) {  // tokens in order: each expert's pairs ascend
        if (lane < K) {
          const int ee = s_pick[t][lane];
          const int at = s_cnt[ee];
          s_cnt[ee] = at + 1;  // distinct experts within a token
          pbe[at] = t * K + lane;
        }
      }
    }
  } else if (slot) {
    // every active expert holds <= T <= 16 tokens: work item == active slot
    // (s < min(E, P) <= E, so the slot's entry is read with the count)
    const int s = blockIdx.y;
    const int na = rv.nact();
    e = rv.expert(s);
    if (s >= na) return;  // block-uniform
  } else if (!find_item<16 * MT>(rv, blockIdx.y, e, q0, ntok)) {
    return;  // block-uniform
  }
  const int r = lane & 15, g = lane >> 4;
  const int row0 = blockIdx.x * 16;
  // packed weights: fragment (e, neuron tile, k-step) is 1 KB, lane-ordered
  const size_t ftile = (size_t)e * (d_ff / 16) + blockIdx.x;
  constexpr int EB = BF16 ? 2 : 4;
  constexpr int KPS = BF16 ? 32 : 16;       // k per step (one 1 KB fragment)
  const int nsteps = H / KPS;
  constexpr int U = 4;  // k-steps in flight per wave
  u32x4 ag[U], au[U];
  f32x4 accg[MT], accu[MT];
#pragma unroll
  for (int tl = 0; tl < MT; ++tl) { accg[tl] = f32x4{0, 0, 0, 0}; accu[tl] = f32x4{0, 0, 0, 0}; }
  int ntiles;

  if constexpr (PF) {
    const int wv = __builtin_amdgcn_readfirstlane(wid);
    const __amdgpu_buffer_rsrc_t rg = buf_rsrc(static_cast<const uint8_t *>(wgv) + ftile * nsteps * 1024,
                                               (uint32_t)nsteps * 1024);
    const __amdgpu_buffer_rsrc_t ru = buf_rsrc(static_cast<const uint8_t *>(wuv) + ftile * nsteps * 1024,
                                               (uint32_t)nsteps * 1024);
    const uint32_t woff = (uint32_t)lane * 16;
    auto load_w = [&](int s0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ks = s0 + W * u;
        if (ks < nsteps) {
          ag[u] = buf_ld16_nt(rg, woff, (uint32_t)ks * 1024);
          if (!GO) au[u] = buf_ld16_nt(ru, woff, (uint32_t)ks * 1024);
        }
      }
    };
    load_w(wv);
    if (VSEL == 0 && slot) {
      q0 = rv.begin(e);
      ntok = rv.end(e) - q0;
    }
    ntiles = (ntok + 15) >> 4;
    // lane (r, g) of tile tl reads token row t at elements k + g * (16 / EB) ..
    const __amdgpu_buffer_rsrc_t rx = buf_rsrc(xv, (uint32_t)rv.T * (uint32_t)H * EB);
    uint32_t xoff[MT];
#pragma unroll
    for (int tl = 0; tl < MT; ++tl) {
      const int c = tl * 16 + r;
      const int t = VSEL > 0 ? xtok : rv.pair_at(q0 + (c < ntok ? c : 0)) / rv.top_k;
      xoff[tl] = ((uint32_t)t * (uint32_t)H + (uint32_t)g * (16 / EB)) * EB;
    }
    for (int s = wv; s < nsteps; s += W * U) {
      if (s != wv) load_w(s);  // round s (the first was issued above)
      u32x4 bx[U][MT];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ks = s + W * u;
#pragma unroll
        for (int tl = 0; tl < MT; ++tl)
          if (ks < nsteps && tl < ntiles) bx[u][tl] = buf_ld16(rx, xoff[tl], (uint32_t)ks * (KPS * EB));
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ks = s + W * u;
        if (ks < nsteps) {
#pragma unroll
          for (int tl = 0; tl < MT; ++tl) {
            if (tl < ntiles) {
              const u32x4 b = bx[u][tl];
              if (BF16) {
                accg[tl] = mfma_bf16(ag[u], b, accg[tl]);
                if (!GO) accu[tl] = mfma_bf16(au[u], b, accu[tl]);
              } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  accg[tl] = mfma_f32(__uint_as_float(ag[u][j]), __uint_as_float(b[j]), accg[tl]);
                  if (!GO) accu[tl] = mfma_f32(__uint_as_float(au[u][j]), __uint_as_float(b[j]), accu[tl]);
                }
              }
            }
          }
        }
      }
    }
  } else {
    const uint8_t *wg = static_cast<const uint8_t *>(wgv) + (ftile * nsteps * 1024 + lane * 16);
    const uint8_t *wu = static_cast<const uint8_t *>(wuv) + (ftile * nsteps * 1024 + lane * 16);
    auto load_round = [&](int s0) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ks = s0 + W * u;
        if (ks < nsteps) {
          ag[u] = ld16_nt(wg + (size_t)ks * 1024);
          if (!GO) au[u] = ld16_nt(wu + (size_t)ks * 1024);
        }
      }
    };
    load_round(wid);
    if (VSEL == 0 && slot) {
      q0 = rv.begin(e);
      ntok = rv.end(e) - q0;
    }
    ntiles = (ntok + 15) >> 4;
    size_t xoff[MT];
    bool xval[MT];
#pragma unroll
    for (int tl = 0; tl < MT; ++tl) {
      const int c = tl * 16 + r;
      xval[tl] = c < ntok;
      const int t = !xval[tl] ? 0 : VSEL > 0 ? xtok : rv.pair_at(q0 + c) / rv.top_k;
      xoff[tl] = (size_t)t * H;
    }
    for (int s = wid; s < nsteps; s += W * U) {
      if (s != wid) load_round(s);  // round s (the first was issued above)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int ks = s + W * u;
        if (ks < nsteps) {
          if (BF16) {
            const int k = ks * 32 + g * 8;
            const uint16_t *x = static_cast<const uint16_t *>(xv);
#pragma unroll
            for (int tl = 0; tl < MT; ++tl) {
              if (tl < ntiles) {
                const u32x4 b = xval[tl] ? ld16(x + xoff[tl] + k) : u32x4{0, 0, 0, 0};
                accg[tl] = mfma_bf16(ag[u], b, accg[tl]);
                if (!GO) accu[tl] = mfma_bf16(au[u], b, accu[tl]);
              }
            }
          } else {
            const int k = ks * 16 + g * 4;
            const float *x = static_cast<const float *>(xv);
#pragma unroll
            for (int tl = 0; tl < MT; ++tl) {
              if (tl < ntiles) {
                const u32x4 b = xval[tl] ? ld16(x + xoff[tl] + k) : u32x4{0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  accg[tl] = mfma_f32(__uint_as_float(ag[u][j]), __uint_as_float(b[j]), accg[tl]);
                  if (!GO) accu[tl] = mfma_f32(__uint_as_float(au[u][j]), __uint_as_float(b[j]), accu[tl]);
                }
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
        if (!GO) red[wid][1][tl][rr][lane] = accu[tl][rr];
      }
    }
  }
  __syncthreads();
  for (int o = threadIdx.x; o < ntiles * 256; o += 64 * W) {
    const int tl = o >> 8, rr = (o >> 6) & 3, ln = o & 63;
    const int c = tl * 16 + (ln & 15);
    if (c < ntok) {
      float gs = 0.f, us = 0.f;
#pragma unroll
      for (int w = 0; w < W; ++w) {  // wave partials in fixed order
        gs += red[w][0][tl][rr][ln];
        if (!GO) us += red[w][1][tl][rr][ln];
      }
      const int neuron = row0 + 4 * (ln >> 4) + rr;
      const int p = VSEL > 0 ? s_pairc[c] : rv.pair_at(q0 + c);
      const float hv = GO ? silu(gs) : silu(gs) * us;
      if (FU) st_agent(hout + (size_t)p * d_ff + neuron, hv);
      else hout[(size_t)p * d_ff + neuron] = hv;
    }
  }
  if constexpr (FU) {  // this tile of expert e is complete and visible
    // the counters follow h in the workspace: their address comes from hout,
    // so the streaming loop above keeps no extra pointer live
    const int eu = __builtin_amdgcn_readfirstlane(e);
    wait_stores();
    __syncthreads();
    if (threadIdx.x == 0)
      atomicAdd(reinterpret_cast<int32_t *>(hout + (size_t)rv.T * rv.top_k * d_ff) +
                    (size_t)eu * kCounterStride, 1);
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
      // float-field digits: exponent, then 8, 8 and 7 mantissa bits
      const int shift = pass == 0 ? 23 : pass == 1 ? 15 : pass == 2 ? 7 : 0;
      const uint32_t dmask = pass == 3 ? 0x7fu : 0xffu;
      hist[tid] = 0;
      __syncthreads();
      for (int j = tid; j < d_ff; j += 256) {
        const uint32_t key = sbits[j] & 0x7fffffffu;
        if ((key & pmask) == tau) atomicAdd(&hist[(key >> shift) & dmask], 1);
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
      pmask |= dmask << shift;
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

// exp_digit_regs over a block of NW waves that share one pair: the largest
// exponent and the eight binade counts are combined across the waves
// through xch (LDS, NW x 5 words, written once), two block barriers in all.
template <int V, int NW>
__device__ __forceinline__ bool exp_digit_regs_block(const uint32_t (&bits)[V], int krem,
                                                     uint32_t (*xch)[5], uint32_t &tau,
                                                     uint32_t &pmask, int &krem_out, bool &whole) {
  static_assert(V <= 32, "per-lane counts must fit 8 bits");
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  uint32_t emax = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) emax = max(emax, (bits[i] & 0x7fffffffu) >> 23);
  emax = wave_max_u32(emax);
  if (lane == 0) xch[wid][0] = emax;
  __syncthreads();
#pragma unroll
  for (int ww = 0; ww < NW; ++ww) emax = max(emax, xch[ww][0]);
  uint32_t a = 0, b = 0;  // binades emax - 0 .. 3 and emax - 4 .. 7, a byte each
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const uint32_t d = emax - ((bits[i] & 0x7fffffffu) >> 23);  // >= 0
    const uint32_t one = 1u << (8 * (d & 3u));
    a += d < 4u ? one : 0u;
    b += d - 4u < 4u ? one : 0u;  // d in 4 .. 7
  }
  const uint32_t w[4] = {(a & 0xffu) | ((a & 0xff00u) << 8), ((a >> 16) & 0xffu) | ((a >> 8) & 0xff0000u),
                         (b & 0xffu) | ((b & 0xff00u) << 8), ((b >> 16) & 0xffu) | ((b >> 8) & 0xff0000u)};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const uint32_t tot = (uint32_t)lane_value(wave_incl_scan((int)w[q]), 63);
    if (lane == 0) xch[wid][1 + q] = tot;  // 16-bit fields: at most d_ff per field
  }
  __syncthreads();
  int run = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    uint32_t tot = 0;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) tot += xch[ww][1 + q];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int c = (int)((tot >> (16 * h)) & 0xffffu);
      if (run + c >= krem) {  // block-uniform; run < krem here
        tau = (emax - (uint32_t)(2 * q + h)) << 23;
        pmask = 0xffu << 23;
        krem_out = krem - run;
        whole = c == krem_out && tau != 0u;
        return true;
      }
      run += c;
    }
  }
  return false;
}

// Register-resident variant for d_ff = 64 * V * NW: a block of NW waves per
// pair, each lane holding V activations of one contiguous index segment
// (lane-major within a wave, waves in order), so the kept list comes out in
// index order from prefix counts alone.  The radix digits follow the float
// fields of |h| (bits 30..23 = exponent, then 22..15, 14..7, 6..0), so the
// first pass already spreads the values.  Each wave counts into its own
// 256-bin LDS histogram (no cross-wave atomic traffic); every wave then sums
// the NW histograms and finds the digit itself from the same counts, so all
// waves agree without a broadcast.  Scans are DPP wavefront scans.  The
// kept list (ids, w * h) is compacted in LDS and written with coalesced
// stores: per lane, kept entries are sparse among its V values, so direct
// stores would be V mostly-masked scattered instructions.
constexpr int kMaskStage = 4096;
template <int V, int NW>
__global__ __launch_bounds__(64 * NW) void neuron_topk_seg_kernel(const float *__restrict__ h,
                                                                  RouteView rv, int d_ff, int k,
                                                                  int32_t *__restrict__ idx,
                                                                  float *__restrict__ hact,
                                                                  void *__restrict__ hm,
                                                                  int hm_bf16) {
  __shared__ int hist[NW][256];
  __shared__ int wtot[2][NW];
  __shared__ uint32_t xch[NW][5];
  constexpr int SN = 64 * V * NW < kMaskStage ? 64 * V * NW : kMaskStage;  // k <= d_ff
  __shared__ int s_idx[SN + 64 * NW];  // + a spare slot per thread
  __shared__ float s_val[SN + 64 * NW];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int p = blockIdx.x;
  const float w = rv.weight(p);
  const int seg = (wid * 64 + lane) * V;  // first index of this lane's segment
  const float *hp = h + (size_t)p * d_ff + seg;
  uint32_t bits[V];
  if (V % 4 == 0) {  // 16-byte aligned: d_ff is a multiple of 64 and seg of 4
#pragma unroll
    for (int i = 0; i < V; i += 4) {
      const u32x4 q = ld16(hp + i);
      bits[i] = q[0]; bits[i + 1] = q[1]; bits[i + 2] = q[2]; bits[i + 3] = q[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) bits[i] = __float_as_uint(hp[i]);
  }

  const bool keep_all = k >= d_ff;
  uint32_t tau = 0, pmask = 0;
  int krem = k;
  bool whole = false;  // the last selected digit's bucket is kept entirely
  if (!keep_all && k > 0) {
    const bool p0 = exp_digit_regs_block<V, NW>(bits, k, xch, tau, pmask, krem, whole);
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      // block-uniform: every wave read the same counts and histograms
      if (whole || (pass == 0 && p0)) continue;
      const int shift = pass == 0 ? 23 : pass == 1 ? 15 : pass == 2 ? 7 : 0;
      const uint32_t dmask = pass == 3 ? 0x7fu : 0xffu;
#pragma unroll
      for (int b = 0; b < 4; ++b) hist[wid][lane * 4 + b] = 0;  // own histogram, in wave order
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const uint32_t key = bits[i] & 0x7fffffffu;
        if ((key & pmask) == tau) atomicAdd(&hist[wid][(key >> shift) & dmask], 1);
      }
      __syncthreads();
      // lane owns digits 255 - 4 lane - b, b = 0..3 (descending)
      int c[4], local = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        int n = 0;
#pragma unroll
        for (int ww = 0; ww < NW; ++ww) n += hist[ww][255 - 4 * lane - b];
        c[b] = n;
        local += n;
      }
      int run = wave_incl_scan(local) - local;  // keys with a larger digit
      int dsel = -1, knew = 0, csel = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (dsel < 0 && run + c[b] >= krem && run < krem) {
          dsel = 255 - 4 * lane - b;
          knew = krem - run;
          csel = c[b];
        }
        run += c[b];
      }
      const uint64_t m = __ballot(dsel >= 0);
      const int L = __ffsll((unsigned long long)m) - 1;  // exactly one lane (counts are exact)
      dsel = lane_value(dsel, L);
      knew = lane_value(knew, L);
      csel = lane_value(csel, L);
      tau |= (uint32_t)dsel << shift;
      pmask |= dmask << shift;
      krem = knew;
      // Keeping the whole bucket settles the set: every key whose prefix is
      // >= tau's, with no ties left to break.  The lower digits need no pass.
      whole = csel == knew && tau != 0u;
      __syncthreads();  // every wave has read the histograms before the next pass clears them
    }
    if (whole) {  // keep key >= tau (its lower bits are zero): key > tau - 1, no equal ones
      tau -= 1u;
      krem = 0;
    }
  }
  int ngt = 0, neq = 0;
  if (!keep_all && k > 0) {
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const uint32_t key = bits[i] & 0x7fffffffu;
      ngt += key > tau;
      neq += key == tau;
    }
  }
  const int gt_incl = wave_incl_scan(ngt), eq_incl = wave_incl_scan(neq);
  int gt_before = gt_incl - ngt, eq_before = eq_incl - neq;
  if (NW > 1) {
    if (lane == 63) { wtot[0][wid] = gt_incl; wtot[1][wid] = eq_incl; }
    __syncthreads();
    for (int ww = 0; ww < wid; ++ww) { gt_before += wtot[0][ww]; eq_before += wtot[1][ww]; }
  }
  int pos = keep_all ? seg : gt_before + min(eq_before, krem);
  int eq_seen = eq_before;
  const bool stage = k <= SN && (idx || hact);  // block-uniform
  float mv[V];
  if (stage && !keep_all && k > 0) {
    // the common case, without a branch per value: every value is written,
    // a dropped one (or one past k, which finite input never produces) to
    // this thread's spare slot (timing: 1.9 -> 0.8 us per select)
    const int spare = SN + threadIdx.x;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const uint32_t key = bits[i] & 0x7fffffffu;
      const int eq = key == tau ? 1 : 0;
      const bool keep = key > tau || (eq != 0 && eq_seen < krem);
      eq_seen += eq;
      const float v = w * __uint_as_float(bits[i]);
      const int slot = keep && pos < k ? pos : spare;
      s_idx[slot] = seg + i;
      s_val[slot] = v;
      pos += keep ? 1 : 0;
      mv[i] = keep ? v : 0.0f;
    }
  } else
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int j = seg + i;
    const uint32_t key = bits[i] & 0x7fffffffu;
    bool keep;
    if (keep_all) keep = true;
    else if (k == 0) keep = false;
    else if (key > tau) keep = true;
    else if (key == tau) keep = eq_seen++ < krem;
    else keep = false;
    const float v = w * __uint_as_float(bits[i]);
    if (keep) {
      if (pos < k) {  // always true: exactly k keys are kept
        if (stage) {
          s_idx[pos] = j;
          s_val[pos] = v;
        } else {
          if (idx) idx[(size_t)p * k + pos] = j;
          if (hact) hact[(size_t)p * k + pos] = v;
        }
      }
      ++pos;
    }
    mv[i] = keep ? v : 0.0f;
  }
  if (stage) {
    __syncthreads();
    for (int q = threadIdx.x; q < k; q += 64 * NW) {
      if (idx) idx[(size_t)p * k + q] = s_idx[q];
      if (hact) hact[(size_t)p * k + q] = s_val[q];
    }
  }
  if (hm) {  // dense masked row: this lane's V consecutive entries
    if (hm_bf16) {
      uint16_t *o = static_cast<uint16_t *>(hm) + (size_t)p * d_ff + seg;
      if (V % 8 == 0) {
#pragma unroll
        for (int i = 0; i < V; i += 8) {
          u32x4 q;
#pragma unroll
          for (int c = 0; c < 4; ++c)
            q[c] = f32_to_bf16_bits(mv[i + 2 * c]) | (f32_to_bf16_bits(mv[i + 2 * c + 1]) << 16);
          *reinterpret_cast<u32x4 *>(o + i) = q;
        }
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) o[i] = (uint16_t)f32_to_bf16_bits(mv[i]);
      }
    } else {
      float *o = static_cast<float *>(hm) + (size_t)p * d_ff + seg;
      if (V % 4 == 0) {
#pragma unroll
        for (int i = 0; i < V; i += 4)
          *reinterpret_cast<f32x4 *>(o + i) = f32x4{mv[i], mv[i + 1], mv[i + 2], mv[i + 3]};
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) o[i] = mv[i];
      }
    }
  }
}

// ---------------------------------------------------------------- sparse up
// The page's own split: the kept neurons' up projections, u_j = W_u[j, :] .
// x_t, for j in the pair's kept list only (W_u row-major, neuron-major like
// W_d).  One block per (pair, 8 kept rows), its waves splitting each row's
// bytes: per 1 KB chunk of a row (64 lanes x 16 bytes), the lane's slice of
// the token row x is loaded once and the 8 rows' slices are loaded together
// and dotted with it; each row's partial is then summed over the wave in a
// fixed DPP order and over the waves in wave order (two waves instead of
// one: OLMoE-like split layer 38.6 -> 37.1 us at one token, 87.0 -> 85.9 us
// at 16, up-rows kernel 8.5 -> 6.8 us at one token; four waves of 1 KB
// segments: up-rows 6.9 -> 6.5 us).  The kept coefficient
// (w * silu(g_j), from the mask) is multiplied by u_j in place, giving the
// down projection's w * h_j.
constexpr int kUpRows = 8;

// Rows i0 .. i0 + kUpRows - 1 (those below n) of pair p's kept list: ids
// idx_row[i], coefficients coef_row[i] multiplied in place by u = W_u row . x.
// NWU waves share the rows: wave w takes the row segments w, w + NWU, ...
// (2 KB, or 1 KB from four waves); the per-wave sums meet in LDS and are
// added in wave order (a fixed
// order, so reruns give the same bits).  Called by all NWU waves alike.
template <bool BF16, int NWU = 1>
__device__ __forceinline__ void up_rows_group(const void *__restrict__ wuv,
                                              const void *__restrict__ xv, const RouteView &rv,
                                              int H, int d_ff, int p, int i0, int n,
                                              const int32_t *__restrict__ idx_row,
                                              float *__restrict__ coef_row) {
  constexpr int EB = BF16 ? 2 : 4;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int t = p / rv.top_k;
  const size_t e = (size_t)rv.expert_of_pair(p);
  const uint8_t *rows[kUpRows];
#pragma unroll
  for (int r = 0; r < kUpRows; ++r) {
    const int i = i0 + r;
    int j = i < n ? idx_row[i] : 0;
    j = (unsigned)j < (unsigned)d_ff ? j : 0;
    rows[r] = static_cast<const uint8_t *>(wuv) + (e * d_ff + j) * H * EB;
  }
  const uint8_t *xr = static_cast<const uint8_t *>(xv) + (size_t)t * H * EB;
  const int row_bytes = H * EB;  // a multiple of 128: H is a multiple of 64
  float acc[kUpRows];
#pragma unroll
  for (int r = 0; r < kUpRows; ++r) acc[r] = 0.f;
  // ST 1 KB steps of every row in flight at once per wave: two with one or
  // two waves, one with four (row_bytes is a multiple of 128, so a step may
  // be partial: lanes past the row end load nothing)
  constexpr int ST = NWU >= 4 ? 1 : 2;
  for (int off0 = 1024 * ST * wid; off0 < row_bytes; off0 += 1024 * ST * NWU) {
    u32x4 xq[ST], q[ST][kUpRows];
#pragma unroll
    for (int h2 = 0; h2 < ST; ++h2) {
      const int off = off0 + 1024 * h2 + lane * 16;
      const bool in = off < row_bytes;
      xq[h2] = in ? ld16(xr + off) : u32x4{0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < kUpRows; ++r)
        q[h2][r] = in && i0 + r < n ? ld16(rows[r] + off) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int h2 = 0; h2 < ST; ++h2) {
#pragma unroll
      for (int r = 0; r < kUpRows; ++r) {
        float a = 0.f;
        if (BF16) {
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            a = fmaf(bf16lo(q[h2][r][c]), bf16lo(xq[h2][c]), a);
            a = fmaf(bf16hi(q[h2][r][c]), bf16hi(xq[h2][c]), a);
          }
        } else {
#pragma unroll
          for (int c = 0; c < 4; ++c)
            a = fmaf(__uint_as_float(q[h2][r][c]), __uint_as_float(xq[h2][c]), a);
        }
        acc[r] += a;
      }
    }
  }
  if constexpr (NWU == 1) {
#pragma unroll
    for (int r = 0; r < kUpRows; ++r) {
      const float u = wave_sum(acc[r]);
      const int i = i0 + r;
      if (lane == 0 && i < n) coef_row[i] *= u;
    }
  } else {
    __shared__ float part[NWU][kUpRows];
#pragma unroll
    for (int r = 0; r < kUpRows; ++r) {
      const float u = wave_sum(acc[r]);
      if (lane == 0) part[wid][r] = u;
    }
    __syncthreads();
    if (threadIdx.x < kUpRows) {
      const int i = i0 + (int)threadIdx.x;
      float u = part[0][threadIdx.x];
#pragma unroll
      for (int w = 1; w < NWU; ++w) u += part[w][threadIdx.x];
      if (i < n) coef_row[i] *= u;
    }
    __syncthreads();  // part is read before a caller's next group writes it
  }
}

// Fixed count k per pair (top-k masks): block (p, g) takes rows 8 g ...
// with kUpWaves waves splitting each row's bytes.
#ifndef MOE_UP_WAVES
#define MOE_UP_WAVES 4
#endif
constexpr int kUpWaves = MOE_UP_WAVES;
template <bool BF16>
__global__ __launch_bounds__(64 * kUpWaves) void up_rows_kernel(const void *__restrict__ wuv,
                                                                const void *__restrict__ xv,
                                                                RouteView rv, int H, int d_ff,
                                                                int k,
                                                                const int32_t *__restrict__ idx,
                                                                float *__restrict__ coef) {
  const int p = blockIdx.x;
  up_rows_group<BF16, kUpWaves>(wuv, xv, rv, H, d_ff, p, blockIdx.y * kUpRows, k,
                                idx + (size_t)p * k, coef + (size_t)p * k);
}

// Per-pair counts (threshold masks), lists at row stride d_ff: block (p, g)
// takes row groups g, g + G, ... below the pair's count (G = gridDim.y), so
// the grid does not depend on the data.
template <bool BF16>
__global__ __launch_bounds__(64 * kUpWaves) void up_rows_var_kernel(const void *__restrict__ wuv,
                                                                    const void *__restrict__ xv,
                                                                    RouteView rv, int H, int d_ff,
                                                                    const int32_t *__restrict__ counts,
                                                                    const int32_t *__restrict__ idx,
                                                                    float *__restrict__ coef) {
  const int p = blockIdx.x;
  int n = counts[p];
  n = n < 0 ? 0 : (n > d_ff ? d_ff : n);
  for (int i0 = blockIdx.y * kUpRows; i0 < n; i0 += gridDim.y * kUpRows)  // block-uniform
    up_rows_group<BF16, kUpWaves>(wuv, xv, rv, H, d_ff, p, i0, n, idx + (size_t)p * d_ff,
                                  coef + (size_t)p * d_ff);
}

// y[t, cols] (+)= sum over the token's pairs (slot order) and their kept rows
// (ascending) of coef * W_d^e[row, cols]: the down projection streams only
// the kept rows, and the weighted scatter-add of the token's experts happens
// in the same block, in a fixed order (no atomics, bitwise reproducible).
// Block = 16 waves, one token x SW output columns (SW = 64 or 128); each
// kept row contributes one SW-element run (128 to 512 bytes).  The host
// takes the wider blocks when the grid still holds >= 256 of them: longer
// runs per row and half the per-block fixed cost.  Rows are read through
// the caches (a partial-line gather, where the non-temporal hint measured
// slower).  The token's row list (expert, row, coefficient) is staged in
// LDS, kDownStage entries at a time, so the weight loads issue back to
// back.  With idx == nullptr the rows are 0..k-1 (coefficient row stride
// k): the dense fp32 path's masked rows, or with weighted != 0 the unmasked
// h itself, each pair's rows scaled by its routing weight here.
template <bool BF16, int SW>
__global__ __launch_bounds__(1024) void down_token_kernel(const void *__restrict__ wdv,
                                                          const int32_t *__restrict__ idx,
                                                          const float *__restrict__ coef,
                                                          RouteView rv, int H, int d_ff, int k,
                                                          int weighted, int accumulate,
                                                          float *__restrict__ y,
                                                          const void *xres, void *xnext) {
  constexpr int VEC = BF16 ? 8 : 4;   // elements per 16-byte load
  constexpr int LPR = SW / VEC;       // lanes per row
  static_assert(LPR <= 64 && 64 % LPR == 0, "a row run must fit one wave");
  __shared__ float red[kDownWaves][SW];
  __shared__ uint32_t srow[kDownStage];  // expert * d_ff + row
  __shared__ float scoef[kDownStage];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int t = blockIdx.x, col0 = blockIdx.y * SW;
  const int top_k = rv.top_k;
  const int nrows = top_k * k;
  const int sub = lane % LPR, rsel = lane / LPR;
  const size_t colo = (size_t)col0 + sub * VEC;
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
  for (int base = 0; base < nrows; base += kDownStage) {
    const int n = min(kDownStage, nrows - base);
    for (int q = threadIdx.x; q < n; q += 1024) {
      const int qq = base + q;
      const int s = qq / k, i = qq - s * k;
      const int p = t * top_k + s;
      int j = idx ? idx[(size_t)p * k + i] : i;
      j = (unsigned)j < (unsigned)d_ff ? j : 0;
      srow[q] = (uint32_t)rv.expert_of_pair(p) * (uint32_t)d_ff + (uint32_t)j;
      const float c = coef[(size_t)p * k + i];
      scoef[q] = weighted ? rv.weight(p) * c : c;
    }
    __syncthreads();
    stream_rows<BF16, SW>(wdv, srow, scoef, n, H, colo, wid, rsel, acc);
    if (base + kDownStage < nrows) __syncthreads();  // consumed before the next chunk is staged
  }
  // lanes with the same columns (same sub) hold different rows: fold them
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] += __shfl_xor(acc[v], o, 64);
  }
  if (rsel == 0) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) red[wid][sub * VEC + v] = acc[v];
  }
  __syncthreads();
  if (threadIdx.x < SW) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kDownWaves; ++w) v += red[w][threadIdx.x];
    const size_t o = (size_t)t * H + col0 + threadIdx.x;
    const float out = accumulate ? y[o] + v : v;
    y[o] = out;
    if (xnext) residual_store<BF16>(xres, xnext, o, out);
  }
}

// ---------------------------------------------------------------- threshold masking
// The page's literal masking: one pass comparing each |h_j| with the
// pair's expert threshold tau_e (calibrated offline), no select.  Kept
// counts vary per pair; ids and w * h are written compacted in index order
// at row stride d_ff, with the count per pair.  Layout as the register-
// resident select (NW waves, V values per lane, contiguous segments), so
// positions come from one wave scan plus the per-wave totals.  tau < 0
// keeps every neuron; otherwise |h| > tau is a compare of the bit patterns
// (order-preserving for non-negative floats).
template <int V, int NW>
__global__ __launch_bounds__(64 * NW) void neuron_threshold_kernel(const float *__restrict__ h,
                                                                   RouteView rv, int d_ff,
                                                                   const float *__restrict__ tau,
                                                                   int32_t *__restrict__ idx,
                                                                   float *__restrict__ coef,
                                                                   int32_t *__restrict__ counts) {
  __shared__ int wtot[NW];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int p = blockIdx.x;
  const float w = rv.weight(p);
  const float te = tau[rv.expert_of_pair(p)];
  const bool all = te < 0.f;
  const uint32_t tkey = __float_as_uint(fabsf(te));
  const int seg = (wid * 64 + lane) * V;
  uint32_t bits[V];
  const float *hp = h + (size_t)p * d_ff + seg;
  if (V % 4 == 0) {
#pragma unroll
    for (int i = 0; i < V; i += 4) {
      const u32x4 q = ld16(hp + i);
      bits[i] = q[0]; bits[i + 1] = q[1]; bits[i + 2] = q[2]; bits[i + 3] = q[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < V; ++i) bits[i] = __float_as_uint(hp[i]);
  }
  int n = 0;
#pragma unroll
  for (int i = 0; i < V; ++i) n += all || (bits[i] & 0x7fffffffu) > tkey;
  const int incl = wave_incl_scan(n);
  int pos = incl - n;
  if (NW > 1) {
    if (lane == 63) wtot[wid] = incl;
    __syncthreads();
    for (int ww = 0; ww < wid; ++ww) pos += wtot[ww];
  }
#pragma unroll
  for (int i = 0; i < V; ++i) {
    if (all || (bits[i] & 0x7fffffffu) > tkey) {
      idx[(size_t)p * d_ff + pos] = seg + i;
      coef[(size_t)p * d_ff + pos] = w * __uint_as_float(bits[i]);
      ++pos;
    }
  }
  if (wid == NW - 1 && lane == 63) counts[p] = pos;  // the last segment's end = the count
}

// ---------------------------------------------------------------- variable-count sparse down
// down_token_kernel for per-pair kept counts (threshold masking): the
// token's pairs' lists (ids and coefficients at row stride d_ff, counts[p]
// entries each) are concatenated in slot order and staged into LDS in
// chunks of kDownStage rows, each chunk streamed like down_token_kernel's
// (SW-column row slices, 4 load instructions in flight per wave) before
// the next is staged; lane folds then waves reduce in a fixed order.
template <bool BF16, int SW>
__global__ __launch_bounds__(1024) void down_var_token_kernel(const void *__restrict__ wdv,
                                                              const int32_t *__restrict__ idx,
                                                              const float *__restrict__ coef,
                                                              const int32_t *__restrict__ counts,
                                                              RouteView rv, int H, int d_ff,
                                                              int accumulate,
                                                              float *__restrict__ y) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int LPR = SW / VEC;
  constexpr int RPI = 64 / LPR;
  __shared__ float red[kDownWaves][SW];
  __shared__ uint32_t srow[kDownStage];
  __shared__ float scoef[kDownStage];
  __shared__ int pref[33];  // row offset of each slot's list (top_k <= 32)
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int t = blockIdx.x, col0 = blockIdx.y * SW;
  const int top_k = rv.top_k;
  if ((int)threadIdx.x < top_k) {
    const int c = counts[t * top_k + threadIdx.x];
    pref[threadIdx.x + 1] = c < 0 ? 0 : (c > d_ff ? d_ff : c);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    pref[0] = 0;
    for (int s = 1; s <= top_k; ++s) pref[s] += pref[s - 1];
  }
  __syncthreads();
  const int nrows = pref[top_k];
  const int sub = lane % LPR, rsel = lane / LPR;
  const size_t colo = (size_t)col0 + sub * VEC;
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
  for (int base = 0; base < nrows; base += kDownStage) {
    const int n = min(kDownStage, nrows - base);
    for (int q = threadIdx.x; q < n; q += 1024) {
      const int qq = base + q;
      int lo = 0, hi = top_k;  // the slot s with pref[s] <= qq < pref[s + 1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (pref[mid] <= qq) lo = mid; else hi = mid;
      }
      const int p = t * top_k + lo, i = qq - pref[lo];
      int j = idx[(size_t)p * d_ff + i];
      j = (unsigned)j < (unsigned)d_ff ? j : 0;
      srow[q] = (uint32_t)rv.expert_of_pair(p) * (uint32_t)d_ff + (uint32_t)j;
      scoef[q] = coef[(size_t)p * d_ff + i];
    }
    __syncthreads();
    stream_rows<BF16, SW>(wdv, srow, scoef, n, H, colo, wid, rsel, acc);
    __syncthreads();  // the chunk is consumed before the next is staged
  }
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] += __shfl_xor(acc[v], o, 64);
  }
  if (rsel == 0) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) red[wid][sub * VEC + v] = acc[v];
  }
  __syncthreads();
  if (threadIdx.x < SW) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kDownWaves; ++w) v += red[w][threadIdx.x];
    float *yp = y + (size_t)t * H + col0 + threadIdx.x;
    *yp = accumulate ? *yp + v : v;
  }
}

// ---------------------------------------------------------------- fused top-k mask + down
// The smallest batches: each down block selects its own token's kept neurons, one
// wave per pair (exact top-k of |h|: the radix select of
// neuron_topk_seg_kernel with NW = 1, V = d_ff / 64 values per lane, its own
// LDS histogram, no block barriers), and writes the kept rows straight into
// the LDS row list at the pair's fixed offset s * k.  The mask kernel and
// its launch go away; the select is repeated by the token's H / SW blocks,
// which costs a read of the token's activations from the caches each.
// Blocks of column chunk 0 also write the kept ids (the caller's
// active_idx_out) if asked.  Requires top_k <= 16, 0 < k < d_ff and
// top_k * k <= kDownStage.
template <bool BF16, int SW, int V>
__global__ __launch_bounds__(1024) void down_topk_token_kernel(
    const void *__restrict__ wdv, const float *__restrict__ h, RouteView rv, int H, int d_ff,
    int k, int accumulate, float *__restrict__ y, int32_t *__restrict__ idx_out,
    const void *xres, void *xnext) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int LPR = SW / VEC;
  constexpr int RPI = 64 / LPR;
  __shared__ float red[kDownWaves][SW];
  __shared__ uint32_t srow[kDownStage + 64 * kDownWaves];  // + a spare slot per selecting lane
  __shared__ float scoef[kDownStage + 64 * kDownWaves];
  __shared__ int hist[kDownWaves][256];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int t = blockIdx.x, col0 = blockIdx.y * SW;
  const int top_k = rv.top_k;
  if (wid < top_k) {  // wave-uniform: this wave selects slot wid's neurons
    const int p = t * top_k + wid;
    const float w = rv.weight(p);
    const uint32_t rbase = (uint32_t)rv.expert_of_pair(p) * (uint32_t)d_ff;
    const int seg = lane * V;
    const float *hp = h + (size_t)p * d_ff + seg;
    uint32_t bits[V];
#pragma unroll
    for (int i = 0; i < V; i += 4) {
      const u32x4 q = ld16(hp + i);
      bits[i] = q[0]; bits[i + 1] = q[1]; bits[i + 2] = q[2]; bits[i + 3] = q[3];
    }
    uint32_t tau = 0, pmask = 0;
    int krem = k;
    bool whole = false;
    int *hw = hist[wid];
    const bool p0 = exp_digit_regs<V>(bits, k, tau, pmask, krem, whole);
#pragma unroll
    for (int pass = 0; pass < 4; ++pass) {
      if (whole || (pass == 0 && p0)) continue;  // wave-uniform
      const int shift = pass == 0 ? 23 : pass == 1 ? 15 : pass == 2 ? 7 : 0;
      const uint32_t dmask = pass == 3 ? 0x7fu : 0xffu;
#pragma unroll
      for (int b = 0; b < 4; ++b) hw[lane * 4 + b] = 0;
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const uint32_t key = bits[i] & 0x7fffffffu;
        if ((key & pmask) == tau) atomicAdd(&hw[(key >> shift) & dmask], 1);
      }
      // lane owns digits 255 - 4 lane - b, b = 0..3 (descending)
      int c[4], local = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        c[b] = hw[255 - 4 * lane - b];
        local += c[b];
      }
      int run = wave_incl_scan(local) - local;
      int dsel = -1, knew = 0, csel = 0;
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        if (dsel < 0 && run + c[b] >= krem && run < krem) {
          dsel = 255 - 4 * lane - b;
          knew = krem - run;
          csel = c[b];
        }
        run += c[b];
      }
      const uint64_t m = __ballot(dsel >= 0);
      const int L = __ffsll((unsigned long long)m) - 1;  // exactly one lane (counts are exact)
      dsel = lane_value(dsel, L);
      knew = lane_value(knew, L);
      csel = lane_value(csel, L);
      tau |= (uint32_t)dsel << shift;
      pmask |= dmask << shift;
      krem = knew;
      whole = csel == knew && tau != 0u;
    }
    if (whole) {  // keep key >= tau: key > tau - 1, no equal ones
      tau -= 1u;
      krem = 0;
    }
    int ngt = 0, neq = 0;
#pragma unroll
    for (int i = 0; i < V; ++i) {
      const uint32_t key = bits[i] & 0x7fffffffu;
      ngt += key > tau;
      neq += key == tau;
    }
    const int eq_before = wave_incl_scan(neq) - neq;
    int pos = wave_incl_scan(ngt) - ngt + min(eq_before, krem);
    int eq_seen = eq_before;
    const int obase = wid * k;
    int32_t *io = (idx_out && blockIdx.y == 0) ? idx_out + (size_t)p * k : nullptr;
    if (io) {
#pragma unroll
      for (int i = 0; i < V; ++i) {
        const uint32_t key = bits[i] & 0x7fffffffu;
        const bool keep = key > tau || (key == tau && eq_seen++ < krem);
        if (keep) {
          srow[obase + pos] = rbase + (uint32_t)(seg + i);
          scoef[obase + pos] = w * __uint_as_float(bits[i]);
          io[pos] = seg + i;
          ++pos;
        }
      }
    } else {
      keep_list_lds(bits, tau, krem, eq_seen, pos, k, seg, rbase, w, srow, scoef, obase,
                    kDownStage + tid);
    }
  }
  __syncthreads();
  const int nr = top_k * k;
  const int sub = lane % LPR, rsel = lane / LPR;
  const size_t colo = (size_t)col0 + sub * VEC;
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
  stream_rows<BF16, SW>(wdv, srow, scoef, nr, H, colo, wid, rsel, acc);
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] += __shfl_xor(acc[v], o, 64);
  }
  if (rsel == 0) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) red[wid][sub * VEC + v] = acc[v];
  }
  __syncthreads();
  if (tid < SW) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kDownWaves; ++w) v += red[w][tid];
    const size_t o = (size_t)t * H + col0 + tid;
    const float out = accumulate ? y[o] + v : v;
    y[o] = out;
    if (xnext) residual_store<BF16>(xres, xnext, o, out);
  }
}

// ---------------------------------------------------------------- fused threshold mask + down
// Decode batches: the threshold compare is one cheap pass, so each down
// block redoes it for its token instead of reading a mask kernel's output,
// and the mask launch disappears.  A token's pairs' activations are one
// contiguous run h[t * top_k * d_ff ..) in (slot, neuron) order; thread i
// owns the C elements [i C, i C + C) (C a multiple of 4, 16-byte loads).
// Pass 1 counts kept elements per thread (|h| > tau[e], or all if tau < 0)
// and per slot; a block scan gives each thread its place in the token's
// kept list, which is then staged into LDS chunk by chunk (pass 2 re-reads
// the thread's elements, from L2) and streamed as in down_token_kernel.
// Blocks of column chunk 0 also write the kept counts and ids if asked.
template <bool BF16, int SW>
__global__ __launch_bounds__(1024) void down_thr_token_kernel(
    const void *__restrict__ wdv, const float *__restrict__ h, const float *__restrict__ tau,
    RouteView rv, int H, int d_ff, int accumulate, float *__restrict__ y,
    int32_t *__restrict__ counts_out, int32_t *__restrict__ idx_out) {
  constexpr int VEC = BF16 ? 8 : 4;
  constexpr int LPR = SW / VEC;
  constexpr int RPI = 64 / LPR;
  __shared__ float red[kDownWaves][SW];
  __shared__ uint32_t srow[kDownStage];
  __shared__ float scoef[kDownStage];
  __shared__ uint32_t skey[32], sbase[32];
  __shared__ float sw[32];
  __shared__ int spref[33], tmp[16];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int t = blockIdx.x, col0 = blockIdx.y * SW;
  const int top_k = rv.top_k, n = top_k * d_ff;
  const int C = ((n + 4095) / 4096) * 4;  // elements per thread
  if (tid < top_k) {
    const int p = t * top_k + tid, e = rv.expert_of_pair(p);
    const float te = tau[e];
    skey[tid] = te < 0.f ? 0xffffffffu : __float_as_uint(fabsf(te));  // ~0: keep all
    sbase[tid] = (uint32_t)e * (uint32_t)d_ff;
    sw[tid] = rv.weight(p);
  }
  __syncthreads();
  const float *ht = h + (size_t)t * n;
  const int q0 = tid * C;
  auto kept = [&](uint32_t bits, int s) {
    const uint32_t k = skey[s];
    return k == 0xffffffffu || (bits & 0x7fffffffu) > k;
  };
  // The thread's first 4 KC elements stay in registers between the passes
  // (all of them for up to 64 K elements per token); the rest are re-read.
  constexpr int KC = 4;
  u32x4 cache[KC];
  auto elems = [&](int c) {  // the 4 elements at offset c of the thread's range
    u32x4 v;
#pragma unroll
    for (int r = 0; r < KC; ++r)
      if (c == 4 * r) v = cache[r];
    return c < 4 * KC ? v : ld16(ht + q0 + c);
  };
  // pass 1: per-thread count.  A slot starts at a multiple of d_ff, and a
  // thread's range (C < d_ff elements) holds at most one such start: that
  // thread notes how many of its kept elements precede it, which after the
  // scan gives the slot's offset in the token's kept list.
  int cnt = 0, my_s = -1, my_before = 0;
#pragma unroll
  for (int r = 0; r < KC; ++r)
    if (4 * r < C && q0 + 4 * r < n) cache[r] = ld16(ht + q0 + 4 * r);
  for (int c = 0; c < C && q0 + c < n; c += 4) {
    const u32x4 v = elems(c);
    const int s = (q0 + c) / d_ff;  // 4 elements never straddle slots (d_ff % 64 == 0)
    if (q0 + c == s * d_ff) { my_s = s; my_before = cnt; }
    int m = 0;
#pragma unroll
    for (int u = 0; u < 4; ++u) m += kept(v[u], s);
    cnt += m;
  }
  int total = 0;
  const int incl = block_incl_scan<1024>(cnt, tmp, &total);
  const int my0 = incl - cnt;
  if (my_s >= 0) spref[my_s] = my0 + my_before;
  if (tid == 0) spref[top_k] = total;
  __syncthreads();
  if (blockIdx.y == 0) {  // the token's counts and kept ids, for the caller
    if (counts_out && tid < top_k) counts_out[t * top_k + tid] = spref[tid + 1] - spref[tid];
    if (idx_out && cnt) {
      int pos = my0;
      for (int c = 0; c < C && q0 + c < n; c += 4) {
        const u32x4 v = elems(c);
        const int s = (q0 + c) / d_ff;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (kept(v[u], s)) {
            const int j = q0 + c + u - s * d_ff;
            idx_out[(size_t)(t * top_k + s) * d_ff + (pos - spref[s])] = j;
            ++pos;
          }
        }
      }
    }
  }
  const int sub = lane % LPR, rsel = lane / LPR;
  const size_t colo = (size_t)col0 + sub * VEC;
  float acc[VEC];
#pragma unroll
  for (int v = 0; v < VEC; ++v) acc[v] = 0.f;
  for (int base = 0; base < total; base += kDownStage) {
    const int nr = min(kDownStage, total - base);
    // pass 2: stage the kept rows whose list positions fall in this chunk
    if (cnt && my0 < base + nr && my0 + cnt > base) {
      int pos = my0;
      for (int c = 0; c < C && q0 + c < n; c += 4) {
        const u32x4 v = elems(c);
        const int s = (q0 + c) / d_ff;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          if (kept(v[u], s)) {
            if (pos >= base && pos < base + nr) {
              const int j = q0 + c + u - s * d_ff;
              srow[pos - base] = sbase[s] + (uint32_t)j;
              scoef[pos - base] = sw[s] * __uint_as_float(v[u]);
            }
            ++pos;
          }
        }
      }
    }
    __syncthreads();
    stream_rows<BF16, SW>(wdv, srow, scoef, nr, H, colo, wid, rsel, acc);
    __syncthreads();  // the chunk is consumed before the next is staged
  }
#pragma unroll
  for (int o = LPR; o < 64; o <<= 1) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) acc[v] += __shfl_xor(acc[v], o, 64);
  }
  if (rsel == 0) {
#pragma unroll
    for (int v = 0; v < VEC; ++v) red[wid][sub * VEC + v] = acc[v];
  }
  __syncthreads();
  if (tid < SW) {
    float v = 0.f;
#pragma unroll
    for (int w = 0; w < kDownWaves; ++w) v += red[w][tid];
    float *yp = y + (size_t)t * H + col0 + tid;
    *yp = accumulate ? *yp + v : v;
  }
}

// ---------------------------------------------------------------- threshold calibration
// tau for one score set: the (c + 1)-th largest |h| of its m scores, c =
// ceil((1 - s) m - 1e-9) (the keep count), or -1 when c >= m.  Block b < E
// takes expert b's scores (its pairs' h rows, all d_ff neurons); block E
// takes every pair's.  An exact radix select over the float-field digits
// of |h| in global memory: 4 passes of block histograms (per-wave LDS
// histograms summed), each keeping the digit whose bucket holds the target
// rank.  Experts with no scores are left for calibrate_fill_kernel.
__global__ __launch_bounds__(1024) void calibrate_kernel(const float *__restrict__ h, RouteView rv,
                                                         int d_ff, double sparsity,
                                                         float *__restrict__ tau,
                                                         float *__restrict__ tau_all) {
  __shared__ int hist[16][256];
  __shared__ int tot[256];
  __shared__ int sel[2];
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int e = blockIdx.x;
  const bool layer = e == rv.E;
  int q0 = 0, q1 = 0;
  if (layer) {
    q1 = rv.T * rv.top_k;     // every pair, in pair-id order
  } else if (rv.implicit) {
    q0 = e * rv.T;
    q1 = q0 + rv.T;
  } else {
    q0 = rv.offsets[e];
    q1 = rv.offsets[e + 1];
  }
  const long long m = (long long)(q1 - q0) * d_ff;
  if (m == 0) return;  // block-uniform
  const long long c = (long long)ceil((1.0 - sparsity) * (double)m - 1e-9);
  float result = -1.f;
  if (c < m) {
    long long krem = c + 1;  // rank of tau among the keys, descending (1-based)
    uint32_t pre = 0, pmask = 0;
    for (int pass = 0; pass < 4; ++pass) {
      const int shift = pass == 0 ? 23 : pass == 1 ? 15 : pass == 2 ? 7 : 0;
      const uint32_t dmask = pass == 3 ? 0x7fu : 0xffu;
      for (int i = lane; i < 256; i += 64) hist[wid][i] = 0;
      __syncthreads();
      for (long long z = tid; z < m; z += 1024) {
        const int qi = (int)(z / d_ff), j = (int)(z - (long long)qi * d_ff);
        const int p = layer ? q0 + qi : rv.pair_at(q0 + qi);
        const uint32_t key = __float_as_uint(h[(size_t)p * d_ff + j]) & 0x7fffffffu;
        if ((key & pmask) == pre) atomicAdd(&hist[wid][(key >> shift) & dmask], 1);
      }
      __syncthreads();
      if (tid < 256) {
        int n = 0;
        for (int w = 0; w < 16; ++w) n += hist[w][tid];
        tot[tid] = n;
      }
      __syncthreads();
      if (tid == 0) {  // 256 buckets, descending: a short serial walk
        long long run = 0;
        int d = 255;
        for (; d > 0; --d) {
          if (run + tot[d] >= krem) break;
          run += tot[d];
        }
        sel[0] = d;
        sel[1] = (int)(krem - run);
      }
      __syncthreads();
      pre |= (uint32_t)sel[0] << shift;
      pmask |= dmask << shift;
      krem = sel[1];
      __syncthreads();
    }
    result = __uint_as_float(pre);
  }
  if (tid == 0) {
    if (layer) *tau_all = result;
    else tau[e] = result;
  }
}

__global__ __launch_bounds__(64) void calibrate_fill_kernel(RouteView rv, const float *tau_all,
                                                            float *__restrict__ tau) {
  for (int e = threadIdx.x; e < rv.E; e += 64) {
    const int n = rv.implicit ? rv.T : rv.offsets[e + 1] - rv.offsets[e];
    if (n == 0) tau[e] = *tau_all;
  }
}

// idx[q] = q mod d_ff: the kept-id lists of calls that keep every neuron.
__global__ __launch_bounds__(256) void iota_rows_kernel(int32_t *__restrict__ idx, size_t n,
                                                        int d_ff) {
  const size_t q = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (q < n) idx[q] = (int32_t)(q % (size_t)d_ff);
}

__global__ __launch_bounds__(256) void zero_kernel(float *__restrict__ y, size_t n) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) y[i] = 0.f;
}

// ---------------------------------------------------------------- host side

static void launch_mask(const FfnArgs &a, const RouteView &rv, int32_t *idx, float *hact, void *hm,
                        int hm_bf16, hipStream_t stream) {
  const int P = a.T * a.top_k;
  timer_begin(kStageMask, stream);
  // register-resident segments: 4 waves per pair up to d_ff = 2048 (d_ff / 256
  // values per lane), one wave for the other multiples of 64 up to 2048, 8
  // waves from 2560 to 8192 (d_ff / 512 values per lane)
#define MOE_MASK_CASE(V, NW)                                                                  \
  case 64 * V * NW:                                                                           \
    neuron_topk_seg_kernel<V, NW><<<P, 64 * NW, 0, stream>>>(a.h, rv, a.d_ff, a.k_keep, idx, \
                                                            hact, hm, hm_bf16);              \
    break;
  switch (a.d_ff) {
    MOE_MASK_CASE(1, 4) MOE_MASK_CASE(2, 4) MOE_MASK_CASE(3, 4) MOE_MASK_CASE(4, 4)
    MOE_MASK_CASE(5, 4) MOE_MASK_CASE(6, 4) MOE_MASK_CASE(7, 4) MOE_MASK_CASE(8, 4)
    MOE_MASK_CASE(1, 1) MOE_MASK_CASE(2, 1) MOE_MASK_CASE(3, 1) MOE_MASK_CASE(5, 1)
    MOE_MASK_CASE(6, 1) MOE_MASK_CASE(7, 1) MOE_MASK_CASE(9, 1) MOE_MASK_CASE(10, 1)
    MOE_MASK_CASE(11, 1) MOE_MASK_CASE(13, 1) MOE_MASK_CASE(14, 1) MOE_MASK_CASE(15, 1)
    MOE_MASK_CASE(17, 1) MOE_MASK_CASE(18, 1) MOE_MASK_CASE(19, 1) MOE_MASK_CASE(21, 1)
    MOE_MASK_CASE(22, 1) MOE_MASK_CASE(23, 1) MOE_MASK_CASE(25, 1) MOE_MASK_CASE(26, 1)
    MOE_MASK_CASE(27, 1) MOE_MASK_CASE(29, 1) MOE_MASK_CASE(30, 1) MOE_MASK_CASE(31, 1)
    MOE_MASK_CASE(5, 8) MOE_MASK_CASE(6, 8) MOE_MASK_CASE(7, 8) MOE_MASK_CASE(8, 8)
    MOE_MASK_CASE(9, 8) MOE_MASK_CASE(10, 8) MOE_MASK_CASE(11, 8) MOE_MASK_CASE(12, 8)
    MOE_MASK_CASE(13, 8) MOE_MASK_CASE(14, 8) MOE_MASK_CASE(15, 8) MOE_MASK_CASE(16, 8)
#undef MOE_MASK_CASE
    default:
      neuron_topk_kernel<<<P, 256, (size_t)a.d_ff * 4, stream>>>(a.h, rv, a.d_ff, a.k_keep, idx,
                                                                  hact, hm, hm_bf16);
  }
  timer_end(stream);
}

// A routed expert never holds more than T tokens, so at T <= 16 one token
// tile per item suffices; that variant splits K over 8 waves (short blocks,
// high occupancy, no tail of half-empty block rounds).  Up to 64 tokens the
// same kernel takes items of one expert and <= 16 of its tokens: at a few
// tokens per expert it beats the grouped GEMM, whose 128-token items and
// staged token tiles only pay off once experts hold many tokens (measured
// on four layer families at T = 32 and 64: 13-22 % faster layers where
// experts hold 1-4 tokens, equal on the OLMoE-like layer at T = 64).
// Always-on (implicit) experts past 16 tokens hold every token, so 16-token
// items stream each expert's weights T / 16 times: bf16 calls take the
// grouped GEMM there, which reads them once per 128 tokens, where its grid
// still has >= 128 blocks (Llama-4-like shared expert, d_ff 8192, T = 64:
// 122.8 -> 61.4 us; DeepSeek-V2-like, two of d_ff 1536, 48 GEMM blocks:
// 27.9 us on 16-token items against 60.0 on the GEMM at T = 32).
// gate_only: the page's own split, h <- silu(W_g x) (the scores), up skipped.
#ifndef MOE_SWIGLU_MAX_T
#define MOE_SWIGLU_MAX_T 64
#endif
static void launch_gateup(const FfnArgs &a, const RouteView &rv, hipStream_t stream,
                          bool gate_only = false) {
  timer_begin(kStageGateup, stream);
  const bool shared_gemm = a.implicit && a.bf16 && a.T > 16 &&
                           (long)n_items(a, 128) * (a.d_ff / 64) >= 128;
  if (a.T <= MOE_SWIGLU_MAX_T && !shared_gemm) {
    // T <= 16: an item is an active-expert slot, at most min(E, P) of them;
    // past that an item is an expert and up to 16 of its tokens
    const int P = a.T * a.top_k;
    dim3 grid(a.d_ff / 16, a.T <= 16 ? (a.implicit ? a.E : (a.E < P ? a.E : P)) : n_items(a, 16));
#define MOE_GU(BF, GOV, PFV) \
  gateup_swiglu_kernel<BF, 1, 8, GOV, PFV><<<grid, 512, 0, stream>>>(a.x, a.w_gate, a.w_up, rv, a.H, a.d_ff, a.h)
#define MOE_GU_PF(BF, GOV) \
  if (a.T == 1) MOE_GU(BF, GOV, true); else MOE_GU(BF, GOV, false);
    if (a.bf16) { if (gate_only) { MOE_GU_PF(true, true) } else { MOE_GU_PF(true, false) } }
    else { if (gate_only) { MOE_GU_PF(false, true) } else { MOE_GU_PF(false, false) } }
#undef MOE_GU_PF
#undef MOE_GU
  } else {
    launch_gateup_gemm(a, rv, gate_only, stream);
  }
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

// Output columns per down block: 128 while that still gives >= 256 blocks
// (one per CU), else 64 so that small batches spread over more CUs.
static int down_block_cols(int T, int H) {
  return H % 128 == 0 && (long)T * (H / 128) >= 256 ? 128 : 64;
}

static void launch_down_token(const FfnArgs &a, const RouteView &rv, const int32_t *idx,
                              const float *coef, int k, hipStream_t stream, int weighted = 0) {
  const int sw = down_block_cols(a.T, a.H);
  dim3 grid(a.T, a.H / sw);
  timer_begin(kStageDownRows, stream);
#define MOE_DOWN(BF, SWV)                                                                     \
  down_token_kernel<BF, SWV><<<grid, 1024, 0, stream>>>(a.w_down, idx, coef, rv, a.H, a.d_ff, k, \
                                                        weighted, a.accumulate, a.y, a.xres,    \
                                                        a.xnext)
  if (a.bf16) {
    if (sw == 128) MOE_DOWN(true, 128); else MOE_DOWN(true, 64);
  } else {
    if (sw == 128) MOE_DOWN(false, 128); else MOE_DOWN(false, 64);
  }
#undef MOE_DOWN
  timer_end(stream);
}

// Whether the kernel that selects inside the down projection takes this
// call: one wave per pair, d_ff / 64 values per lane (a multiple of 4 up to
// 32), the token's kept lists in one LDS stage, and the batches where its
// repeated selects (every column block of a token selects again) cost less
// than the mask launch they save.  Per layer call against the mask and down
// kernels (alternating runs on one box): OLMoE-like 5 tokens 68.3 vs 65.8
// us, Qwen3-MoE-like 47.8 vs 45.1; up to 8 tokens it also beats the fused
// launch (below).  With 24 values per lane (DeepSeek-V2-like, d_ff 1536)
// it wins up to 3 tokens (1: 84.0 vs 86.5 us) and loses from 4 (179.0 vs
// 175.7; 16: 417.5 vs 408.4).  With at most 12 values per lane the select is
// cheap enough past the fused launch's batches too (Qwen3-MoE-like, d_ff
// 768: 17 tokens 68.7 vs 66.0 us, 32: 85.4 vs 83.0, level at 48 and 64).
constexpr int kTopkMaxTokensNarrow = 32;  // d_ff <= 768 (9-16 tokens: the fused launch)
constexpr int kTopkMaxTokens = 8;         // d_ff 1024
constexpr int kTopkMaxTokensWide = 3;     // d_ff 1280 .. 2048
static bool fused_topk_ok(const FfnArgs &a) {
  const int V = a.d_ff / 64;
  const int tmax = V <= 12 ? kTopkMaxTokensNarrow : V <= 16 ? kTopkMaxTokens : kTopkMaxTokensWide;
  return a.T <= tmax && a.top_k <= kDownWaves &&
         a.d_ff % 256 == 0 && V <= 32 &&
         a.k_keep > 0 && a.k_keep < a.d_ff && a.top_k * a.k_keep <= kDownStage;
}

// The fused select + down kernel of the smallest batches (fused_topk_ok).
static void launch_down_topk(const FfnArgs &a, const RouteView &rv, hipStream_t stream) {
  const int sw = down_block_cols(a.T, a.H);
  dim3 grid(a.T, a.H / sw);
  int32_t *io = a.want_idx ? a.idx : nullptr;
  timer_begin(kStageDownRows, stream);
#define MOE_DK(BF, SWV, VV)                                                                   \
  down_topk_token_kernel<BF, SWV, VV><<<grid, 1024, 0, stream>>>(a.w_down, a.h, rv, a.H, a.d_ff, \
                                                               a.k_keep, a.accumulate, a.y, io, \
                                                               a.xres, a.xnext)
#define MOE_DK_V(BF, SWV)                                                                     \
  switch (a.d_ff / 64) {                                                                      \
  case 4: MOE_DK(BF, SWV, 4); break;                                                        \
  case 8: MOE_DK(BF, SWV, 8); break;                                                        \
  case 12: MOE_DK(BF, SWV, 12); break;                                                      \
  case 16: MOE_DK(BF, SWV, 16); break;                                                      \
  case 20: MOE_DK(BF, SWV, 20); break;                                                      \
  case 24: MOE_DK(BF, SWV, 24); break;                                                      \
  case 28: MOE_DK(BF, SWV, 28); break;                                                      \
  default: MOE_DK(BF, SWV, 32); break;                                                      \
  }
  if (a.bf16) { if (sw == 128) { MOE_DK_V(true, 128) } else { MOE_DK_V(true, 64) } }
  else { if (sw == 128) { MOE_DK_V(false, 128) } else { MOE_DK_V(false, 64) } }
#undef MOE_DK_V
#undef MOE_DK
  timer_end(stream);
}

// ---- the fused decode-batch FFN: gate/up, masks, down and combine in one
// launch, from kFusedMinTokens tokens and for d_ff up to 1024.  Measured per
// layer call against the separate kernels that select inside the down
// projection (same box, runs alternating), OLMoE-like: 73.9 vs 71.9 us at 6
// tokens, 83.1 vs 82.1 at 8, 95.4 vs 99.7 at 12, 103.4 vs 104.5 at 16;
// Qwen3-MoE-like: 50.2 vs 47.4 at 6, 54.1 vs 53.6 at 8, 56.5 vs 58.2 at 12,
// 64.4 vs 65.8 at 16.  Below that the down units wait resident through the
// whole weight stream and their polls slow it.  At d_ff 1536
// (DeepSeek-V2-like, 24 activations per lane) the separate mask and down
// kernels were as fast or faster at every batch (5 tokens: 191.5 vs 196.5
// us, 16: 407.2 vs 412.1).
constexpr int kFusedMinTokens = 9;
static bool tail_units_shape_ok(const FfnArgs &a) {
  const int V = a.d_ff / 64;
  // d_ff 512, 768, 1024 (at 2048 the fused kernel spills in its loop)
  return !a.implicit && a.T >= 1 && a.T <= kFusedMaxTokens && a.top_k <= 16 &&
         a.d_ff % 256 == 0 && (V == 8 || V == 12 || V == 16) &&
         a.k_keep > 0 && a.k_keep < a.d_ff && a.k_keep <= kFusedMaxK && a.H % 64 == 0 &&
         a.fpart != nullptr &&
         // the gate/up blocks find the counters right after h
         a.sync == reinterpret_cast<int32_t *>(a.h + (size_t)a.T * a.top_k * a.d_ff);
}
bool fused_ffn_ok(const FfnArgs &a) { return tail_units_shape_ok(a) && a.T >= kFusedMinTokens; }

// Output columns per down unit: at least 512 units where the hidden size
// allows (each unit streams SW columns of the pair's k rows), never below
// 128-byte runs; 64 columns at one or two tokens.
static int fused_cols(const FfnArgs &a) {
  const long P = (long)a.T * a.top_k;
  if (a.T > 2 && a.H % 256 == 0 && P * (a.H / 256) >= 512) return 256;
  if (a.T > 2 && a.H % 128 == 0 && P * (a.H / 128) >= 512) return 128;
  return 64;
}

__global__ __launch_bounds__(256) void zero_i32_kernel(int32_t *__restrict__ p, int n) {
  for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

template <bool BF, int SWV, int FVV>
static void fused_inst(const FfnArgs &a, const RouteView &rv, const FusedArgs &fa, dim3 grid,
                       hipStream_t stream) {
  gateup_swiglu_kernel<BF, 1, 8, false, true, 0, true, SWV, FVV><<<grid, 512, 0, stream>>>(
      a.x, a.w_gate, a.w_up, rv, a.H, a.d_ff, a.h, LayerSel{}, fa);
}
template <bool BF, int SWV>
static void fused_v(const FfnArgs &a, const RouteView &rv, const FusedArgs &fa, dim3 grid,
                    hipStream_t stream) {
  switch (a.d_ff / 64) {
    case 8: fused_inst<BF, SWV, 8>(a, rv, fa, grid, stream); break;
    case 12: fused_inst<BF, SWV, 12>(a, rv, fa, grid, stream); break;
    default: fused_inst<BF, SWV, 16>(a, rv, fa, grid, stream); break;
  }
}
template <bool BF>
static void fused_sw(const FfnArgs &a, const RouteView &rv, const FusedArgs &fa, int sw,
                     dim3 grid, hipStream_t stream) {
  if (sw == 256) fused_v<BF, 256>(a, rv, fa, grid, stream);
  else if (sw == 128) fused_v<BF, 128>(a, rv, fa, grid, stream);
  else fused_v<BF, 64>(a, rv, fa, grid, stream);
}

static FusedArgs fused_args(const FfnArgs &a, int gu_rows, int ncb) {
  FusedArgs fa;
  fa.gu_rows = gu_rows;
  fa.ncb = ncb;
  fa.npairs = a.T * a.top_k;
  fa.k = a.k_keep;
  fa.wd = a.w_down;
  fa.part = a.fpart;
  fa.cnt_e = a.sync;
  fa.cnt_tc = a.sync + (size_t)a.E * kCounterStride;
  fa.abort_flag = fa.cnt_tc + (size_t)a.T * (a.H / 64);
  fa.y = a.y;
  fa.accumulate = a.accumulate;
  fa.xres = a.xres;
  fa.xnext = a.xnext;
  fa.idx_out = a.want_idx ? a.idx : nullptr;
  return fa;
}

// The fused launch (fused_ffn_ok); the routing comes from an earlier kernel.
static hipError_t launch_ffn_fused(const FfnArgs &a, const RouteView &rv, hipStream_t stream) {
  const int P = a.T * a.top_k;
  const int sw = fused_cols(a);
  const int nt = a.d_ff / 16;
  const int gu_rows = a.E < P ? a.E : P;
  const int ncb = a.H / sw;
  const int down_rows = (P * ncb + nt - 1) / nt;
  const int nsync = (int)fused_sync_words(a.T, a.E, a.H);
  if (!a.sync_zeroed) zero_i32_kernel<<<(nsync + 255) / 256, 256, 0, stream>>>(a.sync, nsync);
  const FusedArgs fa = fused_args(a, gu_rows, ncb);
  dim3 grid(nt, gu_rows + down_rows);
  // the gate/up blocks load through buffer resources at every batch here:
  // the plain form sits at the 64-register limit and, with the fused tail
  // in the same kernel, spilled inside its streaming loop
  timer_begin(kStageFused, stream);
  if (a.bf16) fused_sw<true>(a, rv, fa, sw, grid, stream);
  else fused_sw<false>(a, rv, fa, sw, grid, stream);
  timer_end(stream);
  return hipGetLastError();
}

hipError_t launch_ffn_sparse(const FfnArgs &a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  if (zero_contribution(a, stream)) {
    if (a.xnext) return launch_residual(a.xres, a.y, a.xnext, (size_t)a.T * a.H, a.bf16, stream);
    return hipGetLastError();
  }
  const RouteView rv = make_view(a);
  if (fused_ffn_ok(a)) return launch_ffn_fused(a, rv, stream);
  launch_gateup(a, rv, stream);
  if (union_down_ok(a)) {
    launch_mask(a, rv, a.idx, a.hact, nullptr, 0, stream);
    return launch_down_union(a, rv, stream);
  }
  if (fused_topk_ok(a)) {
    launch_down_topk(a, rv, stream);
    return hipGetLastError();
  }
  launch_mask(a, rv, a.idx, a.hact, nullptr, 0, stream);
  launch_down_token(a, rv, a.idx, a.hact, a.k_keep, stream);
  return hipGetLastError();
}

// Layers of up to 8 tokens: logits, then gate/up blocks that select their
// own expert from the logit partials (block (0, 0) writes the routing
// outputs), then the mask and down kernels as launch_ffn_sparse runs them.
// The router's select-and-group launch goes away; every output equals
// moe_route followed by launch_ffn_sparse bit for bit (the selection is the
// router's own code, the grouping its stable order).
// One gate/up wave per token, so up to 8 tokens can select in-kernel; it
// pays only up to 2 (measured per layer call, OLMoE-like: 45.6-47.1 ->
// 44.4 us at 2 tokens, but 62.4 -> 62.8 us at 4 and 84.1 -> 89.2 us at 8,
// where every block rereads T tokens' logit partials and waits on T
// selections; 1 token stays within noise).  The selection code is
// parity-tested up to 8 tokens.
constexpr int kLayerSelMaxTokens = 2;
bool layer_small_ok(const RouteArgs &r, const FfnArgs &a) {
  return a.T >= 1 && a.T <= kLayerSelMaxTokens && r.T == a.T && !a.implicit &&
         r.roster.usage == nullptr && r.E <= 256 && a.E == r.E && a.top_k == r.top_k &&
         a.top_k <= 16 && a.k_keep > 0;
}

hipError_t launch_layer_small(const RouteArgs &r, const FfnArgs &a, hipStream_t stream) {
  if (!layer_small_ok(r, a)) return hipErrorInvalidValue;
  const RouteView rv = make_view(a);
  const int nsplit = launch_router_logits(r, stream);
  const LayerSel sel{r.logits, nsplit, r.norm_topk, r.bias};
  const int P = a.T * a.top_k;
  dim3 grid(a.d_ff / 16, a.E < P ? a.E : P);
  timer_begin(kStageGateup, stream);
#define MOE_GS(BF, PFV, V)                                                                      \
  gateup_swiglu_kernel<BF, 1, 8, false, PFV, V><<<grid, 512, 0, stream>>>(a.x, a.w_gate, a.w_up, \
                                                                         rv, a.H, a.d_ff, a.h, sel)
#define MOE_GS_V(BF, PFV) \
  if (r.E <= 64) MOE_GS(BF, PFV, 1); else if (r.E <= 128) MOE_GS(BF, PFV, 2); else MOE_GS(BF, PFV, 4);
  if (a.bf16) {
    if (a.T == 1) { MOE_GS_V(true, true) } else { MOE_GS_V(true, false) }
  } else {
    if (a.T == 1) { MOE_GS_V(false, true) } else { MOE_GS_V(false, false) }
  }
#undef MOE_GS_V
#undef MOE_GS
  timer_end(stream);
  if (fused_topk_ok(a)) {
    launch_down_topk(a, rv, stream);
  } else {
    launch_mask(a, rv, a.idx, a.hact, nullptr, 0, stream);
    launch_down_token(a, rv, a.idx, a.hact, a.k_keep, stream);
  }
  return hipGetLastError();
}

// The page's own split: dense gate scores, mask on |silu(g)|, the kept
// neurons' up rows (coefficients become w * silu(g_j) * u_j), then the same
// sparse down projection.
hipError_t launch_ffn_updown(const FfnArgs &a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  if (zero_contribution(a, stream)) return hipGetLastError();
  const RouteView rv = make_view(a);
  launch_gateup(a, rv, stream, true);
  launch_mask(a, rv, a.idx, a.hact, nullptr, 0, stream);
  const int P = a.T * a.top_k;
  dim3 grid(P, (a.k_keep + kUpRows - 1) / kUpRows);
  timer_begin(kStageUpRows, stream);
  if (a.bf16)
    up_rows_kernel<true><<<grid, 64 * kUpWaves, 0, stream>>>(a.w_up, a.x, rv, a.H, a.d_ff, a.k_keep, a.idx, a.hact);
  else
    up_rows_kernel<false><<<grid, 64 * kUpWaves, 0, stream>>>(a.w_up, a.x, rv, a.H, a.d_ff, a.k_keep, a.idx, a.hact);
  timer_end(stream);
  launch_down_token(a, rv, a.idx, a.hact, a.k_keep, stream);
  return hipGetLastError();
}

// Register-segment layout of the threshold mask for this d_ff, as the
// select's: 4 waves up to 2048 (multiples of 256), 1 wave for the other
// multiples of 64 up to 2048, 8 waves from 2560 to 8192 (multiples of 512).
bool threshold_supported(int d_ff) {
  if (d_ff <= 2048) return d_ff % 64 == 0;
  return d_ff % 512 == 0 && d_ff <= 8192;
}

// The one-pass threshold mask over the scores in a.h: kept ids and w * score
// at row stride d_ff, and a count per pair.
static hipError_t launch_threshold_mask(const FfnArgs &a, const RouteView &rv, const float *tau,
                                        int32_t *counts, hipStream_t stream) {
  const int P = a.T * a.top_k;
  timer_begin(kStageMask, stream);
  switch (a.d_ff) {
#define MOE_THR_CASE(V, NW)                                                                     \
  case 64 * V * NW:                                                                             \
    neuron_threshold_kernel<V, NW><<<P, 64 * NW, 0, stream>>>(a.h, rv, a.d_ff, tau, a.idx, a.hact, \
                                                             counts);                           \
    break;
    MOE_THR_CASE(1, 4) MOE_THR_CASE(2, 4) MOE_THR_CASE(3, 4) MOE_THR_CASE(4, 4)
    MOE_THR_CASE(5, 4) MOE_THR_CASE(6, 4) MOE_THR_CASE(7, 4) MOE_THR_CASE(8, 4)
    MOE_THR_CASE(1, 1) MOE_THR_CASE(2, 1) MOE_THR_CASE(3, 1) MOE_THR_CASE(5, 1)
    MOE_THR_CASE(6, 1) MOE_THR_CASE(7, 1) MOE_THR_CASE(9, 1) MOE_THR_CASE(10, 1)
    MOE_THR_CASE(11, 1) MOE_THR_CASE(13, 1) MOE_THR_CASE(14, 1) MOE_THR_CASE(15, 1)
    MOE_THR_CASE(17, 1) MOE_THR_CASE(18, 1) MOE_THR_CASE(19, 1) MOE_THR_CASE(21, 1)
    MOE_THR_CASE(22, 1) MOE_THR_CASE(23, 1) MOE_THR_CASE(25, 1) MOE_THR_CASE(26, 1)
    MOE_THR_CASE(27, 1) MOE_THR_CASE(29, 1) MOE_THR_CASE(30, 1) MOE_THR_CASE(31, 1)
    MOE_THR_CASE(5, 8) MOE_THR_CASE(6, 8) MOE_THR_CASE(7, 8) MOE_THR_CASE(8, 8)
    MOE_THR_CASE(9, 8) MOE_THR_CASE(10, 8) MOE_THR_CASE(11, 8) MOE_THR_CASE(12, 8)
    MOE_THR_CASE(13, 8) MOE_THR_CASE(14, 8) MOE_THR_CASE(15, 8) MOE_THR_CASE(16, 8)
#undef MOE_THR_CASE
    default:
      timer_end(stream);
      return hipErrorInvalidValue;  // excluded by threshold_supported()
  }
  timer_end(stream);
  return hipSuccess;
}

// The variable-count sparse down projection over a threshold mask's lists.
static void launch_down_var(const FfnArgs &a, const RouteView &rv, const int32_t *counts,
                            hipStream_t stream) {
  const int sw = down_block_cols(a.T, a.H);
  dim3 grid(a.T, a.H / sw);
  timer_begin(kStageDownRows, stream);
#define MOE_DV(BF, SWV)                                                                           \
  down_var_token_kernel<BF, SWV><<<grid, 1024, 0, stream>>>(a.w_down, a.idx, a.hact, counts, rv, \
                                                            a.H, a.d_ff, a.accumulate, a.y)
  if (a.bf16) { if (sw == 128) MOE_DV(true, 128); else MOE_DV(true, 64); }
  else { if (sw == 128) MOE_DV(false, 128); else MOE_DV(false, 64); }
#undef MOE_DV
  timer_end(stream);
}

// The page's literal masking: gate/up, one compare pass against tau[e],
// then the variable-count sparse down projection.
hipError_t launch_ffn_threshold(const FfnArgs &a, const float *tau, int32_t *counts,
                                bool want_counts, bool want_idx, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const RouteView rv = make_view(a);
  launch_gateup(a, rv, stream);
  if (a.T <= 16) {  // decode batches: the compare runs inside the down kernel
    const int sw = down_block_cols(a.T, a.H);
    dim3 grid(a.T, a.H / sw);
    int32_t *co = want_counts ? counts : nullptr;
    int32_t *io = want_idx ? a.idx : nullptr;
    timer_begin(kStageDownRows, stream);
#define MOE_DT(BF, SWV)                                                                         \
  down_thr_token_kernel<BF, SWV><<<grid, 1024, 0, stream>>>(a.w_down, a.h, tau, rv, a.H, a.d_ff, \
                                                            a.accumulate, a.y, co, io)
    if (a.bf16) { if (sw == 128) MOE_DT(true, 128); else MOE_DT(true, 64); }
    else { if (sw == 128) MOE_DT(false, 128); else MOE_DT(false, 64); }
#undef MOE_DT
    timer_end(stream);
    return hipGetLastError();
  }
  const hipError_t e = launch_threshold_mask(a, rv, tau, counts, stream);
  if (e != hipSuccess) return e;
  launch_down_var(a, rv, counts, stream);
  return hipGetLastError();
}

// The page's own pipeline with its threshold mask: dense gate scores
// silu(W_g x), one compare pass against tau[e], then the up and down
// projections over the kept rows only (w_up row-major).
hipError_t launch_ffn_updown_threshold(const FfnArgs &a, const float *tau, int32_t *counts,
                                       hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const RouteView rv = make_view(a);
  launch_gateup(a, rv, stream, true);
  const hipError_t e = launch_threshold_mask(a, rv, tau, counts, stream);
  if (e != hipSuccess) return e;
  const int P = a.T * a.top_k;
  const int groups = (a.d_ff + kUpRows - 1) / kUpRows;
  int G = (2048 + P - 1) / P;  // about 2048 blocks in all
  G = G < 1 ? 1 : (G > groups ? groups : G);
  dim3 grid(P, G);
  timer_begin(kStageUpRows, stream);
  if (a.bf16)
    up_rows_var_kernel<true><<<grid, 64 * kUpWaves, 0, stream>>>(a.w_up, a.x, rv, a.H, a.d_ff, counts, a.idx,
                                                      a.hact);
  else
    up_rows_var_kernel<false><<<grid, 64 * kUpWaves, 0, stream>>>(a.w_up, a.x, rv, a.H, a.d_ff, counts, a.idx,
                                                       a.hact);
  timer_end(stream);
  launch_down_var(a, rv, counts, stream);
  return hipGetLastError();
}

// Calibration: gate/up (or the gate alone, for the split's scores) on the
// calibration tokens, then the per-expert order statistic (and the
// layer-wide one for experts without tokens).
hipError_t launch_calibrate(const FfnArgs &a, double sparsity, float *tau, float *tau_all,
                            bool gate_only, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  const RouteView rv = make_view(a);
  launch_gateup(a, rv, stream, gate_only);
  calibrate_kernel<<<a.E + 1, 1024, 0, stream>>>(a.h, rv, a.d_ff, sparsity, tau, tau_all);
  calibrate_fill_kernel<<<1, 64, 0, stream>>>(rv, tau_all, tau);
  return hipGetLastError();
}

// Unmasked bf16 calls (k_keep == d_ff) whose experts hold about one token
// each read no more W_d rows streaming every row per pair than the grouped
// GEMM reads per expert, and skip its mask, partials and combine: the row
// kernel then takes h directly (weights applied while staging).  Tokens per
// active expert: T for the always-on experts, else the uniform-routing
// expectation T k_r / (E (1 - (1 - k_r / E)^T)); the rows pass while that
// is at most 2 (repeats among an expert's tokens come from the caches).
// A row block holds one token, so a token's rows must also stay within one
// LDS stage: past that, T x H / 64 blocks stream too many bytes each (a
// single token's 8192 rows took 1.4-2x the GEMM route's time on 32 and 80
// blocks; 3072 rows on 80 blocks saved 30 % of the down stage).  The row
// kernel reads row-major W_d, so a packed W_d always takes the GEMM.
static bool dense_rows_ok(const FfnArgs &a) {
  if (!a.bf16 || a.down_packed || a.k_keep != a.d_ff || (long)a.top_k * a.d_ff > kDownStage)
    return false;
  double n_e = a.T;
  if (!a.implicit) {
    const double E = a.E, K = a.top_k;
    n_e = (double)a.T * K / (E * (1.0 - pow(1.0 - K / E, (double)a.T)));
  }
  return n_e <= 2.0;
}

hipError_t launch_ffn_dense(const FfnArgs &a, hipStream_t stream) {
  if (a.T == 0) return hipSuccess;
  if (zero_contribution(a, stream)) return hipGetLastError();
  const RouteView rv = make_view(a);
  launch_gateup(a, rv, stream);
  if (dense_rows_ok(a)) {
    if (a.want_idx) {  // every neuron is kept: ids 0 .. d_ff - 1 per pair
      const size_t n = (size_t)a.T * a.top_k * a.d_ff;
      iota_rows_kernel<<<(unsigned)((n + 255) / 256), 256, 0, stream>>>(a.idx, n, a.d_ff);
    }
    launch_down_token(a, rv, nullptr, a.h, a.d_ff, stream, 1);
    return hipGetLastError();
  }
  launch_mask(a, rv, a.idx, nullptr, a.hm, a.bf16, stream);
  if (a.bf16) return launch_down_dense(a, rv, stream);
  // fp32: every row of W_d against the dense masked row, on the row kernel
  launch_down_token(a, rv, nullptr, static_cast<const float *>(a.hm), a.d_ff, stream);
  return hipGetLastError();
}

}  // namespace moe
