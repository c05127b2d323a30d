/*
 * moe_mi355x.h -- C ABI of the intra-expert-sparse MoE decode layer for
 * AMD MI355X (gfx950).  Library: libmoe_mi355x.so.
 *
 * The layer (router top-k -> dense SwiGLU gate/up -> zero the lowest-|h|
 * neurons -> down projection over the surviving rows only) follows the page
 * "Uncovering Intra-expert Activation Sparsity for Efficient
 * Mixture-of-Expert Model Execution" (gist.science explainer of the paper by
 * Park, Kim, Gu, Stoica and Cheung), called "the page" below; each entry
 * point names the section of the page it implements.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Every tensor pointer is caller-owned DEVICE memory on the current HIP
 *   device.  The library never allocates, frees or keeps a pointer after
 *   returning.  Scratch memory comes from the caller's `workspace`, sized by
 *   the matching *_workspace_size() call (the workspace contents between
 *   calls are not needed by the library; it may be reused freely once the
 *   stream has consumed the call).
 * - Calls only ENQUEUE kernels on `stream` (0 = the null stream).  They never
 *   synchronise, copy to the host or allocate, so a sequence of them can be
 *   captured into a HIP graph.  Grids depend on shapes only; data-dependent
 *   counts (active experts, tokens per expert) are read on the device.
 * - Arguments are validated before anything is enqueued; on any error
 *   nothing is enqueued and every output is untouched.  moe_last_error()
 *   then gives a description (thread-local).  MOE_ERR_HIP means a launch
 *   failed; the stream's contents are then unspecified.
 * - T == 0 is a valid no-op returning MOE_OK.
 * - NaN or Inf in x or weights gives unspecified (but memory-safe) results.
 * - Every tensor base pointer must be 16-byte aligned (MOE_ERR_MISALIGNED);
 *   256-byte aligned pointers (torch's allocations) always qualify.
 * - Layouts are row-major.  Expert weights are [E, d_ff, H] NEURON-MAJOR for
 *   gate, up AND down: row j of the down matrix is neuron j's H-vector
 *   contribution (the transpose of a torch down_proj.weight [H, d_ff]), so
 *   a kept neuron's down row is one contiguous H * elem_bytes stream.
 *   The FFN calls read gate and up in the PACKED layout that
 *   moe_pack_gate_up produces from that row-major form (once, at load time);
 *   down and the router matrix stay row-major.  The descriptor says which
 *   layout the caller passes (moe_desc.gate_up_layout): a descriptor left at
 *   MOE_LAYOUT_ROWMAJOR (zero) is refused by every FFN call with
 *   MOE_ERR_UNSUPPORTED, so an unpacked tensor is never misread.
 * - dtype MOE_BF16: x, router and expert weights are bf16 (raw bits,
 *   round-to-nearest-even), every accumulation is fp32; MOE_F32: all fp32.
 *   Router logits, softmax weights, h and y are fp32 in both.
 * - The library holds no global state and is reentrant; two calls that
 *   share a workspace must be ordered on one stream.  The one exception is
 *   moe_layer_sparse_noalloc, whose workspace is a static per-device array.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1,  /* NULL where a tensor is required, bad size, k out of range */
  MOE_ERR_MISALIGNED = 2,   /* a tensor base pointer is not 16-byte aligned              */
  MOE_ERR_WORKSPACE = 3,    /* workspace NULL or smaller than *_workspace_size()          */
  MOE_ERR_UNSUPPORTED = 4,  /* shape outside the limits below, unknown dtype or path      */
  MOE_ERR_HIP = 5           /* a kernel launch failed                                     */
} moe_status;

typedef enum { MOE_PATH_SPARSE = 0, MOE_PATH_DENSE = 1 } moe_path;

/* Layout of the gate (and up) tensors a caller passes to the FFN calls.
 * ROWMAJOR: [E, d_ff, H] as loaded; PACKED: after moe_pack_gate_up. */
typedef enum { MOE_LAYOUT_ROWMAJOR = 0, MOE_LAYOUT_PACKED = 1 } moe_layout;

/* Limits (MOE_ERR_UNSUPPORTED outside them). */
#define MOE_MAX_HIDDEN 16384   /* H: multiple of 64                        */
#define MOE_MAX_EXPERTS 1024   /* E                                        */
#define MOE_MAX_DFF 8192       /* d_ff: multiple of 64                     */
#define MOE_MAX_TOPK 32        /* router top_k, <= E                       */
#define MOE_MAX_TOKENS 65536   /* T per call                               */

/* Geometry of ONE expert group (the routed experts, or the shared ones). */
typedef struct {
  int32_t hidden;     /* H                                                        */
  int32_t n_experts;  /* E                                                        */
  int32_t d_ff;       /* per-expert intermediate size                             */
  int32_t top_k;      /* experts per token; for a shared group (routing == NULL)
                         it must equal n_experts                                  */
  int32_t norm_topk;  /* 1: renormalise the selected softmax weights to sum 1    */
  int32_t dtype;      /* moe_dtype                                                */
  int32_t gate_up_layout; /* moe_layout of w_gate, and of w_up where the call reads
                             it densely; the FFN calls need MOE_LAYOUT_PACKED (else
                             MOE_ERR_UNSUPPORTED); moe_route and the packing calls
                             ignore it; a value outside moe_layout ->
                             MOE_ERR_INVALID_ARG                                   */
  int32_t down_layout;    /* moe_layout of w_down: ROWMAJOR (zero) for every call;
                             PACKED (moe_pack_down) is taken by moe_expert_ffn_dense
                             only, bf16 only (the sparse calls gather W_d rows and
                             refuse it with MOE_ERR_UNSUPPORTED, as the dense call
                             does for fp32); outside moe_layout -> INVALID_ARG       */
} moe_desc;

/* Routing of a token batch, written by moe_route, read by the FFN calls.
 * All device pointers, caller-owned.  A pair is one (token, slot):
 * pair id p = t * top_k + slot, P = T * top_k. */
typedef struct {
  int32_t *topk_ids;        /* [T, top_k] expert ids; slot order = descending logit,
                               equal logits -> lower expert id                       */
  float *topk_w;            /* [T, top_k] softmax weight of each selected expert
                               (renormalised over the selection if norm_topk)        */
  int32_t *expert_offsets;  /* [E + 1] CSR offsets into pair_by_expert               */
  int32_t *pair_by_expert;  /* [P] pair ids grouped by expert; within an expert in
                               ascending token order (stable counting sort)          */
  int32_t *active_experts;  /* [E] ids of experts with >= 1 pair, ascending; entries
                               at and after n_active are unspecified                 */
  int32_t *n_active;        /* [1] number of active experts                          */
} moe_routing;

/*
 * moe_route -- router logits, softmax, top-k selection and the
 * token -> expert grouping.
 *
 * The page keeps the router unchanged (technical summary, Methodology: vLLM
 * implementation, router logic preserved); the grouping lets each expert's
 * tokens run as one batched product (same section: the gate projection
 * runs as a batched matrix multiply).
 *
 *   l[t, e] = sum_h x[t, h] * w_router[e, h] + bias[e]       (fp32 accumulate)
 *   S_t     = top_k experts by l[t, :], ties -> lower e
 *   topk_w  = softmax over ALL E of l[t, :], taken at S_t; divided by its
 *             sum over S_t when norm_topk
 *
 * x [T, H] and w_router [E, H] in desc->dtype; bias [E] fp32 or NULL.
 * Writes every field of *out.  workspace: moe_route_workspace_size(d, T).
 */
moe_status moe_route(const moe_desc *d, int32_t T, const void *x, const void *w_router,
                     const float *bias, const moe_routing *out, void *workspace,
                     size_t workspace_bytes, hipStream_t stream);

/*
 * moe_route_roster -- moe_route with the roster rule of the page "Predatory
 * MoE: Serving Mixture-of-Experts with a Sequence-Local Expert Roster"
 * (technical summary, section 2, the roster routing rule), for decode
 * batches where row t is one sequence.
 *
 *   usage [T, E] int32, in/out: how often sequence t has selected expert e
 *       at this layer so far (negative entries read as 0).  The caller keeps
 *       one array per layer and zeroes a row when its slot takes a new
 *       sequence.  Every selection of this call adds one (all phases).
 *   R_t  = the roster_size most-used experts of row t (ties -> lower e).
 *   bias added to l[t, :] before the softmax and the top-k:
 *       pinned[t] != 0                      0 on R_t, -inf elsewhere
 *       fewer than roster_size used so far  0 (exploration)
 *       otherwise                           +delta on R_t, -delta elsewhere
 *   So a non-member is chosen over a member only if its logit is higher by
 *   more than 2 delta, and it displaces the least-used member once its
 *   usage passes that member's.
 * pinned: [T] int32 or NULL (no row pinned).  1 <= roster_size <= E, and
 * roster_size >= top_k when pinned is given; delta finite and >= 0; else
 * MOE_ERR_INVALID_ARG.  usage NULL -> MOE_ERR_INVALID_ARG.  Other
 * arguments, outputs and workspace as moe_route.  Selection costs
 * roster_size extra wavefront max rounds per token.
 */
moe_status moe_route_roster(const moe_desc *d, int32_t T, const void *x, const void *w_router,
                            const float *bias, int32_t *usage, const int32_t *pinned,
                            int32_t roster_size, float delta, const moe_routing *out,
                            void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_expert_ffn_sparse -- the expert FFN with intra-expert activation
 * sparsity, for the small-batch path.
 *
 * For every pair (t, e) of `routing` (or, with routing == NULL, every token
 * with every expert of the group at weight 1, as for always-on shared
 * experts):
 *   h   = silu(W_g^e x_t) * (W_u^e x_t)         dense, fp32   (page: technical
 *         summary, Methodology: vLLM implementation, gate projection run
 *         densely to give activation scores)
 *   K   = the k_keep neurons of largest |h|, ties -> lower index (page:
 *         activation masking, a single O(n) pass with no sort; here an exact
 *         radix select of the k-th |h| then one threshold pass)
 *   y_t (+)= w_te * sum_{j in K} h_j * W_d^e[j, :]  only the kept rows of
 *         W_d are read (page: "how it runs: skip-list system", unneeded
 *         neurons are never loaded; fused up-down projection gathers only
 *         the active neurons' weights)
 * y [T, H] fp32 is overwritten (accumulate == 0) or added to (== 1); the sum
 * over a token's experts runs in slot order with no atomics, so results are
 * bitwise reproducible.
 * Where the experts of a bf16 call hold many tokens on average (n = T * top_k
 * / min(E, T * top_k) routed, T for a shared group: n >= 8, 32 or 128 as the
 * expected active experts' W_d is >= 512 MB, >= 128 MB or smaller), the down
 * projection takes the page's packed-rows form: each active expert's union
 * of kept rows is read once and multiplied with all of its tokens (MFMA),
 * the weighted activations rounded to bf16 for that product (fp32
 * accumulation); rows outside the union are still never read.  Otherwise
 * each token's kept rows are multiplied with its fp32 activations.
 *
 * k_keep in [0, d_ff]; k_keep == d_ff keeps every neuron, 0 adds nothing.
 * x [T, H] and w_down [E, d_ff, H] in desc->dtype; w_gate and w_up the
 * same tensors packed by moe_pack_gate_up.
 * active_idx_out: optional [T * top_k, k_keep] int32, the kept neuron ids of
 * each pair in ascending order (NULL to skip).
 * workspace: moe_ffn_workspace_size(d, T, k_keep, MOE_PATH_SPARSE).
 */
moe_status moe_expert_ffn_sparse(const moe_desc *d, int32_t T, int32_t k_keep, const void *x,
                                 const void *w_gate, const void *w_up, const void *w_down,
                                 const moe_routing *routing, float *y, int32_t accumulate,
                                 int32_t *active_idx_out, void *workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * moe_expert_ffn_sparse_residual -- moe_expert_ffn_sparse followed by the
 * residual stream of a decode step (as moe_residual_add), fused into the
 * down projection's epilogue: once a y element is final, the block that
 * wrote it also writes x_next[t, h] = x_res[t, h] + y[t, h], summed in fp32
 * and rounded to desc->dtype (round to nearest even for bf16).  One launch
 * fewer per layer; the results equal moe_expert_ffn_sparse then
 * moe_residual_add bit for bit.  It must be a layer's last FFN call (after
 * any routed call whose output it accumulates onto): no later call may read
 * x if x_next aliases it.  x_res and x_next [T, H] in desc->dtype, 16-byte
 * aligned, non-NULL when T > 0 (else MOE_ERR_INVALID_ARG /
 * MOE_ERR_MISALIGNED); x_next may be x_res or x.  Other arguments, outputs,
 * workspace and errors as moe_expert_ffn_sparse.  With k_keep == 0 the
 * residual runs as its own pass.
 */
moe_status moe_expert_ffn_sparse_residual(const moe_desc *d, int32_t T, int32_t k_keep,
                                          const void *x, const void *w_gate, const void *w_up,
                                          const void *w_down, const moe_routing *routing,
                                          float *y, int32_t accumulate, int32_t *active_idx_out,
                                          const void *x_res, void *x_next, void *workspace,
                                          size_t workspace_bytes, hipStream_t stream);

/*
 * moe_layer_sparse -- a whole routed layer in one call: moe_route (no bias
 * roster) then moe_expert_ffn_sparse, or moe_expert_ffn_sparse_residual
 * when x_res and x_next are given (both or neither; then the layer's last
 * FFN call), with the same outputs bit for bit (routing_out filled as
 * moe_route fills it, y as the FFN call writes it).
 * Up to 2 tokens (E <= 256, top_k <= 16, k_keep > 0) the gate/up blocks
 * repeat the router's top-k selection on the logits (one wave per token)
 * and each takes its own expert, so the select-and-group launch goes away
 * (three kernels instead of four; the page
 * asks its integration to work with kernel fusion and graph capture:
 * technical summary, Key contributions); other calls run the two calls'
 * kernels in turn.  Arguments as moe_route and moe_expert_ffn_sparse; one
 * workspace of moe_layer_workspace_size(d, T, k_keep) bytes.  Every
 * argument is checked before anything is enqueued.
 */
moe_status moe_layer_sparse(const moe_desc *d, int32_t T, int32_t k_keep, const void *x,
                            const void *w_router, const float *bias, const void *w_gate,
                            const void *w_up, const void *w_down, const moe_routing *routing_out,
                            float *y, int32_t accumulate, int32_t *active_idx_out,
                            const void *x_res, void *x_next, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);

/* Workspace bytes for moe_layer_sparse over at most T tokens with this
 * k_keep (0 on invalid input). */
size_t moe_layer_workspace_size(const moe_desc *d, int32_t T, int32_t k_keep);

/*
 * moe_layer_sparse_noalloc -- moe_layer_sparse for callers that cannot
 * allocate: code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc.  Same arguments, outputs and bits as
 * moe_layer_sparse, without the workspace arguments: the workspace is a
 * static array of MOE_NOALLOC_SCRATCH_BYTES in the library's device code,
 * one per GPU, held until the process ends.  Nothing is allocated (no
 * hipMalloc, hipFree or allocating library routine); the first call on a
 * device looks the array's device address up once.  A call whose
 * moe_layer_workspace_size(d, T, k_keep) exceeds MOE_NOALLOC_SCRATCH_BYTES
 * returns MOE_ERR_WORKSPACE with nothing enqueued (use moe_layer_sparse
 * with a caller workspace then).  Every call on a GPU shares that GPU's
 * array and the array keeps the last call's contents (nothing in it must
 * start at zero): calls that overlap on one GPU (different streams, or
 * different host threads without ordering) race and must not be issued.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)
moe_status moe_layer_sparse_noalloc(const moe_desc *d, int32_t T, int32_t k_keep, const void *x,
                                    const void *w_router, const float *bias, const void *w_gate,
                                    const void *w_up, const void *w_down,
                                    const moe_routing *routing_out, float *y, int32_t accumulate,
                                    int32_t *active_idx_out, const void *x_res, void *x_next,
                                    hipStream_t stream);

/*
 * moe_expert_ffn_dense -- the same layer function on the dense path the
 * page switches to at large batch (technical summary, Methodology: dynamic
 * switch between sparse and dense code paths by batch size).  Gate/up and
 * down run as grouped MFMA GEMMs over every row of each active expert; the
 * k_keep mask is applied to h in between, so the result equals
 * moe_expert_ffn_sparse's up to fp32 rounding order (bf16: h is rounded to
 * bf16 for the down GEMM).  k_keep == d_ff is the plain dense MoE.
 * w_down: row-major, or (bf16, desc->down_layout = MOE_LAYOUT_PACKED) the
 * copy moe_pack_down makes, which the down GEMM streams without staging
 * the weights through LDS.
 * Parameters as moe_expert_ffn_sparse;
 * workspace: moe_ffn_workspace_size(d, T, k_keep, MOE_PATH_DENSE).
 */
moe_status moe_expert_ffn_dense(const moe_desc *d, int32_t T, int32_t k_keep, const void *x,
                                const void *w_gate, const void *w_up, const void *w_down,
                                const moe_routing *routing, float *y, int32_t accumulate,
                                int32_t *active_idx_out, void *workspace,
                                size_t workspace_bytes, hipStream_t stream);

/*
 * moe_expert_ffn_sparse_updown -- the page's own split of the sparse path
 * (technical summary, Methodology, vLLM implementation: the gate projection
 * alone runs densely and yields the activation scores; the fused up-down
 * projection gathers only the active neurons' weights):
 *
 *   s      = silu(W_g^e x_t)                     dense, every pair
 *   K      = the k_keep neurons of largest |s_j| (ties: lower j)
 *   h_j    = s_j * (W_u^e[j, :] . x_t)            j in K only
 *   y_t   (+)= sum over the token's experts (slot order) of w * sum_{j in K} h_j W_d^e[j, :]
 *
 * A different mask from moe_expert_ffn_sparse's (which scores |silu(g) * u|
 * with gate and up both dense); with k_keep == d_ff both are the dense
 * SwiGLU MoE.  Reads half the dense bytes of moe_expert_ffn_sparse plus the
 * kept up rows.  Layouts differ in one place: w_gate is packed by
 * moe_pack_gate_up, but w_up is the plain [E, d_ff, H] neuron-major tensor
 * (like w_down), since its kept rows are gathered.  Other parameters,
 * outputs and errors as moe_expert_ffn_sparse (active_idx_out: the kept ids
 * by gate score); workspace: moe_ffn_workspace_size(d, T, k_keep,
 * MOE_PATH_SPARSE).  There is no dense form of this variant.
 */
moe_status moe_expert_ffn_sparse_updown(const moe_desc *d, int32_t T, int32_t k_keep,
                                        const void *x, const void *w_gate, const void *w_up,
                                        const void *w_down, const moe_routing *routing, float *y,
                                        int32_t accumulate, int32_t *active_idx_out,
                                        void *workspace, size_t workspace_bytes,
                                        hipStream_t stream);

/*
 * moe_pack_gate_up -- rearrange one gate or up tensor [E, d_ff, H] from
 * row-major into the packed layout the FFN calls read: for each expert e,
 * neuron tile nt (16 neurons) and k-step ks (KS = 32 bf16 or 16 fp32
 * columns), one contiguous 1 KB fragment holds W[e, 16 nt + r, KS ks + c]
 * at element offset (r + 16 * (c / (KS/4))) * (KS/4) + c % (KS/4), for
 * r < 16, c < KS; fragment index (e * d_ff/16 + nt) * (H/KS) + ks.  So a
 * wave loads one MFMA operand fragment as 1 KB of consecutive bytes.  Only
 * 16-byte chunks move, so packing is exact.  src and dst must not overlap;
 * both are E * d_ff * H elements of desc->dtype.  moe_unpack_gate_up is the
 * inverse.
 */
moe_status moe_pack_gate_up(const moe_desc *d, const void *src_rowmajor, void *dst_packed,
                            hipStream_t stream);
moe_status moe_unpack_gate_up(const moe_desc *d, const void *src_packed, void *dst_rowmajor,
                              hipStream_t stream);

/*
 * moe_pack_down -- a copy of a bf16 down tensor [E, d_ff, H] in the layout
 * moe_expert_ffn_dense reads with desc->down_layout = MOE_LAYOUT_PACKED: W_d
 * transposed into MFMA operand fragments, so the dense down GEMM streams its
 * weights as the gate/up GEMM does (page: technical summary, Methodology,
 * the dense path at large batch).  For each expert e, column tile ct (16
 * columns of H) and k-step ks (32 rows of d_ff), one contiguous 1 KB
 * fragment holds W_d[e, 32 ks + 8 g + i, 16 ct + r] at element offset
 * 8 (r + 16 g) + i, for r < 16, g < 4, i < 8; fragment index
 * (e * H/16 + ct) * (d_ff/32) + ks.  The sparse calls need the row-major
 * tensor (they read kept rows), so a caller using both paths keeps both
 * copies.  Exact (bits are copied).  bf16 only (else MOE_ERR_UNSUPPORTED);
 * src and dst must not overlap; both E * d_ff * H elements.
 * moe_unpack_down is the inverse.
 */
moe_status moe_pack_down(const moe_desc *d, const void *src_rowmajor, void *dst_packed,
                         hipStream_t stream);
moe_status moe_unpack_down(const moe_desc *d, const void *src_packed, void *dst_rowmajor,
                           hipStream_t stream);

/*
 * moe_expert_ffn_sparse_threshold -- the sparse path with the page's literal
 * masking (technical summary, Methodology: activation masking by a
 * threshold in one O(n) pass, without a top-k sort): neuron j of pair
 * (t, e) is kept iff |h_j| > tau[e], with h = silu(W_g x) * (W_u x) as in
 * moe_expert_ffn_sparse, so the kept count varies per pair.  tau [E] fp32
 * device thresholds, e.g. from moe_calibrate_thresholds; tau[e] < 0 keeps
 * every neuron of expert e.
 * counts_out: optional [T * top_k] int32, kept count of each pair;
 * active_idx_out: optional [T * top_k, d_ff] int32, the first counts_out[p]
 * entries of row p are pair p's kept ids, ascending.  Other parameters,
 * outputs and errors as moe_expert_ffn_sparse (no k_keep); d_ff up to 2048
 * (a multiple of 64) or a multiple of 512 up to 8192, else
 * MOE_ERR_UNSUPPORTED.  workspace: moe_ffn_threshold_workspace_size(d, T).
 */
moe_status moe_expert_ffn_sparse_threshold(const moe_desc *d, int32_t T, const float *tau,
                                           const void *x, const void *w_gate, const void *w_up,
                                           const void *w_down, const moe_routing *routing,
                                           float *y, int32_t accumulate, int32_t *counts_out,
                                           int32_t *active_idx_out, void *workspace,
                                           size_t workspace_bytes, hipStream_t stream);

/*
 * moe_calibrate_thresholds -- offline calibration of the thresholds for a
 * target sparsity s.  The page masks by a threshold (technical summary,
 * Methodology: activation masking) but does not say how it is chosen; this
 * per-expert order statistic of calibration scores is the reading taken.
 * On T calibration tokens x with their routing (from moe_route; NULL for
 * the always-on group, top_k == n_experts), with the scores
 * |h| = |silu(W_g x) * (W_u x)| of every (calibration pair, neuron):
 *   tau[e] = the (c + 1)-th largest of expert e's m scores, c = ceil((1 - s) m),
 *            or -1 when c = m (keep everything);
 *   an expert that no calibration token reaches gets the same statistic
 *   over all routed scores.
 * So 'keep |h| > tau[e]' keeps exactly c of expert e's m calibration scores
 * when they are distinct.  w_gate and w_up packed (moe_pack_gate_up);
 * tau_out [E] fp32 device.  d_ff as moe_expert_ffn_sparse_threshold.
 * Errors: sparsity outside [0, 1] (or NaN), tau_out NULL ->
 * MOE_ERR_INVALID_ARG; T * top_k * d_ff >= 2^31 -> MOE_ERR_UNSUPPORTED
 * (calibrate on fewer tokens).  T == 0 leaves tau_out untouched.
 * workspace: moe_calibrate_workspace_size(d, T).
 */
moe_status moe_calibrate_thresholds(const moe_desc *d, int32_t T, const void *x,
                                    const void *w_gate, const void *w_up,
                                    const moe_routing *routing, double sparsity, float *tau_out,
                                    void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * moe_expert_ffn_sparse_updown_threshold -- the page's own pipeline with its
 * threshold mask (technical summary, Methodology: the gate projection runs
 * densely and gives the activation scores, a single-pass threshold mask
 * replaces the top-k sort, and the fused up-down projection gathers only
 * the active neurons' weights): per pair (t, e), s = silu(W_g x) densely,
 * neuron j kept iff |s_j| > tau[e] (tau[e] < 0 keeps all), and for kept j
 * only h_j = s_j * (W_u[j] . x), then the sparse down projection of
 * moe_expert_ffn_sparse.  w_gate packed (moe_pack_gate_up), w_up and w_down
 * row-major.  tau [E] fp32 device, e.g. from moe_calibrate_thresholds_gate.
 * counts_out, active_idx_out, workspace (moe_ffn_threshold_workspace_size),
 * outputs and errors as moe_expert_ffn_sparse_threshold.
 */
moe_status moe_expert_ffn_sparse_updown_threshold(const moe_desc *d, int32_t T, const float *tau,
                                                  const void *x, const void *w_gate,
                                                  const void *w_up, const void *w_down,
                                                  const moe_routing *routing, float *y,
                                                  int32_t accumulate, int32_t *counts_out,
                                                  int32_t *active_idx_out, void *workspace,
                                                  size_t workspace_bytes, hipStream_t stream);

/*
 * moe_calibrate_thresholds_gate -- moe_calibrate_thresholds on the split's
 * scores |silu(W_g x)| (no up projection is run or needed), for
 * moe_expert_ffn_sparse_updown_threshold.  Arguments, workspace
 * (moe_calibrate_workspace_size) and errors as moe_calibrate_thresholds
 * without w_up.
 */
moe_status moe_calibrate_thresholds_gate(const moe_desc *d, int32_t T, const void *x,
                                         const void *w_gate, const moe_routing *routing,
                                         double sparsity, float *tau_out, void *workspace,
                                         size_t workspace_bytes, hipStream_t stream);

/*
 * moe_residual_add -- the residual stream between the layers of a decode
 * step: x_out[t, h] = x_in[t, h] + y[t, h], rounded to desc->dtype (round to
 * nearest even for bf16; finite values).  x_in, x_out [T, H] in desc->dtype,
 * y [T, H] fp32 (a layer call's output); all 16-byte aligned; x_out may be
 * x_in.  Not part of the MoE layer itself: with it a multi-layer decode step
 * runs, and can be captured as one HIP graph, entirely in this library's
 * kernels (the intra-expert page requires graph compatibility of its
 * integration: technical summary, Key contributions).  Errors as for the
 * other calls.
 */
moe_status moe_residual_add(const moe_desc *d, int32_t T, const void *x_in, const float *y,
                            void *x_out, hipStream_t stream);

/* Workspace bytes for moe_route over at most T tokens (0 on invalid input). */
size_t moe_route_workspace_size(const moe_desc *d, int32_t T);

/* Workspace bytes for an FFN call over at most T tokens with this k_keep and
 * path (0 on invalid input).  A workspace sized for (T, k_keep) serves any
 * call with fewer tokens and the same k_keep. */
size_t moe_ffn_workspace_size(const moe_desc *d, int32_t T, int32_t k_keep, moe_path path);

/* Workspace bytes for moe_expert_ffn_sparse_threshold and for
 * moe_calibrate_thresholds over at most T tokens (0 on invalid input). */
size_t moe_ffn_threshold_workspace_size(const moe_desc *d, int32_t T);
size_t moe_calibrate_workspace_size(const moe_desc *d, int32_t T);

/* One workspace size for a whole layer over at most T_max tokens: enough
 * for moe_route, for the FFN call on `path` with this k_keep, and (sparse
 * path) for moe_layer_sparse, so one buffer serves every call of the layer
 * in turn (0 on invalid input). */
size_t moe_workspace_size(const moe_desc *d, int32_t T_max, int32_t k_keep, moe_path path);

/* Kept neurons per (token, expert) at sparsity s: ceil((1 - s) * d_ff).  The
 * page zeroes the lowest-scoring fraction of each selected expert's neurons
 * (technical summary, Methodology: empirical analysis; Results: the
 * sparsity levels that keep 95 % of the baseline accuracy), so s is the
 * fraction zeroed and the rest is kept, rounded up.  Computed as
 * ceil((1 - s) * d_ff - 1e-9) so that exact products do not round up,
 * clamped to [0, d_ff]; -1 if d_ff < 0 or s is not finite. */
int32_t moe_keep_count(double sparsity, int32_t d_ff);

/* Host-side, shape-only choice between the sparse and dense paths for T
 * tokens at this k_keep (the page's batch-size switch; technical summary,
 * Methodology: dynamic switching by batch size).  It compares the down
 * projection's cost under uniform routing: the sparse path's per-pair rows,
 * with rows repeated among an expert's tokens costed at 0.3 (served by the
 * caches), against 1.2 x every row of the active experts for the dense
 * GEMM; k_keep == d_ff always takes the dense path.  The constants fit the
 * measured sweeps of four layer families.  Call it per expert group (routed
 * and shared separately).  Never reads device memory; safe during graph
 * capture.  Returns MOE_PATH_SPARSE on invalid input.
 * MOE_FORCE_PATH=sparse|dense in the environment overrides it. */
moe_path moe_select_path(const moe_desc *d, int32_t T, int32_t k_keep);

/*
 * Measurement hook (not part of the layer's function).  Kernel stages the
 * library launches: */
typedef enum {
  MOE_STAGE_ROUTER_LOGITS = 0,
  MOE_STAGE_ROUTER_TOPK = 1,
  MOE_STAGE_ROUTE_GROUP = 2,
  MOE_STAGE_GATEUP = 3,
  MOE_STAGE_NEURON_MASK = 4,
  MOE_STAGE_DOWN_ROWS = 5,
  MOE_STAGE_DOWN_DENSE = 6,
  MOE_STAGE_COMBINE = 7,
  MOE_STAGE_ZERO = 8,
  MOE_STAGE_UP_ROWS = 9,
  MOE_STAGE_FUSED_FFN = 10, /* gate/up, masks, down and combine in one launch */
  MOE_STAGE_UNION_ROWS = 11, /* per-expert union of kept rows + its coefficients */
  MOE_STAGE_DOWN_UNION = 12, /* down product over each expert's union of rows   */
  MOE_N_STAGES = 13
} moe_stage;

/* While attached, every kernel the library launches from this thread is
 * bracketed by two caller-created timing events recorded on its launch
 * stream: the i-th launch records events[2i] before and events[2i+1] after
 * itself and writes its moe_stage to stages[i]; once `capacity` launches are
 * recorded, further launches are not bracketed.  events: 2 * capacity
 * caller-owned hipEvent_t (host array); stages: capacity int32 (host).
 * Nothing is allocated.  Recording adds a marker per launch to the stream,
 * so time the layer without the hook attached. */
moe_status moe_timer_attach(hipEvent_t *events, int32_t *stages, int32_t capacity);
/* Detach; returns the number of launches recorded since attaching. */
int32_t moe_timer_detach(void);

/* Measurement helper, not part of the layer: one plain streaming read of
 * `bytes` of device memory at `src` (16-byte aligned, bytes a positive
 * multiple of 16), with non-temporal 16-byte loads in blocks of 256
 * threads: about 8 loads per thread, at least 1024 and at most 16384
 * blocks, so any size has its loads in flight at once.  Timing it gives the
 * practical HBM read rate, at 4 GiB or at a kernel's own size, that the
 * layer's kernels are compared with.  Block b writes the XOR of its chunks to
 * sink[4b .. 4b+3]: `sink` holds MOE_STREAM_READ_SINK_WORDS uint32 of device
 * memory.  Errors as for the other calls; nothing is allocated. */
#define MOE_STREAM_READ_SINK_WORDS 65536
moe_status moe_stream_read(const void *src, size_t bytes, uint32_t *sink, hipStream_t stream);

/* Static name of a status code. */
const char *moe_status_string(moe_status s);

/* Detail of the last error returned on this thread ("" if none). */
const char *moe_last_error(void);

/* Library version string. */
const char *moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
