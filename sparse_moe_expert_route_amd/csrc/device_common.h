// Device-side building blocks shared by the gfx950 kernels of the MoE layer:
// vector types, bf16 handling, MFMA wrappers, the routing view and
// wavefront/block scans.  gfx950 (CDNA4): wave64, 16x16 MFMA tiles.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// One 16-byte global load (dwordx4).
__device__ __forceinline__ u32x4 ld16(const void *p) {
  return *reinterpret_cast<const u32x4 *>(p);
}

// 16-byte load with the non-temporal (streaming) hint: for weight streams
// that are read exactly once per call.
__device__ __forceinline__ u32x4 ld16_nt(const void *p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4 *>(p));
}

// Raw buffer resource over [p, p + bytes): stride 0, byte offsets, the
// gfx9 data-format word.  Callers keep every load inside the range.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)bytes, 0x00020000);
}
// 16 bytes at voff + soff of the resource (soff wave-uniform); _nt with
// the non-temporal hint, as ld16_nt.
__device__ __forceinline__ u32x4 buf_ld16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 0));
}
__device__ __forceinline__ u32x4 buf_ld16_nt(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 2));
}

// ---- device-coherent (agent-scope) accesses, for data handed between
// blocks inside one kernel.  Each XCD has its own L2 and they are not kept
// coherent with one another: a plain store may sit in the writer's L2 and a
// plain load may hit a stale line in the reader's.  Agent-scope accesses
// carry the sc1 bit (write through / read past the non-coherent L2), and
// the writer waits for its stores to complete (wait_stores) before it
// signals with an atomic; read-modify-write atomics are device-coherent as
// issued.  No release/acquire fence is used: on this chip each one writes
// back or invalidates the whole L2 of the XCD, serialised per block.
__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }
__device__ __forceinline__ void compiler_barrier() { asm volatile("" ::: "memory"); }
__device__ __forceinline__ void st_agent(float *p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent(const float *p) {
  return __hip_atomic_load(const_cast<float *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int ld_agent(const int32_t *p) {
  return __hip_atomic_load(const_cast<int32_t *>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_agent(int32_t *p, int32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// 16 bytes at voff + soff of a buffer resource, read coherently (sc1)
__device__ __forceinline__ u32x4 buf_ld16_agent(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, 16));
}

// Bounded wait (one lane): until *cnt >= target.  Gives up after about one
// second of the 100 MHz real-time counter or once another block has given
// up (*abort != 0), sets *abort and returns false; a wait that cannot be
// satisfied therefore ends the kernel with wrong outputs, never a hang.
// Polls back off from ~0.1 to ~1.5 us apart, so that many waiting blocks
// do not crowd the memory channel of the polled line.
__device__ __forceinline__ bool wait_count(const int32_t *cnt, int target, int32_t *abort) {
  if (ld_agent(cnt) >= target) return true;
  const uint64_t t0 = wall_clock64();
  for (uint32_t it = 0;; ++it) {
    if (it < 4) __builtin_amdgcn_s_sleep(4);
    else if (it < 12) __builtin_amdgcn_s_sleep(16);
    else __builtin_amdgcn_s_sleep(56);
    if (ld_agent(cnt) >= target) return true;
    if (ld_agent(abort) != 0) return false;
    if (wall_clock64() - t0 > 100000000ull || it > (1u << 26)) {
      st_agent(abort, 1);
      return false;
    }
  }
}

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// D += A * B for a 16x16 output tile, K = 32 bf16.  Lane l supplies row
// (l % 16) of A and column (l % 16) of B, each with the 8 consecutive k of
// k-group (l / 16); it receives D rows 4 * (l / 16) + r, column l % 16.
__device__ __forceinline__ f32x4 mfma_bf16(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(a), as_bf16x8(b), c, 0, 0, 0);
}

// Same tile shape with fp32 operands and K = 4: lane l supplies A[l % 16][l / 16]
// and B[l / 16][l % 16].
__device__ __forceinline__ f32x4 mfma_f32(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Routing of one FFN call as the kernels see it.  `implicit` is the
// always-on (shared) group: every token pairs with every expert, weight 1,
// pair p = t * E + e, and expert e's tokens sit at positions [e*T, (e+1)*T).
struct RouteView {
  const int32_t *topk_ids;
  const float *topk_w;
  const int32_t *offsets;
  const int32_t *pair_by_expert;
  const int32_t *active;
  const int32_t *n_active;
  int32_t implicit;
  int32_t T;
  int32_t top_k;
  int32_t E;

  __device__ __forceinline__ int nact() const { return implicit ? E : *n_active; }
  __device__ __forceinline__ int expert(int s) const { return implicit ? s : active[s]; }
  __device__ __forceinline__ int begin(int e) const { return implicit ? e * T : offsets[e]; }
  __device__ __forceinline__ int end(int e) const { return implicit ? (e + 1) * T : offsets[e + 1]; }
  __device__ __forceinline__ int pair_at(int q) const {
    return implicit ? (q % T) * top_k + q / T : pair_by_expert[q];
  }
  __device__ __forceinline__ int expert_of_pair(int p) const {
    return implicit ? p % top_k : topk_ids[p];
  }
  __device__ __forceinline__ float weight(int p) const { return implicit ? 1.0f : topk_w[p]; }
};

// ---- wavefront reductions and scans
// Built on DPP row shifts and row broadcasts (register-to-register, no LDS
// round trip): row_shr:1,2,4,8 scan each row of 16 lanes, row_bcast:15 and
// row_bcast:31 carry row totals into the following rows.  Every caller runs
// them with all 64 lanes active.  The order of operations is fixed, so the
// results are deterministic.

template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ int dpp(int v) {
  return __builtin_amdgcn_update_dpp(0, v, CTRL, ROW_MASK, 0xf, BOUND_ZERO);
}
constexpr int kShr1 = 0x111, kShr2 = 0x112, kShr4 = 0x114, kShr8 = 0x118;
constexpr int kBcast15 = 0x142, kBcast31 = 0x143;

// Inclusive prefix sum over the lanes of a wave.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += dpp<kShr1, 0xf, true>(v);
  v += dpp<kShr2, 0xf, true>(v);
  v += dpp<kShr4, 0xf, true>(v);
  v += dpp<kShr8, 0xf, true>(v);
  v += dpp<kBcast15, 0xa, false>(v);
  v += dpp<kBcast31, 0xc, false>(v);
  return v;
}

__device__ __forceinline__ int lane_value(int v, int lane) {
  return __builtin_amdgcn_readlane(v, lane);
}

__device__ __forceinline__ float wave_sum(float v) {
#define MOE_FADD(C, M, B) v += __int_as_float(dpp<C, M, B>(__float_as_int(v)))
  MOE_FADD(kShr1, 0xf, true);
  MOE_FADD(kShr2, 0xf, true);
  MOE_FADD(kShr4, 0xf, true);
  MOE_FADD(kShr8, 0xf, true);
  MOE_FADD(kBcast15, 0xa, false);
  MOE_FADD(kBcast31, 0xc, false);
#undef MOE_FADD
  return __int_as_float(lane_value(__float_as_int(v), 63));
}

__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
#define MOE_UMAX(C, M, B) v = max(v, (uint32_t)dpp<C, M, B>((int)v))
  MOE_UMAX(kShr1, 0xf, true);
  MOE_UMAX(kShr2, 0xf, true);
  MOE_UMAX(kShr4, 0xf, true);
  MOE_UMAX(kShr8, 0xf, true);
  MOE_UMAX(kBcast15, 0xa, false);
  MOE_UMAX(kBcast31, 0xc, false);
#undef MOE_UMAX
  return (uint32_t)lane_value((int)v, 63);
}

// Maximum 64-bit key over the wave: the high words first, then the low
// words among the lanes that hold the maximal high word.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  const uint32_t hi = (uint32_t)(v >> 32), lo = (uint32_t)v;
  const uint32_t mh = wave_max_u32(hi);
  const uint32_t ml = wave_max_u32(hi == mh ? lo : 0u);
  return ((uint64_t)mh << 32) | ml;
}

// Inclusive prefix sum over a whole block of NT threads (NT/64 <= 64 waves).
// `tmp` is __shared__ scratch of at least NT/64 ints.  Ends with a barrier.
template <int NT>
__device__ __forceinline__ int block_incl_scan(int v, int *tmp, int *total = nullptr) {
  constexpr int NW = NT / kWave;
  const int lane = threadIdx.x & (kWave - 1);
  const int wid = threadIdx.x / kWave;
  int s = wave_incl_scan(v);
  if (lane == kWave - 1) tmp[wid] = s;
  __syncthreads();
  if (wid == 0) {
    int t = lane < NW ? tmp[lane] : 0;
    t = wave_incl_scan(t);
    if (lane < NW) tmp[lane] = t;
  }
  __syncthreads();
  if (wid > 0) s += tmp[wid - 1];
  if (total) *total = tmp[NW - 1];
  __syncthreads();
  return s;
}

// Order-preserving map of a float to uint32 (larger float -> larger key);
// -0 is folded onto +0 first.
__device__ __forceinline__ uint32_t ordered_key(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) == 0u) u = 0u;
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Inverse of ordered_key on the upper 32 bits of a 64-bit selection key.
__device__ __forceinline__ float key_value(uint64_t key) {
  const uint32_t u = (uint32_t)(key >> 32);
  return __uint_as_float((u & 0x80000000u) ? (u & 0x7fffffffu) : ~u);
}

}  // namespace moe
