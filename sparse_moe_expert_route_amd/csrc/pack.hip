// Gate/up (and, for the dense path, down) weight packing into the MFMA
// fragment layout.
//
// The gate/up kernel consumes each expert's [d_ff, H] matrix as 16-neuron x
// KS-column MFMA A fragments (KS = 32 bf16 or 16 fp32 elements).  Stored
// row-major, one fragment is 16 separate 64-byte pieces; packed, it is one
// contiguous 1 KB block in exactly the order the 64 lanes of a wave load it
// (lane l = (j % 16) + 16 * group holds 16 bytes: neuron j, k-group `group`),
// so every load instruction of the weight stream reads 8 whole 128-byte
// lines.  Packing moves 16-byte chunks only, so it is exact for any dtype.
#include "device_common.h"
#include "internal.h"

namespace moe {

// Chunk c of the packed matrix (16 bytes) <- its source chunk in row-major.
__global__ __launch_bounds__(256) void pack_gate_up_kernel(const u32x4 *__restrict__ src,
                                                           u32x4 *__restrict__ dst, int E,
                                                           int d_ff, int H, int ks_elems,
                                                           int elem_bytes, int unpack) {
  const size_t n_chunks = (size_t)E * d_ff * H * elem_bytes / 16;
  const size_t c = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= n_chunks) return;
  const int lane = (int)(c & 63);
  const size_t frag = c >> 6;
  const int nsteps = H / ks_elems;
  const int ks = (int)(frag % nsteps);
  const size_t tile = frag / nsteps;  // e * (d_ff / 16) + neuron tile
  const int r = lane & 15, g = lane >> 4;
  const size_t row = tile * 16 + r;   // e * d_ff + neuron
  const size_t elem = row * H + (size_t)ks * ks_elems + g * (ks_elems / 4);
  const size_t s = elem * elem_bytes / 16;
  if (unpack)
    dst[s] = src[c];
  else
    dst[c] = src[s];
}

// Down weight packing for the dense path (bf16).  The dense down GEMM takes
// W_d^T as its MFMA A operand: 16 output columns x 32 k (d_ff) per fragment,
// lane l = r + 16 g holding column r, k = 8 g .. 8 g + 7.  Fragments are
// ordered (expert, column tile, k-step), so a wave streams one column
// tile's fragments as contiguous 1 KB blocks.  In row-major W_d [E, d_ff, H]
// a fragment chunk's 8 elements are one column of 8 consecutive rows, so
// each thread moves one chunk element by element; exact (bits are copied).
__global__ __launch_bounds__(256) void pack_down_kernel(const uint16_t *__restrict__ src,
                                                        uint16_t *__restrict__ dst, int E,
                                                        int d_ff, int H, int unpack) {
  const size_t n_chunks = (size_t)E * d_ff * H / 8;
  const size_t c = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (c >= n_chunks) return;
  const int lane = (int)(c & 63);
  const size_t frag = c >> 6;
  const int nsteps = d_ff / 32;
  const int ks = (int)(frag % nsteps);
  const size_t tile = frag / nsteps;  // e * (H / 16) + column tile
  const size_t ncol = (size_t)H / 16;
  const size_t e = tile / ncol, ct = tile - e * ncol;
  const int r = lane & 15, g = lane >> 4;
  const size_t col = ct * 16 + r;
  const size_t k = (size_t)ks * 32 + 8 * g;
  const size_t base = (e * d_ff + k) * H + col;  // element (k, col) of expert e
  if (unpack) {
    const u32x4 v = reinterpret_cast<const u32x4 *>(src)[c];
#pragma unroll
    for (int i = 0; i < 8; ++i) dst[base + (size_t)i * H] = (uint16_t)(v[i >> 1] >> (16 * (i & 1)));
  } else {
    u32x4 v;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      v[i] = (uint32_t)src[base + (size_t)(2 * i) * H] |
             ((uint32_t)src[base + (size_t)(2 * i + 1) * H] << 16);
    reinterpret_cast<u32x4 *>(dst)[c] = v;
  }
}

hipError_t launch_pack_down(const void *src, void *dst, int E, int d_ff, int H, int unpack,
                            hipStream_t stream) {
  const size_t n_chunks = (size_t)E * d_ff * H / 8;
  if (n_chunks == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n_chunks + 255) / 256);
  pack_down_kernel<<<blocks, 256, 0, stream>>>(static_cast<const uint16_t *>(src),
                                               static_cast<uint16_t *>(dst), E, d_ff, H, unpack);
  return hipGetLastError();
}

hipError_t launch_pack_gate_up(const void *src, void *dst, int E, int d_ff, int H, int bf16,
                               int unpack, hipStream_t stream) {
  const int eb = bf16 ? 2 : 4;
  const size_t n_chunks = (size_t)E * d_ff * H * eb / 16;
  if (n_chunks == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((n_chunks + 255) / 256);
  pack_gate_up_kernel<<<blocks, 256, 0, stream>>>(static_cast<const u32x4 *>(src),
                                                  static_cast<u32x4 *>(dst), E, d_ff, H,
                                                  bf16 ? 32 : 16, eb, unpack);
  return hipGetLastError();
}

}  // namespace moe
