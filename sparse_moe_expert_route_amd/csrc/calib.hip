// Measurement helper: a plain streaming read of a device buffer, the
// practical HBM read peak that the kernels' bandwidth is compared with.
#include "device_common.h"
#include "internal.h"

namespace moe {

// Every thread XOR-folds 16-byte chunks of its grid-stride share, 8 loads in
// flight, with the non-temporal hint (each byte is read once); block b
// writes the fold of its 256 threads to sink[4 b .. 4 b + 3].
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ src,
                                                          size_t n_chunks,
                                                          uint32_t *__restrict__ sink) {
  __shared__ u32x4 red[256];
  const size_t stride = (size_t)gridDim.x * 256;
  size_t c = (size_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = u32x4{0, 0, 0, 0};
  constexpr int U = 8;
  for (; c + (U - 1) * stride < n_chunks; c += U * stride) {
    u32x4 q[U];
#pragma unroll
    for (int u = 0; u < U; ++u) q[u] = ld16_nt(src + c + u * stride);
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= q[u];
  }
  {  // the rest: fewer than U chunks of this thread, all loads in flight
    u32x4 q[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      q[u] = c + u * stride < n_chunks ? ld16_nt(src + c + u * stride) : u32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < U; ++u) acc ^= q[u];
  }
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x < 4) sink[4 * blockIdx.x + threadIdx.x] = red[0][threadIdx.x];
}

// Grid sized to the read: about U chunks per thread (one unrolled round),
// at least 1024 blocks (4 per CU, so even a few MB has every CU's loads in
// flight at once) and at most max_blocks.
hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, int max_blocks,
                              hipStream_t stream) {
  const size_t n = bytes / 16, per_block = 8 * 256;
  size_t blocks = (n + per_block - 1) / per_block;
  blocks = blocks < 1024 ? 1024 : blocks;
  blocks = blocks > (size_t)max_blocks ? (size_t)max_blocks : blocks;
  stream_read_kernel<<<(unsigned)blocks, 256, 0, stream>>>(static_cast<const u32x4 *>(src), n, sink);
  return hipGetLastError();
}

}  // namespace moe
