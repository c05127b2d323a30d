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
  for (; c < n_chunks; c += stride) acc ^= ld16_nt(src + c);
  red[threadIdx.x] = acc;
  __syncthreads();
  for (int s = 128; s > 0; s >>= 1) {
    if ((int)threadIdx.x < s) red[threadIdx.x] ^= red[threadIdx.x + s];
    __syncthreads();
  }
  if (threadIdx.x < 4) sink[4 * blockIdx.x + threadIdx.x] = red[0][threadIdx.x];
}

hipError_t launch_stream_read(const void *src, size_t bytes, uint32_t *sink, int blocks,
                              hipStream_t stream) {
  stream_read_kernel<<<blocks, 256, 0, stream>>>(static_cast<const u32x4 *>(src), bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace moe
