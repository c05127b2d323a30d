// The residual stream between the MoE layers of a decode step.
//
// A decode step runs its layers in sequence; each MoE block's output y (fp32)
// is added to the block's input x and the sum, rounded to the layers' dtype,
// is the next layer's input.  One elementwise pass, HBM-bound and tiny at
// decode batches; it lets a whole multi-layer step be captured as one graph
// with every step in this library's kernels.
#include "device_common.h"
#include "internal.h"

namespace moe {

// Thread i handles elements [8 i, 8 i + 8): one 16-byte load of bf16 x (two
// of fp32 x), two of y, one or two stores.  x_in and x_out may alias.
template <bool BF16>
__global__ __launch_bounds__(256) void residual_kernel(const void *x_in, const float *__restrict__ y,
                                                       void *x_out, size_t n8) {
  const size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n8) return;
  const u32x4 y0 = ld16(y + 8 * i), y1 = ld16(y + 8 * i + 4);
  const float yv[8] = {__uint_as_float(y0[0]), __uint_as_float(y0[1]), __uint_as_float(y0[2]),
                       __uint_as_float(y0[3]), __uint_as_float(y1[0]), __uint_as_float(y1[1]),
                       __uint_as_float(y1[2]), __uint_as_float(y1[3])};
  if (BF16) {
    const u32x4 xv = ld16(static_cast<const uint16_t *>(x_in) + 8 * i);
    u32x4 o;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t lo = f32_to_bf16_bits(bf16lo(xv[j]) + yv[2 * j]);
      const uint32_t hi = f32_to_bf16_bits(bf16hi(xv[j]) + yv[2 * j + 1]);
      o[j] = lo | (hi << 16);
    }
    *reinterpret_cast<u32x4 *>(static_cast<uint16_t *>(x_out) + 8 * i) = o;
  } else {
    const float *xf = static_cast<const float *>(x_in) + 8 * i;
    const u32x4 a = ld16(xf), b = ld16(xf + 4);
    u32x4 oa, ob;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      oa[j] = __float_as_uint(__uint_as_float(a[j]) + yv[j]);
      ob[j] = __float_as_uint(__uint_as_float(b[j]) + yv[4 + j]);
    }
    float *of = static_cast<float *>(x_out) + 8 * i;
    *reinterpret_cast<u32x4 *>(of) = oa;
    *reinterpret_cast<u32x4 *>(of + 4) = ob;
  }
}

hipError_t launch_residual(const void *x_in, const float *y, void *x_out, size_t n, int bf16,
                           hipStream_t stream) {
  const size_t n8 = n / 8;
  const unsigned blocks = (unsigned)((n8 + 255) / 256);
  if (bf16) residual_kernel<true><<<blocks, 256, 0, stream>>>(x_in, y, x_out, n8);
  else residual_kernel<false><<<blocks, 256, 0, stream>>>(x_in, y, x_out, n8);
  return hipGetLastError();
}

}  // namespace moe
