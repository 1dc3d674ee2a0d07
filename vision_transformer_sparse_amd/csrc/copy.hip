// A plain streaming copy (16 bytes per lane per step). It has no part in the
// attention computation: it is a kernel of exactly known traffic, used to
// calibrate hardware byte counters and to measure attainable HBM bandwidth.
#include "bra_internal.h"

namespace bra {
namespace {

__global__ __launch_bounds__(256) void copy_kernel(const uint4* __restrict__ src,
                                                   uint4* __restrict__ dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    dst[i] = src[i];
}

}  // namespace

hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 16;
  if (n == 0) return hipSuccess;
  size_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  launch(copy_kernel, dim3((unsigned)blocks), dim3(256), 0, st,
                     (const uint4*)src, (uint4*)dst, n);
  return hipGetLastError();
}

}  // namespace bra
