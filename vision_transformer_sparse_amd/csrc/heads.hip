// Layout moves of the per-head routing variant (the qqiyuan.cn blog's BRA
// class routes each head on its own channels, section on region-level
// routing): the variant runs the operator once per head on that head's
// channels, so the heads are first copied out of the NHWC tensors into
// head-major ones ([heads][N][H][W][32]), and the per-head outputs and routes
// are put back into the caller's layouts afterwards. All moves are 16-byte
// pieces (a head's 32 channels are 4 pieces in bf16, 8 in fp32); each kernel
// walks its destination in order, so the writes are contiguous and the reads
// are whole 64- or 128-byte head slices.
#include "bra_internal.h"

namespace bra {
namespace {

constexpr int kMoveThreads = 256;
constexpr long long kMoveMaxBlocks = 8192;

// dst[h][t][sub] = src[t][h * ph + sub] (t over all N*H*W tokens)
__global__ __launch_bounds__(kMoveThreads) void head_split_kernel(const uint4* __restrict__ src,
                                                                  uint4* __restrict__ dst, long long tokens,
                                                                  int heads, int ph) {
  const long long total = tokens * heads * ph;
  for (long long e = (long long)blockIdx.x * kMoveThreads + threadIdx.x; e < total;
       e += (long long)gridDim.x * kMoveThreads) {
    const long long ht = e / ph;
    const int sub = (int)(e - ht * ph);
    const long long h = ht / tokens, t = ht - h * tokens;
    dst[e] = src[(t * heads + h) * ph + sub];
  }
}

// dst[t][h * ph + sub] = src[h][t][sub]
__global__ __launch_bounds__(kMoveThreads) void head_merge_kernel(const uint4* __restrict__ src,
                                                                  uint4* __restrict__ dst, long long tokens,
                                                                  int heads, int ph) {
  const long long total = tokens * heads * ph;
  for (long long e = (long long)blockIdx.x * kMoveThreads + threadIdx.x; e < total;
       e += (long long)gridDim.x * kMoveThreads) {
    const long long row = e / ph;  // t * heads + h
    const int sub = (int)(e - row * ph);
    const long long t = row / heads, h = row - t * heads;
    dst[e] = src[(h * tokens + t) * ph + sub];
  }
}

// dst[n][h][r][k] = src[h][n][r][k] (rk = R * topk entries per (n, h))
__global__ __launch_bounds__(kMoveThreads) void route_heads_kernel(const int32_t* __restrict__ src,
                                                                   int32_t* __restrict__ dst, int N, int heads,
                                                                   int rk) {
  const long long total = (long long)N * heads * rk;
  for (long long e = (long long)blockIdx.x * kMoveThreads + threadIdx.x; e < total;
       e += (long long)gridDim.x * kMoveThreads) {
    const long long nh = e / rk;
    const int i = (int)(e - nh * rk);
    const long long n = nh / heads, h = nh - n * heads;
    dst[e] = src[(h * N + n) * rk + i];
  }
}

unsigned move_blocks(long long items) {
  const long long b = (items + kMoveThreads - 1) / kMoveThreads;
  return (unsigned)(b < kMoveMaxBlocks ? (b > 0 ? b : 1) : kMoveMaxBlocks);
}

}  // namespace

hipError_t launch_head_split(const void* src, void* dst, long long tokens, int heads, int esz, hipStream_t st) {
  const int ph = 32 * esz / 16;
  launch(head_split_kernel, dim3(move_blocks(tokens * heads * ph)), dim3(kMoveThreads), 0, st,
         (const uint4*)src, (uint4*)dst, tokens, heads, ph);
  return hipGetLastError();
}

hipError_t launch_head_merge(const void* src, void* dst, long long tokens, int heads, int esz, hipStream_t st) {
  const int ph = 32 * esz / 16;
  launch(head_merge_kernel, dim3(move_blocks(tokens * heads * ph)), dim3(kMoveThreads), 0, st,
         (const uint4*)src, (uint4*)dst, tokens, heads, ph);
  return hipGetLastError();
}

hipError_t launch_route_heads(const int32_t* src, int32_t* dst, int N, int heads, int rk, hipStream_t st) {
  launch(route_heads_kernel, dim3(move_blocks((long long)N * heads * rk)), dim3(kMoveThreads), 0, st, src, dst, N,
         heads, rk);
  return hipGetLastError();
}

}  // namespace bra
