// Region-to-region routing: the S^2 x S^2 affinity A = (Q^r * C^-1/2) K^r^T
// (Eq. 4) and, per row, the indices of its topk largest entries (Eq. 5) --
// TopkRouting.forward in the walk-through at
// TRANSFORMER.niftyadmin.cn/n/347023.html, section BRA模块. The routing
// embedding is the identity; the softmax of the selected logits
// (routing weights) is not consumed by the gather and is not computed.
//
// Layout: a workgroup of 4 waves owns 16 consecutive query regions of one
// image (4 per wave); lane l of a wave owns candidate regions l, l+64, ...
// K^r is staged through LDS a channel slice at a time (row stride padded by
// one float so the lane-strided reads hit distinct banks); the 16 Q^r rows of
// the slice are read as LDS broadcasts. Each logit is one fp32 fma chain in
// ascending channel order, so it is reproducible bit for bit.
//
// Top-k: each (logit, region) pair is packed into one 64-bit key whose
// unsigned order is "larger logit first, then lower region index first";
// topk rounds of a wave-wide maximum pick the winners in descending order,
// which realises the tie rule (equal logits -> lower region index) exactly.
#include "bra_internal.h"

namespace bra {
namespace {

constexpr int kRouteThreads = 256;
constexpr int kRowsPerWave = 4;
constexpr int kRowsPerBlock = kRowsPerWave * (kRouteThreads / 64);

__device__ __forceinline__ uint64_t route_key(float a, int s) {
  if (a == 0.0f) a = 0.0f;  // -0 and +0 are the same logit
  uint32_t u = __float_as_uint(a);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // order-preserving map to unsigned
  return ((uint64_t)u << 32) | (uint32_t)(0xffffffffu - (uint32_t)s);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    uint64_t y = __shfl_xor(x, off, 64);
    x = y > x ? y : x;
  }
  return x;
}

template <int MPL, int CK>
__global__ __launch_bounds__(kRouteThreads) void route_kernel(
    const float* __restrict__ qr, const float* __restrict__ kr, int R, int C,
    int topk, float scale, int32_t* __restrict__ route) {
  extern __shared__ float smem[];
  float* ks = smem;                          // [R][CK + 1]
  float* qs = smem + (size_t)R * (CK + 1);   // [16][CK]
  const int n = blockIdx.y;
  const int r0 = blockIdx.x * kRowsPerBlock;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const float* krn = kr + (size_t)n * R * C;
  const float* qrn = qr + (size_t)n * R * C;

  float acc[kRowsPerWave][MPL];
#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i)
#pragma unroll
    for (int m = 0; m < MPL; ++m) acc[i][m] = 0.f;

  for (int c0 = 0; c0 < C; c0 += CK) {
    __syncthreads();
    for (int e = threadIdx.x; e < R * CK; e += kRouteThreads) {
      const int s = e / CK, cc = e - s * CK;
      ks[s * (CK + 1) + cc] = krn[(size_t)s * C + c0 + cc];
    }
    for (int e = threadIdx.x; e < kRowsPerBlock * CK; e += kRouteThreads) {
      const int rr = e / CK, cc = e - rr * CK;
      const int r = r0 + rr;
      qs[rr * CK + cc] = r < R ? qrn[(size_t)r * C + c0 + cc] * scale : 0.f;
    }
    __syncthreads();
#pragma unroll 4
    for (int cc = 0; cc < CK; ++cc) {
      float qv[kRowsPerWave];
#pragma unroll
      for (int i = 0; i < kRowsPerWave; ++i) qv[i] = qs[(wave * kRowsPerWave + i) * CK + cc];
#pragma unroll
      for (int m = 0; m < MPL; ++m) {
        const int s = lane + 64 * m;
        const float kv = s < R ? ks[s * (CK + 1) + cc] : 0.f;
#pragma unroll
        for (int i = 0; i < kRowsPerWave; ++i) acc[i][m] = fmaf(qv[i], kv, acc[i][m]);
      }
    }
  }

#pragma unroll
  for (int i = 0; i < kRowsPerWave; ++i) {
    const int r = r0 + wave * kRowsPerWave + i;
    if (r >= R) break;  // wave-uniform
    uint64_t key[MPL];
#pragma unroll
    for (int m = 0; m < MPL; ++m) {
      const int s = lane + 64 * m;
      key[m] = s < R ? route_key(acc[i][m], s) : 0ull;
    }
    int32_t* out = route + ((size_t)n * R + r) * topk;
    for (int p = 0; p < topk; ++p) {
      uint64_t best = 0ull;
#pragma unroll
      for (int m = 0; m < MPL; ++m) best = key[m] > best ? key[m] : best;
      best = wave_max_u64(best);
      const int win = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffu));
#pragma unroll
      for (int m = 0; m < MPL; ++m)
        if (lane + 64 * m == win) key[m] = 0ull;
      if (lane == 0) out[p] = win;
    }
  }
}

template <int MPL, int CK>
hipError_t launch_t(const float* qr, const float* kr, int N, int R, int C,
                    int topk, int32_t* route, hipStream_t st) {
  const size_t lds = ((size_t)R * (CK + 1) + (size_t)kRowsPerBlock * CK) * sizeof(float);
  dim3 grid((unsigned)((R + kRowsPerBlock - 1) / kRowsPerBlock), (unsigned)N);
  const float scale = (float)(1.0 / __builtin_sqrt((double)C));
  hipLaunchKernelGGL((route_kernel<MPL, CK>), grid, dim3(kRouteThreads), lds, st,
                     qr, kr, R, C, topk, scale, route);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* qr, const float* kr, int N, int R, int C,
                        int topk, int32_t* route, hipStream_t st) {
  // C is a multiple of 32 (head_dim 32); CK must divide it.
  if (R <= 64) return launch_t<1, 32>(qr, kr, N, R, C, topk, route, st);
  if (R <= 128) return launch_t<2, 32>(qr, kr, N, R, C, topk, route, st);
  if (R <= 256) return launch_t<4, 32>(qr, kr, N, R, C, topk, route, st);
  if (R <= 512) return launch_t<8, 16>(qr, kr, N, R, C, topk, route, st);
  return launch_t<16, 8>(qr, kr, N, R, C, topk, route, st);
}

}  // namespace bra
