// Region-to-region routing: A = (Q^r * C^-1/2) K^r^T, an S^2 x S^2 affinity
// (Eq. 4), and per row the indices of the topk largest entries (Eq. 5) --
// TopkRouting.forward in the BRA walk-through at
// TRANSFORMER.niftyadmin.cn/n/347023.html, section BRA模块. The routing
// embedding is the identity; the softmax of the selected logits (routing
// weights) is not consumed by the gather and is not computed.
//
// One workgroup (4 waves) per (image, block of 4*RPW query regions), RPW
// query rows per wave (4 when there are at most 64 regions, else 1). K^r of the image is staged through LDS in channel slices
// with coalesced 16-byte loads (whole, when it fits), the 4 Q^r rows next to
// it; lane l owns the candidate regions l, l+64, ... and reads K^r and Q^r
// four channels at a time. Each logit is one fp32 fma chain in ascending
// channel order, then one multiply by C^-1/2 -- a fixed order, so the result
// is reproducible bit for bit.
//
// Top-k with an exact tie rule: every (A, s) becomes a 64-bit key whose
// unsigned order is "larger A first, then lower s first". With at most 64
// candidates each lane ranks its own key against all others (broadcast LDS
// reads, no cross-lane chain) and lanes of rank < topk write their index at
// that rank. With more candidates, topk rounds of a wave-wide maximum pick
// the winners in descending order.
#include "bra_internal.h"

namespace bra {
namespace {

constexpr int kThreads = 256;
constexpr size_t kLdsBudget = 48 * 1024;

__device__ __forceinline__ uint64_t route_key(float a, int s) {
  if (a == 0.0f) a = 0.0f;  // -0 and +0 are the same logit
  uint32_t u = __float_as_uint(a);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);  // order-preserving map to unsigned
  return ((uint64_t)u << 32) | (uint32_t)(0xffffffffu - (uint32_t)s);
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const uint64_t y = __shfl_xor(x, off, 64);
    x = y > x ? y : x;
  }
  return x;
}

// Channel slice staged per pass: the whole of C when K^r fits the budget
// (C is a multiple of 32; the slice stays a multiple of 4 dividing C). K^r
// rows are padded by 4 floats so the lanes' 16-byte reads spread over banks.
__host__ __device__ inline int slice_channels(int R, int C, int rows) {
  int ck = C;
  while (ck % 8 == 0 && ((size_t)R * (ck + 4) + (size_t)rows * ck) * 4 > kLdsBudget) ck /= 2;
  return ck;
}

template <int MPL, int RPW>
__global__ __launch_bounds__(kThreads) void route_kernel(const float* __restrict__ qr,
                                                         const float* __restrict__ kr, int R, int C,
                                                         int topk, float scale,
                                                         int32_t* __restrict__ route) {
  constexpr int kRowsPerBlock = RPW * kThreads / 64;
  extern __shared__ __attribute__((aligned(16))) float smem[];
  const int ck = slice_channels(R, C, kRowsPerBlock), ks_stride = ck + 4;
  float* ks = smem;                            // [R][ck + 4]
  float* qs = smem + (size_t)R * ks_stride;    // [rows][ck]
  __shared__ uint64_t keys[kThreads / 64][64];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int blocks_per_img = (R + kRowsPerBlock - 1) / kRowsPerBlock;
  const int n = blockIdx.x / blocks_per_img;
  const int r0 = (blockIdx.x - n * blocks_per_img) * kRowsPerBlock;
  const int rw0 = r0 + wave * RPW;  // this wave's first query row (rows past R: not stored)
  const float* krn = kr + (size_t)n * R * C;
  const float* qrn = qr + (size_t)n * R * C;

  float acc[RPW][MPL];
#pragma unroll
  for (int i = 0; i < RPW; ++i)
#pragma unroll
    for (int m = 0; m < MPL; ++m) acc[i][m] = 0.f;

  for (int c0 = 0; c0 < C; c0 += ck) {
    if (c0) __syncthreads();
    const int q4 = ck / 4;  // float4 pieces per row slice
    // batches of 8 loads in flight per thread, then their LDS stores
    for (int e0 = tid; e0 < R * q4; e0 += 8 * kThreads) {
      float4 buf[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = min(e0 + i * kThreads, R * q4 - 1);
        const int s = e / q4, j = e - s * q4;
        buf[i] = *reinterpret_cast<const float4*>(krn + (size_t)s * C + c0 + 4 * j);
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int e = e0 + i * kThreads;
        if (e < R * q4) {
          const int s = e / q4, j = e - s * q4;
          *reinterpret_cast<float4*>(ks + (size_t)s * ks_stride + 4 * j) = buf[i];
        }
      }
    }
    for (int e = tid; e < kRowsPerBlock * q4; e += kThreads) {
      const int rr = e / q4, j = e - rr * q4;
      const int rq = min(r0 + rr, R - 1);
      *reinterpret_cast<float4*>(qs + (size_t)rr * ck + 4 * j) =
          *reinterpret_cast<const float4*>(qrn + (size_t)rq * C + c0 + 4 * j);
    }
    __syncthreads();
    const float* qw = qs + (size_t)wave * RPW * ck;
#pragma unroll 4
    for (int c = 0; c < ck; c += 4) {
      float4 qv[RPW];
#pragma unroll
      for (int i = 0; i < RPW; ++i) qv[i] = *reinterpret_cast<const float4*>(qw + i * ck + c);
#pragma unroll
      for (int m = 0; m < MPL; ++m) {
        const int s = min(lane + 64 * m, R - 1);
        const float4 kv = *reinterpret_cast<const float4*>(ks + (size_t)s * ks_stride + c);
#pragma unroll
        for (int i = 0; i < RPW; ++i) {
          acc[i][m] = fmaf(qv[i].x, kv.x, acc[i][m]);
          acc[i][m] = fmaf(qv[i].y, kv.y, acc[i][m]);
          acc[i][m] = fmaf(qv[i].z, kv.z, acc[i][m]);
          acc[i][m] = fmaf(qv[i].w, kv.w, acc[i][m]);
        }
      }
    }
  }

#pragma unroll
  for (int i = 0; i < RPW; ++i) {
  const int r = rw0 + i;
  if (r >= R) break;  // wave-uniform; no barrier follows
  int32_t* out = route + ((size_t)n * R + r) * topk;
  uint64_t key[MPL];
#pragma unroll
  for (int m = 0; m < MPL; ++m) {
    const int s = lane + 64 * m;
    key[m] = s < R ? route_key(acc[i][m] * scale, s) : 0ull;
  }
  if (MPL == 1) {
    uint64_t* kw = keys[wave];
    __builtin_amdgcn_wave_barrier();  // the previous row's reads of kw are done
    kw[lane] = key[0];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    if (lane < R) {
      int rank = 0;
#pragma unroll 8
      for (int s2 = 0; s2 < R; s2 += 2) {
        const uint4 two = *reinterpret_cast<const uint4*>(kw + s2);  // keys s2, s2+1
        const uint64_t k0 = ((uint64_t)two.y << 32) | two.x, k1 = ((uint64_t)two.w << 32) | two.z;
        rank += (k0 > key[0]) + (s2 + 1 < R && k1 > key[0]);
      }
      if (rank < topk) out[rank] = lane;
    }
  } else {
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
}

template <int MPL, int RPW>
hipError_t launch_t(const float* qr, const float* kr, int N, int R, int C, int topk,
                    int32_t* route, hipStream_t st) {
  constexpr int rows = RPW * kThreads / 64;
  const float scale = (float)(1.0 / __builtin_sqrt((double)C));
  const int ck = slice_channels(R, C, rows);
  const size_t lds = ((size_t)R * (ck + 4) + (size_t)rows * ck) * sizeof(float);
  const unsigned blocks = (unsigned)(N * ((R + rows - 1) / rows));
  hipLaunchKernelGGL((route_kernel<MPL, RPW>), dim3(blocks), dim3(kThreads), lds, st, qr, kr, R,
                     C, topk, scale, route);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* qr, const float* kr, int N, int R, int C, int topk,
                        int32_t* route, hipStream_t st) {
  if (R <= 64) return launch_t<1, 4>(qr, kr, N, R, C, topk, route, st);
  if (R <= 128) return launch_t<2, 1>(qr, kr, N, R, C, topk, route, st);
  if (R <= 256) return launch_t<4, 1>(qr, kr, N, R, C, topk, route, st);
  if (R <= 512) return launch_t<8, 1>(qr, kr, N, R, C, topk, route, st);
  return launch_t<16, 1>(qr, kr, N, R, C, topk, route, st);
}

}  // namespace bra
