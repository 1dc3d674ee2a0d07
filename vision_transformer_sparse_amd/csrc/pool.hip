// Region-mean pooling: Q^r and K^r, the per-region means of q and k over the
// region's tokens (not over channels) -- the q_win / k_win step of the BRA
// walk-through at TRANSFORMER.niftyadmin.cn/n/347023.html, section BRA模块.
//
// One workgroup per (image, region). Each thread owns one 16-byte channel
// chunk of a token and walks a fixed subset of the region's tokens, so every
// load is a coalesced 16-byte NHWC read; the per-thread partial sums are then
// combined in LDS in a fixed order. The result is bit-reproducible from run
// to run (the routing that follows compares it with an exact tie rule).
#include "bra_internal.h"

namespace bra {
namespace {

constexpr int kPoolThreads = 256;

template <typename T>
struct Vec16;
template <>
struct Vec16<uint16_t> {
  static constexpr int n = 8;
  __device__ static void add(const uint16_t* p, float* acc) {
    uint4 w = *reinterpret_cast<const uint4*>(p);
    acc[0] += bf16_lo(w.x); acc[1] += bf16_hi(w.x);
    acc[2] += bf16_lo(w.y); acc[3] += bf16_hi(w.y);
    acc[4] += bf16_lo(w.z); acc[5] += bf16_hi(w.z);
    acc[6] += bf16_lo(w.w); acc[7] += bf16_hi(w.w);
  }
};
template <>
struct Vec16<float> {
  static constexpr int n = 4;
  __device__ static void add(const float* p, float* acc) {
    float4 w = *reinterpret_cast<const float4*>(p);
    acc[0] += w.x; acc[1] += w.y; acc[2] += w.z; acc[3] += w.w;
  }
};

template <typename T>
__global__ __launch_bounds__(kPoolThreads) void region_pool_kernel(
    const T* __restrict__ q, const T* __restrict__ k, int H, int W, int C, int S,
    float* __restrict__ qr, float* __restrict__ kr) {
  constexpr int V = Vec16<T>::n;
  extern __shared__ float part[];  // [2][lanes][C]
  const int R = S * S;
  const int nr = blockIdx.x;
  const int n = nr / R, r = nr - n * R;
  const int j = r / S, i = r - j * S;
  const int rh = H / S, rw = W / S, T_ = rh * rw;
  const int nchunk = C / V;
  const int lanes = kPoolThreads / nchunk;  // tokens walked in parallel
  const int tid = threadIdx.x;
  const int chunk = tid % nchunk, tl = tid / nchunk;

  float aq[V], ak[V];
#pragma unroll
  for (int e = 0; e < V; ++e) { aq[e] = 0.f; ak[e] = 0.f; }
  if (tl < lanes) {
    const size_t img = (size_t)n * H * W;
#pragma unroll 4
    for (int t = tl; t < T_; t += lanes) {
      const int y = j * rh + t / rw, x = i * rw + t % rw;
      const size_t off = ((img + (size_t)y * W + x) * C) + (size_t)chunk * V;
      Vec16<T>::add(q + off, aq);
      Vec16<T>::add(k + off, ak);
    }
    float* pq = part + (size_t)tl * C + chunk * V;
    float* pk = part + (size_t)(lanes + tl) * C + chunk * V;
#pragma unroll
    for (int e = 0; e < V; ++e) { pq[e] = aq[e]; pk[e] = ak[e]; }
  }
  __syncthreads();
  const float count = (float)T_;
  for (int c = tid; c < C; c += kPoolThreads) {
    float sq = 0.f, sk = 0.f;
    for (int l = 0; l < lanes; ++l) {
      sq += part[(size_t)l * C + c];
      sk += part[(size_t)(lanes + l) * C + c];
    }
    qr[(size_t)nr * C + c] = sq / count;
    kr[(size_t)nr * C + c] = sk / count;
  }
}

}  // namespace

hipError_t launch_region_pool(const void* q, const void* k, const Shape& s,
                              int dtype, float* qr, float* kr, hipStream_t st) {
  const int V = dtype == 1 ? 8 : 4;
  const int nchunk = s.C / V;
  const int lanes = kPoolThreads / nchunk;
  const size_t lds = (size_t)2 * lanes * s.C * sizeof(float);
  dim3 grid((unsigned)(s.N * s.R)), block(kPoolThreads);
  if (dtype == 1)
    hipLaunchKernelGGL(region_pool_kernel<uint16_t>, grid, block, lds, st,
                       (const uint16_t*)q, (const uint16_t*)k, s.H, s.W, s.C, s.S, qr, kr);
  else
    hipLaunchKernelGGL(region_pool_kernel<float>, grid, block, lds, st,
                       (const float*)q, (const float*)k, s.H, s.W, s.C, s.S, qr, kr);
  return hipGetLastError();
}

}  // namespace bra
