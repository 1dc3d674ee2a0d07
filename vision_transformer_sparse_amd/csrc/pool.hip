// Region-mean pooling: Q^r and K^r, the per-region means of q and k over the
// region's tokens (not over channels) -- the q_win / k_win step of the BRA
// walk-through at TRANSFORMER.niftyadmin.cn/n/347023.html, section BRA模块.
//
// One workgroup per (image, region), sized to the region (64-256 threads).
// A thread owns one 16-byte channel chunk and up to TPT tokens of the region;
// it issues 2*TPT coalesced NHWC loads at a time before adding any of them,
// so a whole region is in flight at once (the kernel is bound by memory
// latency x bytes in flight, not by arithmetic). Per-thread partial sums are
// combined in LDS in a fixed order, so the means are reproducible bit for bit
// (the routing that follows breaks ties exactly).
//
// On request (kn non-null, bf16) the kernel also reports, per (image,
// region, head of 32 channels), the largest squared norm |k_t|^2 of the
// head's slice over the region's tokens. The large-region attention kernel
// bounds every score of a query by |q| * max |k| over its routed regions
// (Cauchy-Schwarz) and uses that bound as the softmax's fixed maximum. The
// four 16-byte chunks of one head are consecutive threads (one lane quad),
// so a token's head norm is a quad sum.
#include "bra_internal.h"

namespace bra {
namespace {

template <typename T>
struct Vec16;
template <>
struct Vec16<uint16_t> {
  static constexpr int n = 8;
  __device__ static void add(const uint4 w, float* acc) {
    acc[0] += bf16_lo(w.x); acc[1] += bf16_hi(w.x);
    acc[2] += bf16_lo(w.y); acc[3] += bf16_hi(w.y);
    acc[4] += bf16_lo(w.z); acc[5] += bf16_hi(w.z);
    acc[6] += bf16_lo(w.w); acc[7] += bf16_hi(w.w);
  }
};
template <>
struct Vec16<float> {
  static constexpr int n = 4;
  __device__ static void add(const uint4 w, float* acc) {
    acc[0] += __uint_as_float(w.x); acc[1] += __uint_as_float(w.y);
    acc[2] += __uint_as_float(w.z); acc[3] += __uint_as_float(w.w);
  }
};

template <typename T, int TPT>
__global__ __launch_bounds__(256) void region_pool_kernel(
    const T* __restrict__ q, const T* __restrict__ k, int H, int W, int C, int S,
    float* __restrict__ qr, float* __restrict__ kr, const uint16_t* __restrict__ lw,
    uint32_t* __restrict__ wpk, float* __restrict__ kn) {
  constexpr int V = Vec16<T>::n;
  extern __shared__ float part[];  // [2][lanes][C]
  const int R = S * S;
  const int nr = blockIdx.x;
  const int n = nr / R, r = nr - n * R;
  const int j = r / S, i = r - j * S;
  const int rh = H / S, rw = W / S, T_ = rh * rw;
  const int nchunk = C / V;
  const int lanes = blockDim.x / nchunk;  // tokens walked in parallel
  const int tid = threadIdx.x;
  const int chunk = tid % nchunk, tl = tid / nchunk;
  const size_t img = (size_t)n * H * W;

  // Side job: the LCE weights repacked for the attention kernel's dot2s.
  if (wpk)
    for (int e = blockIdx.x * blockDim.x + tid; e < lce_pack_items(C); e += gridDim.x * blockDim.x)
      pack_lce_item(lw, C, e, wpk);

  float aq[V], ak[V];
#pragma unroll
  for (int e = 0; e < V; ++e) { aq[e] = 0.f; ak[e] = 0.f; }
  float kmax2 = 0.f;  // largest |k|^2 of this thread's head over its tokens (kn only)
  const bool norms = V == 8 && kn != nullptr;
  if (tl < lanes) {
    for (int t0 = tl; t0 < T_; t0 += TPT * lanes) {
      uint4 bq[TPT], bk[TPT];
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        const int t = t0 + u * lanes;
        if (t < T_) {
          const int y = j * rh + t / rw, x = i * rw + t % rw;
          const size_t off = ((img + (size_t)y * W + x) * C) + (size_t)chunk * V;
          bq[u] = *reinterpret_cast<const uint4*>(q + off);
          bk[u] = *reinterpret_cast<const uint4*>(k + off);
        }
      }
#pragma unroll
      for (int u = 0; u < TPT; ++u) {
        if (t0 + u * lanes < T_) {
          Vec16<T>::add(bq[u], aq);
          Vec16<T>::add(bk[u], ak);
          if (norms) {
            // the quad (one token's four chunks of a head) shares the branch
            float n2 = 0.f;
            n2 = fmaf(bf16_lo(bk[u].x), bf16_lo(bk[u].x), n2); n2 = fmaf(bf16_hi(bk[u].x), bf16_hi(bk[u].x), n2);
            n2 = fmaf(bf16_lo(bk[u].y), bf16_lo(bk[u].y), n2); n2 = fmaf(bf16_hi(bk[u].y), bf16_hi(bk[u].y), n2);
            n2 = fmaf(bf16_lo(bk[u].z), bf16_lo(bk[u].z), n2); n2 = fmaf(bf16_hi(bk[u].z), bf16_hi(bk[u].z), n2);
            n2 = fmaf(bf16_lo(bk[u].w), bf16_lo(bk[u].w), n2); n2 = fmaf(bf16_hi(bk[u].w), bf16_hi(bk[u].w), n2);
            kmax2 = fmaxf(kmax2, quad_sum(n2));
          }
        }
      }
    }
    float* pq = part + (size_t)tl * C + chunk * V;
    float* pk = part + (size_t)(lanes + tl) * C + chunk * V;
#pragma unroll
    for (int e = 0; e < V; ++e) { pq[e] = aq[e]; pk[e] = ak[e]; }
    if (norms && (chunk & 3) == 0) part[(size_t)2 * lanes * C + (size_t)tl * (C / 32) + chunk / 4] = kmax2;
  }
  __syncthreads();
  if (norms) {
    const int heads = C / 32;
    for (int h = tid; h < heads; h += blockDim.x) {
      float mx = 0.f;
      for (int l = 0; l < lanes; ++l) mx = fmaxf(mx, part[(size_t)2 * lanes * C + (size_t)l * heads + h]);
      kn[(size_t)nr * heads + h] = mx;
    }
  }
  const float count = (float)T_;
  for (int c = tid; c < C; c += blockDim.x) {
    float sq = 0.f, sk = 0.f;
    for (int l = 0; l < lanes; ++l) {
      sq += part[(size_t)l * C + c];
      sk += part[(size_t)(lanes + l) * C + c];
    }
    qr[(size_t)nr * C + c] = sq / count;
    kr[(size_t)nr * C + c] = sk / count;
  }
}

template <typename T>
hipError_t launch_t(const void* q, const void* k, const Shape& s, float* qr, float* kr,
                    const void* lw, uint32_t* wpk, float* kn, hipStream_t st) {
  constexpr int V = Vec16<T>::n;
  const int nchunk = s.C / V;                 // <= 256 (C <= 1024)
  int threads, lanes;
  if (s.rh == 4 && s.rw == 4 && nchunk * 4 <= 256) {
    // 4x4 regions: a token lane per region column, so the sum runs down each
    // column and then across the four columns -- the order the one-kernel
    // forward pools in
    lanes = 4;
    threads = nchunk * 4;
  } else {
    // threads: a multiple of 64 holding whole token lanes, aiming at <= 8 tokens per thread
    int lanes_wanted = (s.T + 7) / 8;
    threads = nchunk * lanes_wanted;
    threads = threads < 64 ? 64 : threads;
    threads = threads > 256 ? 256 : threads;
    threads = ((threads + 63) / 64) * 64;
    lanes = threads / nchunk;
    if (lanes < 1) lanes = 1;
  }
  const int tpt = (s.T + lanes - 1) / lanes;  // tokens per thread (looped in batches of <= 8)
  const size_t lds = ((size_t)2 * lanes * s.C + (kn ? (size_t)lanes * (s.C / 32) : 0)) * sizeof(float);
  dim3 grid((unsigned)(s.N * s.R)), block(threads);
#define BRA_POOL(TP)                                                                    \
  launch((region_pool_kernel<T, TP>), grid, block, lds, st, (const T*)q,    \
                     (const T*)k, s.H, s.W, s.C, s.S, qr, kr, (const uint16_t*)lw, wpk, kn)
  if (tpt <= 1) BRA_POOL(1);
  else if (tpt <= 2) BRA_POOL(2);
  else if (tpt <= 4) BRA_POOL(4);
  else BRA_POOL(8);
#undef BRA_POOL
  return hipGetLastError();
}

}  // namespace

hipError_t launch_region_pool(const void* q, const void* k, const Shape& s, int dtype,
                              float* qr, float* kr, const void* lce_w, uint32_t* wpk,
                              float* kn, hipStream_t st) {
  return dtype == 1 ? launch_t<uint16_t>(q, k, s, qr, kr, lce_w, wpk, kn, st)
                    : launch_t<float>(q, k, s, qr, kr, nullptr, nullptr, nullptr, st);
}

}  // namespace bra
