// Token-to-token attention over the routed regions plus LCE, on the vector
// ALUs in fp32 -- the path for fp32 tensors, whose tolerance rules out bf16
// matrix cores. Eq. 6-7 of the BRA walk-through at
// TRANSFORMER.niftyadmin.cn/n/347023.html, section BRA模块: the keys/values of
// a query region are the tokens of its topk routed regions, rank-major and
// token-minor; each head (channels [h*32, h*32+32)) runs a softmax over all
// of them jointly; LCE(V) (5x5 depthwise conv, zero padding 2, bias) is added.
//
// Work split: one workgroup per (image, query region, head, query slice).
// Each thread owns one query: its 32-dim q row (pre-multiplied by
// head_dim^-1/2 * log2(e), so the softmax runs on exp2), a running max, a
// running sum and a 32-dim output, updated once per 32-key tile (online
// softmax). The keys/values of a tile are gathered by route index straight
// from NHWC memory into LDS, so the routed copy of K/V never exists in HBM.
#include "bra_internal.h"

namespace bra {
namespace {

constexpr int kHD = kHeadDim;
constexpr int kTile = 32;

template <typename T>
__device__ __forceinline__ void load_row32(const T* p, float* dst);
template <>
__device__ __forceinline__ void load_row32<float>(const float* p, float* dst) {
#pragma unroll
  for (int e = 0; e < kHD; e += 4) {
    float4 w = *reinterpret_cast<const float4*>(p + e);
    dst[e] = w.x; dst[e + 1] = w.y; dst[e + 2] = w.z; dst[e + 3] = w.w;
  }
}
template <>
__device__ __forceinline__ void load_row32<uint16_t>(const uint16_t* p, float* dst) {
#pragma unroll
  for (int e = 0; e < kHD; e += 8) {
    uint4 w = *reinterpret_cast<const uint4*>(p + e);
    dst[e] = bf16_lo(w.x); dst[e + 1] = bf16_hi(w.x);
    dst[e + 2] = bf16_lo(w.y); dst[e + 3] = bf16_hi(w.y);
    dst[e + 4] = bf16_lo(w.z); dst[e + 5] = bf16_hi(w.z);
    dst[e + 6] = bf16_lo(w.w); dst[e + 7] = bf16_hi(w.w);
  }
}

// LCE at one pixel for the 32 channels [c0, c0+32): bias + 25 taps.
template <typename T>
__device__ __forceinline__ void lce32(const T* __restrict__ v, const T* __restrict__ w,
                                      const T* __restrict__ b, int n, int y, int x,
                                      int H, int W, int C, int c0, float* acc) {
#pragma unroll
  for (int d = 0; d < kHD; ++d) acc[d] = b ? Elem<T>::load(b, c0 + d) : 0.f;
  for (int a = 0; a < 5; ++a) {
    const int yy = y + a - 2;
    if (yy < 0 || yy >= H) continue;
    for (int e = 0; e < 5; ++e) {
      const int xx = x + e - 2;
      if (xx < 0 || xx >= W) continue;
      float vv[kHD];
      load_row32<T>(v + (((size_t)n * H + yy) * W + xx) * C + c0, vv);
#pragma unroll
      for (int d = 0; d < kHD; ++d)
        acc[d] = fmaf(Elem<T>::load(w, (size_t)(c0 + d) * 25 + a * 5 + e), vv[d], acc[d]);
    }
  }
}

template <typename T>
__global__ __launch_bounds__(256) void attn_valu_kernel(
    const T* __restrict__ q, const T* __restrict__ k, const T* __restrict__ v,
    const T* __restrict__ w, const T* __restrict__ b,
    const int32_t* __restrict__ route, int H, int W, int C, int heads, int S,
    int topk, int qslices, float qscale, T* __restrict__ out) {
  __shared__ float Ks[kTile][kHD + 1];
  __shared__ float Vs[kTile][kHD + 1];
  const int R = S * S;
  const int rh = H / S, rw = W / S, T_ = rh * rw, L = topk * T_;
  int u = blockIdx.x;
  const int slice = u % qslices; u /= qslices;
  const int h = u % heads; u /= heads;
  const int r = u % R;
  const int n = u / R;
  const int jr = r / S, ir = r - jr * S;
  const int c0 = h * kHD;
  const int32_t* rt = route + ((size_t)n * R + r) * topk;

  const int t = slice * blockDim.x + threadIdx.x;  // query token in the region
  const bool valid = t < T_;
  const int y = jr * rh + (valid ? t / rw : 0), x = ir * rw + (valid ? t % rw : 0);

  float qv[kHD], o[kHD];
  float mx = -INFINITY, sum = 0.f;
  if (valid) {
    load_row32<T>(q + (((size_t)n * H + y) * W + x) * C + c0, qv);
#pragma unroll
    for (int d = 0; d < kHD; ++d) qv[d] *= qscale;
  }
#pragma unroll
  for (int d = 0; d < kHD; ++d) o[d] = 0.f;

  for (int base = 0; base < L; base += kTile) {
    __syncthreads();
    for (int e = threadIdx.x; e < kTile * (kHD / 4); e += blockDim.x) {
      const int key = e / (kHD / 4), part = e % (kHD / 4);
      const int kk = base + key;
      float kv[4] = {0.f, 0.f, 0.f, 0.f}, vv[4] = {0.f, 0.f, 0.f, 0.f};
      if (kk < L) {
        const int p = kk / T_, tt = kk - p * T_;
        const int s = rt[p];
        const int js = s / S, is = s - js * S;
        const int yy = js * rh + tt / rw, xx = is * rw + tt % rw;
        const size_t off = (((size_t)n * H + yy) * W + xx) * C + c0 + part * 4;
#pragma unroll
        for (int z = 0; z < 4; ++z) {
          kv[z] = Elem<T>::load(k, off + z);
          vv[z] = Elem<T>::load(v, off + z);
        }
      }
#pragma unroll
      for (int z = 0; z < 4; ++z) {
        Ks[key][part * 4 + z] = kv[z];
        Vs[key][part * 4 + z] = vv[z];
      }
    }
    __syncthreads();
    if (!valid) continue;
    const int nk = min(kTile, L - base);
    float sc[kTile];
    float tmax = -INFINITY;
#pragma unroll
    for (int e = 0; e < kTile; ++e) {
      float s = 0.f;
#pragma unroll
      for (int d = 0; d < kHD; ++d) s = fmaf(qv[d], Ks[e][d], s);
      sc[e] = e < nk ? s : -INFINITY;
      tmax = fmaxf(tmax, sc[e]);
    }
    const float nmx = fmaxf(mx, tmax);
    const float corr = __builtin_amdgcn_exp2f(mx - nmx);  // 0 on the first tile
    sum *= corr;
#pragma unroll
    for (int d = 0; d < kHD; ++d) o[d] *= corr;
#pragma unroll
    for (int e = 0; e < kTile; ++e) {
      const float p = __builtin_amdgcn_exp2f(sc[e] - nmx);
      sum += p;
#pragma unroll
      for (int d = 0; d < kHD; ++d) o[d] = fmaf(p, Vs[e][d], o[d]);
    }
    mx = nmx;
  }
  if (!valid) return;
  float l[kHD];
  lce32<T>(v, w, b, n, y, x, H, W, C, c0, l);
  const float inv = 1.0f / sum;
  const size_t ob = (((size_t)n * H + y) * W + x) * C + c0;
#pragma unroll
  for (int d = 0; d < kHD; ++d) Elem<T>::store(out, ob + d, fmaf(o[d], inv, l[d]));
}

template <typename T>
__global__ __launch_bounds__(256) void lce_kernel(
    const T* __restrict__ v, const T* __restrict__ w, const T* __restrict__ b,
    int N, int H, int W, int C, float* __restrict__ out) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t groups = (size_t)N * H * W * (C / kHD);
  if (idx >= groups) return;
  const int cg = (int)(idx % (C / kHD));
  size_t p = idx / (C / kHD);
  const int x = (int)(p % W); p /= W;
  const int y = (int)(p % H);
  const int n = (int)(p / H);
  float acc[kHD];
  lce32<T>(v, w, b, n, y, x, H, W, C, cg * kHD, acc);
  const size_t ob = (((size_t)n * H + y) * W + x) * C + cg * kHD;
#pragma unroll
  for (int d = 0; d < kHD; ++d) out[ob + d] = acc[d];
}

}  // namespace

hipError_t launch_attend_valu(const void* q, const void* k, const void* v,
                              const void* w, const void* b, const int32_t* route,
                              const Shape& s, int dtype, void* out, hipStream_t st) {
  const int threads = s.T >= 256 ? 256 : ((s.T + 63) / 64) * 64;
  const int qslices = (s.T + threads - 1) / threads;
  const size_t blocks = (size_t)s.N * s.R * s.heads * qslices;
  const float qscale = (float)(1.4426950408889634 / __builtin_sqrt((double)s.hd));
  if (dtype == 1)
    launch(attn_valu_kernel<uint16_t>, dim3((unsigned)blocks), dim3(threads), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                       (const uint16_t*)w, (const uint16_t*)b, route, s.H, s.W, s.C,
                       s.heads, s.S, s.topk, qslices, qscale, (uint16_t*)out);
  else
    launch(attn_valu_kernel<float>, dim3((unsigned)blocks), dim3(threads), 0, st,
                       (const float*)q, (const float*)k, (const float*)v,
                       (const float*)w, (const float*)b, route, s.H, s.W, s.C,
                       s.heads, s.S, s.topk, qslices, qscale, (float*)out);
  return hipGetLastError();
}

hipError_t launch_lce(const void* v, const void* w, const void* b, const Shape& s,
                      int dtype, float* out, hipStream_t st) {
  const size_t groups = (size_t)s.N * s.H * s.W * (s.C / kHD);
  const unsigned blocks = (unsigned)((groups + 255) / 256);
  if (dtype == 1)
    launch(lce_kernel<uint16_t>, dim3(blocks), dim3(256), 0, st,
                       (const uint16_t*)v, (const uint16_t*)w, (const uint16_t*)b,
                       s.N, s.H, s.W, s.C, out);
  else
    launch(lce_kernel<float>, dim3(blocks), dim3(256), 0, st,
                       (const float*)v, (const float*)w, (const float*)b,
                       s.N, s.H, s.W, s.C, out);
  return hipGetLastError();
}

}  // namespace bra
