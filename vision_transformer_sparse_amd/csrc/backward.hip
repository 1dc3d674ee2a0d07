// Backward of the BRA operator for given routes: gradients of the output
// with respect to q, k, v and the LCE weights and bias. The walk-through at
// TRANSFORMER.niftyadmin.cn/n/347023.html (section BRA模块) detaches the
// region means before the router, so no gradient flows through routing; the
// forward's routes are inputs here. For image n, head h and query region r
// with gathered keys/values K, V (its topk routed regions, rank-major),
// queries Q and output gradient G:
//   s = hd^-1/2 Q K^T, P = softmax(s) per query, O = P V,
//   dP = G V^T, D = rowsum(G * O), dS = P * (dP - D),
//   dQ = hd^-1/2 dS K, and for every routed region: dK += hd^-1/2 dS^T Q,
//   dV += P^T G, plus LCE: dV += dout correlated with the flipped 5x5 kernel,
//   dW[c][a][e] = sum dout * v shifted, db[c] = sum dout.
//
// bf16 tensors, head_dim 32, regions of a multiple of 16 tokens. Kernels:
//  * inv_route_kernel: per image, the routers of every region (CSR, routers
//    in ascending order), so the key side gathers instead of scattering and
//    every gradient is a fixed-order sum (no atomics).
//  * bwd_query_kernel: one workgroup per (image, region, head, up to 64
//    queries), a wave per 16 queries; 32-key tiles of the gathered K and V
//    staged in LDS and shared by the waves. Pass 1 is the forward with an
//    online maximum (S^T = K Q^T, O^T = V^T P^T on 16x16x32 bf16 products)
//    and leaves per query the base-2 log-sum-exp and D = G . O; pass 2
//    recomputes P and forms dP^T = V G^T, dS^T, and dQ^T += K^T dS^T (K^T by
//    transposing LDS reads, dS^T from the lane's own eight keys, the same
//    key order on both operands).
//  * bwd_key_kernel: one workgroup per (image, region, head, up to 64 keys),
//    a wave per 16 keys; for every router region, 32-query tiles of Q and G
//    (and their log-sum-exp and D) staged in LDS: S = Q K^T and dP = G V^T
//    with lane = key, P and dS from the saved statistics, dV^T += G^T P and
//    dK^T += Q^T dS (Q^T, G^T by transposing LDS reads); then the LCE term of
//    dV from the key's 5x5 window of dout.
//  * lce_grad_rows_kernel / lce_grad_sum_kernel: per image row and channel
//    the 25 tap sums and the bias sum, then a fixed-order sum over rows.
#include "bra_internal.h"

namespace bra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kTile = 32;                                // keys (query side) / queries (key side) a tile
constexpr float kQs = 0.17677669529663687f * 1.4426950408889634f;  // hd^-1/2 in log2 units
constexpr float kScale = 0.17677669529663687f;                     // hd^-1/2

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;   // dout
  const uint16_t* w;   // LCE weights [C][25]
  const int32_t* route;
  const int32_t* inv_off;  // [N][R+1]
  const int32_t* inv_ent;  // [N][R*topk]
  float* lse;              // [N][H*W][heads], base 2
  float* dsum;             // [N][H*W][heads]
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int N, H, W, C, heads, S, topk, R, rh, rw, T, L;
};

__device__ __forceinline__ bf16x4 ld_tr(const char* p) {
  // within each 16-lane group, lanes 4r..4r+3 address row r's 16 consecutive
  // bf16 (4 each); lane i receives element i of rows 0..3
  const s16x4 x = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<char*>(p)));
  return __builtin_bit_cast(bf16x4, x);
}
__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}
__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 as8(uint4 x) { return __builtin_bit_cast(bf16x8, x); }

// Stores a 16-lane group layout (lane (col, g) holding channels 4g..4g+3 in
// a and 16+4g..16+4g+3 in b, fp32) as bf16: two lane swaps give lane group g
// channels 8g..8g+7, one 16-byte store a lane at byte offset off + 16g.
__device__ __forceinline__ void store_slice(Rsrc r, uint32_t off, int g, const float* a, const float* b,
                                            bool live) {
  const uint32_t la[2] = {float_to_bf16_bits(a[0]) | (float_to_bf16_bits(a[1]) << 16),
                          float_to_bf16_bits(a[2]) | (float_to_bf16_bits(a[3]) << 16)};
  const uint32_t hb[2] = {float_to_bf16_bits(b[0]) | (float_to_bf16_bits(b[1]) << 16),
                          float_to_bf16_bits(b[2]) | (float_to_bf16_bits(b[3]) << 16)};
  uint32_t xs[2], ys[2];
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const auto h32 = __builtin_amdgcn_permlane32_swap(la[j], hb[j], false, false);
    const auto h16 = __builtin_amdgcn_permlane16_swap(h32[0], h32[1], false, false);
    xs[j] = h16[0];
    ys[j] = h16[1];
  }
  if (live) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w4 = {xs[0], xs[1], ys[0], ys[1]};
    __builtin_amdgcn_raw_buffer_store_b128(w4, r, off + 16 * g, 0, 0);
  }
}

// ---------------------------------------------------------------- routers
// Per image: off[s] .. off[s+1] index the routers of region s in ent, in
// ascending order of the routing region r.
__global__ __launch_bounds__(256) void inv_route_kernel(const int32_t* __restrict__ route, int R, int topk,
                                                        int32_t* __restrict__ off, int32_t* __restrict__ ent) {
  extern __shared__ int cnt[];  // [R]
  const int n = blockIdx.x, tid = threadIdx.x;
  const int32_t* rt = route + (size_t)n * R * topk;
  for (int s = tid; s < R; s += blockDim.x) {
    int c = 0;
    for (int e = 0; e < R * topk; ++e) c += rt[e] == s;
    cnt[s] = c;
  }
  __syncthreads();
  if (tid == 0) {
    int acc = 0;
    for (int s = 0; s < R; ++s) {
      const int c = cnt[s];
      cnt[s] = acc;
      acc += c;
    }
    off[(size_t)n * (R + 1) + R] = acc;
  }
  __syncthreads();
  for (int s = tid; s < R; s += blockDim.x) {
    int o = cnt[s];
    off[(size_t)n * (R + 1) + s] = o;
    for (int e = 0; e < R * topk; ++e)
      if (rt[e] == s) ent[(size_t)n * R * topk + o++] = e / topk;
  }
}

// ---------------------------------------------------------------- query side
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void bwd_query_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kTile * 64];  // K tile | V tile, [32][64 bytes]
  __shared__ uint32_t rbase[16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, g = lane >> 4;
  const int GPR = a.T / 16 / WAVES;  // query groups of a region
  int u = xcd_unit(blockIdx.x, gridDim.x);
  const int qg = u % GPR;
  u /= GPR;
  const int h = u % a.heads;
  u /= a.heads;
  const int r = u % a.R, n = u / a.R;
  const int HW = a.H * a.W;
  const uint32_t rowb = (uint32_t)a.C * 2, hoff = (uint32_t)h * 64;
  const size_t img = (size_t)n * HW * a.C;
  const uint32_t img_bytes = (uint32_t)HW * rowb;
  const Rsrc qr = rsrc(a.q + img, img_bytes), kr = rsrc(a.k + img, img_bytes), vr = rsrc(a.v + img, img_bytes);
  const Rsrc gr = rsrc(a.g + img, img_bytes), dqr = rsrc(a.dq + img, img_bytes);

  // this wave's 16 queries of region r
  const int t = 16 * (qg * WAVES + wave) + col;
  const int qpix = ((r / a.S) * a.rh + t / a.rw) * a.W + (r % a.S) * a.rw + t % a.rw;
  const uint32_t qoff = (uint32_t)qpix * rowb + hoff;
  const bf16x8 bq = as8(ld16(qr, qoff + 16 * g));
  const bf16x8 bg = as8(ld16(gr, qoff + 16 * g));
  if (tid < a.topk) {
    const int s = a.route[((size_t)n * a.R + r) * a.topk + tid];
    rbase[tid] = (uint32_t)(((s / a.S) * a.rh * a.W + (s % a.S) * a.rw)) * rowb + hoff;
  }
  __syncthreads();

  char* kt_lds = lds;
  char* vt_lds = lds + kTile * 64;
  // keys u0 .. u0+31 of the gathered sequence into LDS (rows past L read zero)
  auto load_tile = [&](int u0) {
    for (int e = tid; e < kTile * 4; e += 64 * WAVES) {
      const int kk = e >> 2, ch = e & 3, uu = u0 + kk;
      uint32_t off = kOut;
      if (uu < a.L) {
        const int p = uu / a.T, j = uu - p * a.T;
        off = rbase[p] + (uint32_t)((j / a.rw) * a.W + j % a.rw) * rowb + ch * 16;
      }
      const uint4 kx = ld16(kr, off), vx = ld16(vr, off);
      *reinterpret_cast<uint4*>(kt_lds + kk * 64 + ch * 16) = kx;
      *reinterpret_cast<uint4*>(vt_lds + kk * 64 + ch * 16) = vx;
    }
  };
  const int r4 = col >> 2, c4 = col & 3;  // this lane's row and piece of the transposing reads

  // pass 1: forward with an online maximum
  float m = -__builtin_inff(), l = 0.f;
  f32x4 o[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int u0 = 0; u0 < a.L; u0 += kTile) {
    __syncthreads();
    load_tile(u0);
    __syncthreads();
    f32x4 sc[2];
    float mt = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      sc[kt] = mfma(*reinterpret_cast<const bf16x8*>(kt_lds + (16 * kt + col) * 64 + 16 * g), bq,
                    f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sc[kt][i] = u0 + 16 * kt + 4 * g + i < a.L ? sc[kt][i] * kQs : -__builtin_inff();
        mt = __builtin_elementwise_maximum(mt, sc[kt][i]);
      }
    }
    const float mn = __builtin_elementwise_maximum(m, group_max(mt));
    const float alpha = __builtin_amdgcn_exp2f(m - mn);
    l *= alpha;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int i = 0; i < 4; ++i) o[dt][i] *= alpha;
    bf16x4 p[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[kt][i] = (__bf16)__builtin_amdgcn_exp2f(sc[kt][i] - mn);
        l += (float)p[kt][i];
      }
    const bf16x8 pb = cat(p[0], p[1]);
    const char* v0 = vt_lds + (4 * g + r4) * 64 + 8 * c4;
    const char* v1 = vt_lds + (16 + 4 * g + r4) * 64 + 8 * c4;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) o[dt] = mfma(cat(ld_tr(v0 + 32 * dt), ld_tr(v1 + 32 * dt)), pb, o[dt]);
    m = mn;
  }
  l = group_sum(l);
  const float inv = 1.f / l;
  // D = G . O over the head's 32 channels (the lane holds 8 of them)
  float dpart = 0.f;
#pragma unroll
  for (int dt = 0; dt < 2; ++dt) {
    const uint32_t x0 = __builtin_amdgcn_raw_buffer_load_b32(gr, qoff + (16 * dt + 4 * g) * 2, 0, 0);
    const uint32_t x1 = __builtin_amdgcn_raw_buffer_load_b32(gr, qoff + (16 * dt + 4 * g) * 2 + 4, 0, 0);
    dpart = fmaf(o[dt][0], bf16_lo(x0), dpart);
    dpart = fmaf(o[dt][1], bf16_hi(x0), dpart);
    dpart = fmaf(o[dt][2], bf16_lo(x1), dpart);
    dpart = fmaf(o[dt][3], bf16_hi(x1), dpart);
  }
  const float D = group_sum(dpart) * inv;
  const float lse = m + __builtin_amdgcn_logf(l);  // base 2
  if (g == 0) {
    const size_t si = ((size_t)n * HW + qpix) * a.heads + h;
    a.lse[si] = lse;
    a.dsum[si] = D;
  }

  // pass 2: dQ^T += K^T dS^T
  f32x4 dqt[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  for (int u0 = 0; u0 < a.L; u0 += kTile) {
    __syncthreads();
    load_tile(u0);
    __syncthreads();
    bf16x4 ds[2];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt) {
      const f32x4 sc = mfma(*reinterpret_cast<const bf16x8*>(kt_lds + (16 * kt + col) * 64 + 16 * g), bq,
                            f32x4{0.f, 0.f, 0.f, 0.f});
      const f32x4 dp = mfma(*reinterpret_cast<const bf16x8*>(vt_lds + (16 * kt + col) * 64 + 16 * g), bg,
                            f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = u0 + 16 * kt + 4 * g + i < a.L ? __builtin_amdgcn_exp2f(fmaf(sc[i], kQs, -lse)) : 0.f;
        ds[kt][i] = (__bf16)(p * (dp[i] - D));
      }
    }
    const bf16x8 dsb = cat(ds[0], ds[1]);
    const char* k0 = kt_lds + (4 * g + r4) * 64 + 8 * c4;
    const char* k1 = kt_lds + (16 + 4 * g + r4) * 64 + 8 * c4;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) dqt[dt] = mfma(cat(ld_tr(k0 + 32 * dt), ld_tr(k1 + 32 * dt)), dsb, dqt[dt]);
  }
  float d0[4], d1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    d0[i] = dqt[0][i] * kScale;
    d1[i] = dqt[1][i] * kScale;
  }
  store_slice(dqr, qoff, g, d0, d1, true);
}

// ---------------------------------------------------------------- key side
template <int WAVES>
__global__ __launch_bounds__(64 * WAVES) void bwd_key_kernel(BwdArgs a) {
  __shared__ __attribute__((aligned(16))) char lds[2 * kTile * 64];  // Q tile | G tile
  __shared__ float st_lse[kTile], st_d[kTile];
  __shared__ float wl[25 * 32];  // the head's LCE weights, [tap][channel]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, g = lane >> 4;
  const int GPR = a.T / 16 / WAVES;
  int u = xcd_unit(blockIdx.x, gridDim.x);
  const int kg = u % GPR;
  u /= GPR;
  const int h = u % a.heads;
  u /= a.heads;
  const int s = u % a.R, n = u / a.R;
  const int HW = a.H * a.W;
  const uint32_t rowb = (uint32_t)a.C * 2, hoff = (uint32_t)h * 64;
  const size_t img = (size_t)n * HW * a.C;
  const uint32_t img_bytes = (uint32_t)HW * rowb;
  const Rsrc qr = rsrc(a.q + img, img_bytes), kr = rsrc(a.k + img, img_bytes), vr = rsrc(a.v + img, img_bytes);
  const Rsrc gr = rsrc(a.g + img, img_bytes);
  const Rsrc dkr = rsrc(a.dk + img, img_bytes), dvr = rsrc(a.dv + img, img_bytes);

  // this wave's 16 keys of region s: K and V rows as B operands
  const int j = 16 * (kg * WAVES + wave) + col;
  const int ky = (s / a.S) * a.rh + j / a.rw, kx = (s % a.S) * a.rw + j % a.rw;
  const uint32_t koff = (uint32_t)(ky * a.W + kx) * rowb + hoff;
  const bf16x8 bk = as8(ld16(kr, koff + 16 * g));
  const bf16x8 bv = as8(ld16(vr, koff + 16 * g));
  for (int e = tid; e < 25 * 32; e += 64 * WAVES) {
    const int tap = e >> 5, c = e & 31;
    wl[e] = bf16_bits_to_float(a.w[(size_t)(h * 32 + c) * 25 + tap]);
  }

  char* qt_lds = lds;
  char* gt_lds = lds + kTile * 64;
  const int r4 = col >> 2, c4 = col & 3;
  f32x4 dkt[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  f32x4 dvt[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
  const int beg = a.inv_off[(size_t)n * (a.R + 1) + s], end = a.inv_off[(size_t)n * (a.R + 1) + s + 1];
  for (int ei = beg; ei < end; ++ei) {
    const int r = a.inv_ent[(size_t)n * a.R * a.topk + ei];
    const int ry = (r / a.S) * a.rh, rx = (r % a.S) * a.rw;
    for (int t0 = 0; t0 < a.T; t0 += kTile) {
      __syncthreads();
      for (int e = tid; e < kTile * 4; e += 64 * WAVES) {  // query rows t0 .. t0+31 of region r
        const int kk = e >> 2, ch = e & 3, tq = t0 + kk;
        const uint32_t off = tq < a.T ? (uint32_t)((ry + tq / a.rw) * a.W + rx + tq % a.rw) * rowb + hoff + ch * 16
                                      : kOut;
        const uint4 qx = ld16(qr, off), gx = ld16(gr, off);
        *reinterpret_cast<uint4*>(qt_lds + kk * 64 + ch * 16) = qx;
        *reinterpret_cast<uint4*>(gt_lds + kk * 64 + ch * 16) = gx;
      }
      if (tid < kTile) {
        const int tq = t0 + tid;
        float lv = 0.f, dv_ = 0.f;
        if (tq < a.T) {
          const size_t si = ((size_t)n * HW + (ry + tq / a.rw) * a.W + rx + tq % a.rw) * a.heads + h;
          lv = a.lse[si];
          dv_ = a.dsum[si];
        }
        st_lse[tid] = lv;
        st_d[tid] = dv_;
      }
      __syncthreads();
      bf16x4 pb[2], dsb[2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const f32x4 sc = mfma(*reinterpret_cast<const bf16x8*>(qt_lds + (16 * qt + col) * 64 + 16 * g), bk,
                              f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 dp = mfma(*reinterpret_cast<const bf16x8*>(gt_lds + (16 * qt + col) * 64 + 16 * g), bv,
                              f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int qi = 16 * qt + 4 * g + i;
          const float p = t0 + qi < a.T ? __builtin_amdgcn_exp2f(fmaf(sc[i], kQs, -st_lse[qi])) : 0.f;
          pb[qt][i] = (__bf16)p;
          dsb[qt][i] = (__bf16)(p * (dp[i] - st_d[qi]));
        }
      }
      const bf16x8 pB = cat(pb[0], pb[1]), dsB = cat(dsb[0], dsb[1]);
      const int q0 = (4 * g + r4) * 64 + 8 * c4, q1 = (16 + 4 * g + r4) * 64 + 8 * c4;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        dvt[dt] = mfma(cat(ld_tr(gt_lds + q0 + 32 * dt), ld_tr(gt_lds + q1 + 32 * dt)), pB, dvt[dt]);
        dkt[dt] = mfma(cat(ld_tr(qt_lds + q0 + 32 * dt), ld_tr(qt_lds + q1 + 32 * dt)), dsB, dkt[dt]);
      }
    }
  }
  __syncthreads();  // the weights are in LDS
  // dV's LCE term: the key pixel feeds outputs (ky + 2 - a, kx + 2 - e) through tap (a, e)
  float lv0[4] = {0.f, 0.f, 0.f, 0.f}, lv1[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
  for (int ta = 0; ta < 5; ++ta) {  // one window row's loads in flight at a time
    const int yy = ky + 2 - ta;
#pragma unroll
    for (int te = 0; te < 5; ++te) {
      const int xx = kx + 2 - te;
      const bool in = yy >= 0 && yy < a.H && xx >= 0 && xx < a.W;
      const uint32_t go = in ? (uint32_t)(yy * a.W + xx) * rowb + hoff : kOut;
      const float* wt = wl + (5 * ta + te) * 32;
      const uint32_t g0a = __builtin_amdgcn_raw_buffer_load_b32(gr, go + 8 * g, 0, 0);
      const uint32_t g0b = __builtin_amdgcn_raw_buffer_load_b32(gr, go + 8 * g + 4, 0, 0);
      const uint32_t g1a = __builtin_amdgcn_raw_buffer_load_b32(gr, go + 32 + 8 * g, 0, 0);
      const uint32_t g1b = __builtin_amdgcn_raw_buffer_load_b32(gr, go + 32 + 8 * g + 4, 0, 0);
      lv0[0] = fmaf(wt[4 * g + 0], bf16_lo(g0a), lv0[0]);
      lv0[1] = fmaf(wt[4 * g + 1], bf16_hi(g0a), lv0[1]);
      lv0[2] = fmaf(wt[4 * g + 2], bf16_lo(g0b), lv0[2]);
      lv0[3] = fmaf(wt[4 * g + 3], bf16_hi(g0b), lv0[3]);
      lv1[0] = fmaf(wt[16 + 4 * g + 0], bf16_lo(g1a), lv1[0]);
      lv1[1] = fmaf(wt[16 + 4 * g + 1], bf16_hi(g1a), lv1[1]);
      lv1[2] = fmaf(wt[16 + 4 * g + 2], bf16_lo(g1b), lv1[2]);
      lv1[3] = fmaf(wt[16 + 4 * g + 3], bf16_hi(g1b), lv1[3]);
    }
  }
  float k0[4], k1[4], v0[4], v1[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    k0[i] = dkt[0][i] * kScale;
    k1[i] = dkt[1][i] * kScale;
    v0[i] = dvt[0][i] + lv0[i];
    v1[i] = dvt[1][i] + lv1[i];
  }
  store_slice(dkr, koff, g, k0, k1, true);
  store_slice(dvr, koff, g, v0, v1, true);
}

// ---------------------------------------------------------------- LCE weights
// Row (n, y), channel c: the 25 tap sums sum_x dout[y][x][c] * v[y+a-2][x+e-2][c]
// and the bias sum, into part[(n*H + y)][c][26].
__global__ __launch_bounds__(256) void lce_grad_rows_kernel(const uint16_t* __restrict__ v,
                                                            const uint16_t* __restrict__ g, int H, int W, int C,
                                                            float* __restrict__ part) {
  const int ny = blockIdx.x, n = ny / H, y = ny - n * H;
  const size_t img = (size_t)n * H * W * C;
  for (int c = threadIdx.x; c < C; c += blockDim.x) {
    float acc[25], accb = 0.f;
#pragma unroll
    for (int i = 0; i < 25; ++i) acc[i] = 0.f;
    for (int x = 0; x < W; ++x) {
      const float gv = bf16_bits_to_float(g[img + ((size_t)y * W + x) * C + c]);
      accb += gv;
#pragma unroll
      for (int ta = 0; ta < 5; ++ta) {
        const int yy = y + ta - 2;
        if (yy < 0 || yy >= H) continue;
#pragma unroll
        for (int te = 0; te < 5; ++te) {
          const int xx = x + te - 2;
          if (xx < 0 || xx >= W) continue;
          acc[5 * ta + te] = fmaf(gv, bf16_bits_to_float(v[img + ((size_t)yy * W + xx) * C + c]), acc[5 * ta + te]);
        }
      }
    }
    float* o = part + ((size_t)ny * C + c) * 26;
#pragma unroll
    for (int i = 0; i < 25; ++i) o[i] = acc[i];
    o[25] = accb;
  }
}

// dw[c][tap] and db[c]: the row partials summed in row order
__global__ __launch_bounds__(256) void lce_grad_sum_kernel(const float* __restrict__ part, int rows, int C,
                                                           float* __restrict__ dw, float* __restrict__ db) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;  // c * 26 + tap
  if (e >= C * 26) return;
  float acc = 0.f;
  for (int r = 0; r < rows; ++r) acc += part[(size_t)r * C * 26 + e];
  const int c = e / 26, tap = e - c * 26;
  if (tap < 25) dw[(size_t)c * 25 + tap] = acc;
  else if (db) db[c] = acc;
}

template <int WAVES>
hipError_t launch_sides(const BwdArgs& a, hipStream_t st) {
  const unsigned units = (unsigned)(a.N * a.R * a.heads * (a.T / 16 / WAVES));
  launch(bwd_query_kernel<WAVES>, dim3(units), dim3(64 * WAVES), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch(bwd_key_kernel<WAVES>, dim3(units), dim3(64 * WAVES), 0, st, a);
  return hipGetLastError();
}

}  // namespace

bool backward_supports(const Shape& s, int dtype) {
  return dtype == 1 && s.hd == 32 && s.T % 16 == 0 && s.topk <= 16 && s.R <= 1024;
}

size_t backward_workspace_bytes(const Shape& s) {
  const size_t stats = (size_t)s.N * s.H * s.W * s.heads * sizeof(float);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return 2 * al(stats) + al((size_t)s.N * (s.R + 1) * 4) + al((size_t)s.N * s.R * s.topk * 4) +
         al((size_t)s.N * s.H * s.C * 26 * sizeof(float));
}

hipError_t launch_backward(const void* q, const void* k, const void* v, const void* w, const int32_t* route,
                           const void* dout, const Shape& s, void* dq, void* dk, void* dv, float* dw, float* db,
                           void* ws, hipStream_t st) {
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  char* p = static_cast<char*>(ws);
  const size_t stats = (size_t)s.N * s.H * s.W * s.heads * sizeof(float);
  BwdArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.g = (const uint16_t*)dout;
  a.w = (const uint16_t*)w;
  a.route = route;
  a.lse = reinterpret_cast<float*>(p);
  p += al(stats);
  a.dsum = reinterpret_cast<float*>(p);
  p += al(stats);
  int32_t* off = reinterpret_cast<int32_t*>(p);
  p += al((size_t)s.N * (s.R + 1) * 4);
  int32_t* ent = reinterpret_cast<int32_t*>(p);
  p += al((size_t)s.N * s.R * s.topk * 4);
  float* part = reinterpret_cast<float*>(p);
  a.inv_off = off;
  a.inv_ent = ent;
  a.dq = (uint16_t*)dq;
  a.dk = (uint16_t*)dk;
  a.dv = (uint16_t*)dv;
  a.N = s.N; a.H = s.H; a.W = s.W; a.C = s.C; a.heads = s.heads; a.S = s.S; a.topk = s.topk;
  a.R = s.R; a.rh = s.rh; a.rw = s.rw; a.T = s.T; a.L = s.L;

  launch(inv_route_kernel, dim3((unsigned)s.N), dim3(256), (size_t)s.R * sizeof(int), st, route, s.R, s.topk, off,
         ent);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int qgroups = s.T / 16;
  e = qgroups % 4 == 0 ? launch_sides<4>(a, st) : qgroups % 2 == 0 ? launch_sides<2>(a, st) : launch_sides<1>(a, st);
  if (e != hipSuccess) return e;
  launch(lce_grad_rows_kernel, dim3((unsigned)(s.N * s.H)), dim3(s.C < 256 ? ((s.C + 63) / 64) * 64 : 256), 0, st,
         (const uint16_t*)v, (const uint16_t*)dout, s.H, s.W, s.C, part);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch(lce_grad_sum_kernel, dim3((unsigned)((s.C * 26 + 255) / 256)), dim3(256), 0, st, (const float*)part,
         s.N * s.H, s.C, dw, db);
  return hipGetLastError();
}

}  // namespace bra
