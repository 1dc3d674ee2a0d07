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
//  * inv_route_kernel: per (image, region), the regions that route to it, in
//    ascending order, so the key side gathers instead of scattering and
//    every gradient is a fixed-order sum (no atomics).
//  * bwd_query_kernel: one workgroup per (image, region, head, group of
//    query blocks), a wave per one or two 16-query blocks (the whole 256-token
//    region in one workgroup of 8 waves where the region allows it); tiles of
//    64 or 128 gathered keys (K and V) staged in LDS through registers, one
//    tile ahead, and shared by the waves. Pass 1 is the forward with an
//    online maximum (S^T = K Q^T, O^T = V^T P^T on 16x16x32 bf16 products,
//    row sums on the matrix cores) and leaves per query the base-2
//    log-sum-exp and D = G . O; pass 2 recomputes P and forms dP^T = V G^T,
//    dS^T, and dQ^T += K^T dS^T (K^T by transposing LDS reads, dS^T from the
//    lane's own eight keys, the same key order on both operands).
//  * bwd_key_kernel: the same decomposition over key blocks; for every
//    router region, tiles of its queries' Q and G (and their log-sum-exp and
//    D) staged in LDS: S = Q K^T and dP = G V^T with lane = key, P and dS
//    from the saved statistics, dV^T += G^T P and dK^T += Q^T dS (Q^T, G^T
//    by transposing LDS reads); then it adds dV's LCE term.
//    Whether the last tile can be partial is a template parameter, so whole
//    tiles run without masks.
//  * lce_grad_rows_kernel / lce_grad_sum_kernel: per block of image rows and
//    of 8 channels, the 25 tap sums, the bias sum and dV's LCE term (dout
//    correlated with the flipped 5x5 kernel); then a fixed-order sum of the
//    tap and bias sums over the row blocks.
#include "bra_internal.h"

namespace bra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kBwdMaxWaves = 8;  // waves of a backward workgroup, at most
constexpr float kQs = 0.17677669529663687f * 1.4426950408889634f;  // hd^-1/2 in log2 units
constexpr float kScale = 0.17677669529663687f;                     // hd^-1/2

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* g;   // dout
  const uint16_t* w;   // LCE weights [C][25]
  const int32_t* route;
  const int32_t* inv_cnt;  // [N][R]: routers of each region
  const int32_t* inv_ent;  // [N][R][R]: their indices, ascending
  float* lse;              // [N][H*W][heads], base 2
  float* dsum;             // [N][H*W][heads]
  const float* dv_lce;     // [N][C/8][H][W][8]: dv's LCE term, channel blocks of 8
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
  const uint32_t la[2] = {pack_bf16x2(a[0], a[1]),
                          pack_bf16x2(a[2], a[3])};
  const uint32_t hb[2] = {pack_bf16x2(b[0], b[1]),
                          pack_bf16x2(b[2], b[3])};
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
// One wave per (image, region s): the routers of s (the regions r whose row
// of the route table holds s) in ascending order of r, at most R of them (a
// row's routes are distinct), into ent[n][s][0 .. cnt-1]: the wave walks the
// image's table 64 entries at a time and compacts the matches with a ballot.
__global__ __launch_bounds__(64) void inv_route_kernel(const int32_t* __restrict__ route, int R, int topk,
                                                       int32_t* __restrict__ cnt, int32_t* __restrict__ ent) {
  const int ns = blockIdx.x, n = ns / R, s = ns - n * R, lane = threadIdx.x;
  const int RK = R * topk;
  const int32_t* rt = route + (size_t)n * RK;
  int32_t* out = ent + (size_t)ns * R;
  int c = 0;
  for (int e0 = 0; e0 < RK; e0 += 64) {
    const int e = e0 + lane;
    const bool hit = e < RK && rt[e] == s;
    const uint64_t mask = __ballot(hit);
    if (hit) out[c + __builtin_popcountll(mask & ((1ull << lane) - 1))] = e / topk;
    c += __builtin_popcountll(mask);
  }
  if (lane == 0) cnt[ns] = c;
}

// ---------------------------------------------------------------- query side
// Rows [0, TILE) of two [TILE][64-byte] LDS tiles, loaded as 16-byte pieces:
// thread `tid` of `threads` holds pieces tid, tid + threads, ... (PPT of
// them) in registers between the load and the store, so the next tile's loads
// are in flight while the current tile is used.
template <int TILE, int THREADS>
struct TilePair {
  static constexpr int PPT = (TILE * 4 + THREADS - 1) / THREADS;
  uint4 a[PPT], b[PPT];
};

template <int WAVES, int TK, int QB, bool FULL>
__global__ __launch_bounds__(64 * WAVES) void bwd_query_kernel(BwdArgs a) {
  // FULL: every key tile is whole (L a multiple of TK), so no key is masked
  // QB 16-query blocks a wave: every K / V / K^T / V^T operand read from LDS
  // serves all of them
  constexpr int TH = 64 * WAVES;
  __shared__ __attribute__((aligned(16))) char lds[2 * TK * 64];  // K tile | V tile, [TK][64 bytes]
  __shared__ uint32_t rbase[16];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, g = lane >> 4;
  const int GPR = a.T / 16 / (WAVES * QB);  // query groups of a region
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

  // this wave's QB blocks of 16 queries of region r
  int qpix[QB];
  uint32_t qoff[QB];
  bf16x8 bq[QB], bg[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const int t = 16 * ((qg * WAVES + wave) * QB + b) + col;
    qpix[b] = ((r / a.S) * a.rh + t / a.rw) * a.W + (r % a.S) * a.rw + t % a.rw;
    qoff[b] = (uint32_t)qpix[b] * rowb + hoff;
    bq[b] = as8(ld16(qr, qoff[b] + 16 * g));
    bg[b] = as8(ld16(gr, qoff[b] + 16 * g));
  }
  if (tid < a.topk) {
    const int s = a.route[((size_t)n * a.R + r) * a.topk + tid];
    rbase[tid] = (uint32_t)(((s / a.S) * a.rh * a.W + (s % a.S) * a.rw)) * rowb + hoff;
  }
  __syncthreads();

  char* kt_lds = lds;
  char* vt_lds = lds + TK * 64;
  TilePair<TK, TH> pre;
  auto fetch = [&](int u0) {  // keys u0 .. u0+TK-1 of the gathered sequence (past L: zeros)
#pragma unroll
    for (int i = 0; i < TilePair<TK, TH>::PPT; ++i) {
      const int e = tid + i * TH, kk = e >> 2, ch = e & 3, uu = u0 + kk;
      uint32_t off = kOut;
      if (e < TK * 4 && uu < a.L) {
        const int p = uu / a.T, j = uu - p * a.T;
        off = rbase[p] + (uint32_t)((j / a.rw) * a.W + j % a.rw) * rowb + ch * 16;
      }
      pre.a[i] = ld16(kr, off);
      pre.b[i] = ld16(vr, off);
    }
  };
  auto park = [&]() {
#pragma unroll
    for (int i = 0; i < TilePair<TK, TH>::PPT; ++i) {
      const int e = tid + i * TH;
      if (e < TK * 4) {
        *reinterpret_cast<uint4*>(kt_lds + e * 16) = pre.a[i];
        *reinterpret_cast<uint4*>(vt_lds + e * 16) = pre.b[i];
      }
    }
  };
  const int r4 = col >> 2, c4 = col & 3;  // this lane's row and piece of the transposing reads
  constexpr int KS = TK / 32;             // 32-key steps of a tile

  // pass 1: forward with an online maximum (one maximum a tile); the row
  // sums of the bf16 P on the matrix cores (ones x P^T). Only the last tile
  // can hold keys past L; the others skip the masks.
  const bf16x8 ones = {(__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f,
                       (__bf16)1.f, (__bf16)1.f, (__bf16)1.f, (__bf16)1.f};
  float m[QB];
  f32x4 o[QB][2], lsum[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    m[b] = -__builtin_inff();
    o[b][0] = o[b][1] = lsum[b] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto tile1 = [&](int u0) {
    f32x4 sc[QB][2 * KS];
    float mt[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) mt[b] = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < 2 * KS; ++kt) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kt_lds + (16 * kt + col) * 64 + 16 * g);
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        sc[b][kt] = mfma(ka, bq[b], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if constexpr (!FULL)
            if (u0 + 16 * kt + 4 * g + i >= a.L) sc[b][kt][i] = -__builtin_inff();
          mt[b] = __builtin_elementwise_maximum(mt[b], sc[b][kt][i]);
        }
      }
    }
    float mn[QB];
#pragma unroll
    for (int b = 0; b < QB; ++b) {
      mn[b] = __builtin_elementwise_maximum(m[b], group_max(mt[b]) * kQs);  // the scale is positive
      const float alpha = __builtin_amdgcn_exp2f(m[b] - mn[b]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        o[b][0][i] *= alpha;
        o[b][1][i] *= alpha;
        lsum[b][i] *= alpha;
      }
      m[b] = mn[b];
    }
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x8 pb[QB];
#pragma unroll
      for (int b = 0; b < QB; ++b) {
        bf16x4 p[2];
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            p[j][i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sc[b][2 * ks + j][i], kQs, -mn[b]));
        pb[b] = cat(p[0], p[1]);
        lsum[b] = mfma(ones, pb[b], lsum[b]);
      }
      const char* v0 = vt_lds + (32 * ks + 4 * g + r4) * 64 + 8 * c4;
      const char* v1 = vt_lds + (32 * ks + 16 + 4 * g + r4) * 64 + 8 * c4;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const bf16x8 va = cat(ld_tr(v0 + 32 * dt), ld_tr(v1 + 32 * dt));
#pragma unroll
        for (int b = 0; b < QB; ++b) o[b][dt] = mfma(va, pb[b], o[b][dt]);
      }
    }
  };
  fetch(0);
  for (int u0 = 0; u0 < a.L; u0 += TK) {
    __syncthreads();
    park();
    __syncthreads();
    if (u0 + TK < a.L) fetch(u0 + TK);
    tile1(u0);
  }
  float lse[QB], D[QB];
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    const float lb = lsum[b][0];
    // D = G . O over the head's 32 channels (the lane holds 8 of them)
    float dpart = 0.f;
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const uint32_t x0 = __builtin_amdgcn_raw_buffer_load_b32(gr, qoff[b] + (16 * dt + 4 * g) * 2, 0, 0);
      const uint32_t x1 = __builtin_amdgcn_raw_buffer_load_b32(gr, qoff[b] + (16 * dt + 4 * g) * 2 + 4, 0, 0);
      dpart = fmaf(o[b][dt][0], bf16_lo(x0), dpart);
      dpart = fmaf(o[b][dt][1], bf16_hi(x0), dpart);
      dpart = fmaf(o[b][dt][2], bf16_lo(x1), dpart);
      dpart = fmaf(o[b][dt][3], bf16_hi(x1), dpart);
    }
    D[b] = group_sum(dpart) / lb;
    lse[b] = m[b] + __builtin_amdgcn_logf(lb);  // base 2
    if (g == 0) {
      const size_t si = ((size_t)n * HW + qpix[b]) * a.heads + h;
      a.lse[si] = lse[b];
      a.dsum[si] = D[b];
    }
  }

  // pass 2: dQ^T += K^T dS^T. The dP products start from -D, so
  // dS = P * dP' takes no subtraction. (The scores are scaled in fp32: a
  // query rounded to bf16 after scaling, as the forward's large-region
  // kernel takes it, moves P by up to ~2^-9 |score| relative, which dS
  // passes on to the gradients undamped.)
  f32x4 dqt[QB][2];
#pragma unroll
  for (int b = 0; b < QB; ++b) dqt[b][0] = dqt[b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  auto tile2 = [&](int u0) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      bf16x4 ds[QB][2];
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int row = 32 * ks + 16 * j + col;
        const bf16x8 ka = *reinterpret_cast<const bf16x8*>(kt_lds + row * 64 + 16 * g);
        const bf16x8 vb = *reinterpret_cast<const bf16x8*>(vt_lds + row * 64 + 16 * g);
#pragma unroll
        for (int b = 0; b < QB; ++b) {
          const f32x4 sc = mfma(ka, bq[b], f32x4{0.f, 0.f, 0.f, 0.f});
          const f32x4 dp = mfma(vb, bg[b], f32x4{-D[b], -D[b], -D[b], -D[b]});
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float p = __builtin_amdgcn_exp2f(fmaf(sc[i], kQs, -lse[b]));
            if constexpr (!FULL)
              if (u0 + 32 * ks + 16 * j + 4 * g + i >= a.L) p = 0.f;
            ds[b][j][i] = (__bf16)(p * dp[i]);
          }
        }
      }
      const char* k0 = kt_lds + (32 * ks + 4 * g + r4) * 64 + 8 * c4;
      const char* k1 = kt_lds + (32 * ks + 16 + 4 * g + r4) * 64 + 8 * c4;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const bf16x8 ka = cat(ld_tr(k0 + 32 * dt), ld_tr(k1 + 32 * dt));
#pragma unroll
        for (int b = 0; b < QB; ++b) dqt[b][dt] = mfma(ka, cat(ds[b][0], ds[b][1]), dqt[b][dt]);
      }
    }
  };
  fetch(0);
  for (int u0 = 0; u0 < a.L; u0 += TK) {
    __syncthreads();
    park();
    __syncthreads();
    if (u0 + TK < a.L) fetch(u0 + TK);
    tile2(u0);
  }
#pragma unroll
  for (int b = 0; b < QB; ++b) {
    float d0[4], d1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      d0[i] = dqt[b][0][i] * kScale;
      d1[i] = dqt[b][1][i] * kScale;
    }
    store_slice(dqr, qoff[b], g, d0, d1, true);
  }
}

// ---------------------------------------------------------------- key side
// (8 waves: at most 128 VGPRs, so two workgroups share a CU; the few values
// this spills are the epilogue's and the tile loader's, not the products')
template <int WAVES, int TQ, int KB, bool FULL>
__global__ __launch_bounds__(64 * WAVES, WAVES == 8 ? 4 : 1) void bwd_key_kernel(BwdArgs a) {
  // FULL: every query tile is whole (T a multiple of TQ), so no query is masked
  // KB 16-key blocks a wave: every Q / G / Q^T / G^T operand read from LDS
  // serves all of them
  constexpr int TH = 64 * WAVES;
  __shared__ __attribute__((aligned(16))) char lds[2 * TQ * 64];  // Q tile | G tile
  __shared__ __attribute__((aligned(16))) float st_lse[TQ];  // LSE of the staged queries
  __shared__ __attribute__((aligned(16))) float st_d[TQ];    // D of the staged queries
  __shared__ int routers[1024];  // the regions routing to s, ascending
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, g = lane >> 4;
  const int GPR = a.T / 16 / (WAVES * KB);
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

  // this wave's KB blocks of 16 keys of region s: K and V rows as B operands
  int ky[KB], kx[KB];
  uint32_t koff[KB];
  bf16x8 bk[KB], bv[KB];
#pragma unroll
  for (int b = 0; b < KB; ++b) {
    const int j = 16 * ((kg * WAVES + wave) * KB + b) + col;
    ky[b] = (s / a.S) * a.rh + j / a.rw;
    kx[b] = (s % a.S) * a.rw + j % a.rw;
    koff[b] = (uint32_t)(ky[b] * a.W + kx[b]) * rowb + hoff;
    bk[b] = as8(ld16(kr, koff[b] + 16 * g));
    bv[b] = as8(ld16(vr, koff[b] + 16 * g));
  }
  const int nrout = a.inv_cnt[(size_t)n * a.R + s];
  for (int e = tid; e < nrout; e += TH) routers[e] = a.inv_ent[((size_t)n * a.R + s) * a.R + e];
  __syncthreads();

  char* qt_lds = lds;
  char* gt_lds = lds + TQ * 64;
  const int r4 = col >> 2, c4 = col & 3;
  constexpr int QS = TQ / 32;
  f32x4 dkt[KB][2], dvt[KB][2];
#pragma unroll
  for (int b = 0; b < KB; ++b) dkt[b][0] = dkt[b][1] = dvt[b][0] = dvt[b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  const int tiles_per_router = (a.T + TQ - 1) / TQ, ntiles = nrout * tiles_per_router;
  TilePair<TQ, TH> pre;
  float pl = 0.f, pd = 0.f;  // the statistics of query tid of the prefetched tile
  auto fetch = [&](int it) {  // tile it: router it / tiles_per_router, its queries t0 .. t0+TQ-1
    const int r = routers[it / tiles_per_router];
    const int t0 = (it % tiles_per_router) * TQ;
    const int ry = (r / a.S) * a.rh, rx = (r % a.S) * a.rw;
#pragma unroll
    for (int i = 0; i < TilePair<TQ, TH>::PPT; ++i) {
      const int e = tid + i * TH, kk = e >> 2, ch = e & 3, tq = t0 + kk;
      const uint32_t off = e < TQ * 4 && tq < a.T
                               ? (uint32_t)((ry + tq / a.rw) * a.W + rx + tq % a.rw) * rowb + hoff + ch * 16
                               : kOut;
      pre.a[i] = ld16(qr, off);
      pre.b[i] = ld16(gr, off);
    }
    pl = pd = 0.f;
    if (tid < TQ && t0 + tid < a.T) {
      const int tq = t0 + tid;
      const size_t si = ((size_t)n * HW + (ry + tq / a.rw) * a.W + rx + tq % a.rw) * a.heads + h;
      pl = a.lse[si];
      pd = a.dsum[si];
    }
  };
  auto ktile = [&](int t0) {
#pragma unroll
    for (int qs = 0; qs < QS; ++qs) {
      bf16x4 pb[KB][2], dsb[KB][2];
#pragma unroll
      for (int qt = 0; qt < 2; ++qt) {
        const int row = 32 * qs + 16 * qt + col;
        const bf16x8 qa = *reinterpret_cast<const bf16x8*>(qt_lds + row * 64 + 16 * g);
        const bf16x8 ga = *reinterpret_cast<const bf16x8*>(gt_lds + row * 64 + 16 * g);
        const int q4 = 32 * qs + 16 * qt + 4 * g;  // this lane's four query rows
        const f32x4 lq = *reinterpret_cast<const f32x4*>(st_lse + q4);
        const f32x4 dq4 = *reinterpret_cast<const f32x4*>(st_d + q4);
#pragma unroll
        for (int b = 0; b < KB; ++b) {
          const f32x4 sc = mfma(qa, bk[b], f32x4{0.f, 0.f, 0.f, 0.f});
          const f32x4 dp = mfma(ga, bv[b], f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            float p = __builtin_amdgcn_exp2f(fmaf(sc[i], kQs, -lq[i]));
            if constexpr (!FULL)
              if (t0 + q4 + i >= a.T) p = 0.f;
            pb[b][qt][i] = (__bf16)p;
            dsb[b][qt][i] = (__bf16)(p * (dp[i] - dq4[i]));
          }
        }
      }
      const int q0 = (32 * qs + 4 * g + r4) * 64 + 8 * c4, q1 = (32 * qs + 16 + 4 * g + r4) * 64 + 8 * c4;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) {
        const bf16x8 gta = cat(ld_tr(gt_lds + q0 + 32 * dt), ld_tr(gt_lds + q1 + 32 * dt));
        const bf16x8 qta = cat(ld_tr(qt_lds + q0 + 32 * dt), ld_tr(qt_lds + q1 + 32 * dt));
#pragma unroll
        for (int b = 0; b < KB; ++b) {
          dvt[b][dt] = mfma(gta, cat(pb[b][0], pb[b][1]), dvt[b][dt]);
          dkt[b][dt] = mfma(qta, cat(dsb[b][0], dsb[b][1]), dkt[b][dt]);
        }
      }
    }
  };
  if (ntiles > 0) fetch(0);
  for (int it = 0; it < ntiles; ++it) {
    const int t0 = (it % tiles_per_router) * TQ;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < TilePair<TQ, TH>::PPT; ++i) {
      const int e = tid + i * TH;
      if (e < TQ * 4) {
        *reinterpret_cast<uint4*>(qt_lds + e * 16) = pre.a[i];
        *reinterpret_cast<uint4*>(gt_lds + e * 16) = pre.b[i];
      }
    }
    if (tid < TQ) {
      st_lse[tid] = pl;
      st_d[tid] = pd;
    }
    __syncthreads();
    if (it + 1 < ntiles) fetch(it + 1);
    ktile(t0);
  }
  // dV's LCE term, computed beforehand in fp32 ([N][C/8][H][W][8])
#pragma unroll
  for (int b = 0; b < KB; ++b) {
    auto lce4 = [&](int ch) {  // channels ch .. ch+3 of the key pixel
      return *reinterpret_cast<const f32x4*>(
          a.dv_lce + ((((size_t)n * (a.C / 8) + ch / 8) * a.H + ky[b]) * a.W + kx[b]) * 8 + ch % 8);
    };
    const f32x4 lv0 = lce4(h * 32 + 4 * g);
    const f32x4 lv1 = lce4(h * 32 + 16 + 4 * g);
    float k0[4], k1[4], v0[4], v1[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      k0[i] = dkt[b][0][i] * kScale;
      k1[i] = dkt[b][1][i] * kScale;
      v0[i] = dvt[b][0][i] + lv0[i];
      v1[i] = dvt[b][1][i] + lv1[i];
    }
    store_slice(dkr, koff[b], g, k0, k1, true);
    store_slice(dvr, koff[b], g, v0, v1, true);
  }
}

// ---------------------------------------------------------------- LCE terms
// One workgroup per (image, block of rows, block of kLceCh channels): the V
// rows and the dout rows of the block and two more on each side are staged in
// LDS channel-major, [row][channel][column] bf16 (column x at x + 2, zero
// outside the image and for kLceRun + pad columns past W + 2), so a 32-bit
// read is a horizontal pixel pair of one channel: one v_dot2_f32_bf16 then
// applies two taps, and an odd-aligned pair is one v_alignbyte of two even
// ones. Thread (channel c, group xg) walks (row, run of kLceRun = 4
// columns) items xg, xg + XG, ... (XG column groups: 32, or 64 for images
// at least 32 columns wide, whose eight staged rows are then walked by
// twice the waves); per window row ta it reads the eight
// V and eight dout values of the run's window as four even pairs each and
// adds, over the run,
//   the 25 tap terms dout[y][x] * v[y+ta-2][x+te-2]  (pairs of x), and
//   dv's LCE term w[ta][te] * dout[y-ta+2][x-te+2]    (pairs of taps te),
// plus the bias term (sum of dout). The column groups' tap sums are then
// added in a fixed order into part[block][c][26], and dv's LCE term is
// written in fp32 by channel block, [N][C/8][H][W][8] (a block's writes are
// whole rows; the key side adds it to the attention part). Images up to 32
// rows tall are one block each (the halo rows are then read once); taller
// ones go in blocks of 8 rows.
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), c, false);
}

constexpr int kLceCh = 8;                 // channels of a block: one 16-byte piece a pixel
constexpr int kLceRun = 4;                // consecutive columns a thread takes at once
constexpr int kLceBatch = 4;              // staged pixel pairs of each tensor a thread has in flight
constexpr int kLceRowsTall = 8;           // rows of a block of a tall image
constexpr int kLceRowsWhole = 32;         // images up to this height: one block
constexpr size_t kLceStageMax = 64 * 1024;
// staged row pitch in bf16 columns: W + 4 + kLceRun, rounded to 4 (8-byte
// pair reads); for images at least 32 columns wide (a wave's eight column
// groups then read one row) raised to 32 mod 64, so the eight channels'
// 8-byte reads of a wave start 16 banks apart and take the minimum two
// passes
__host__ __device__ inline int lce_pitch(int W) {
  int p = (W + 4 + kLceRun + 3) & ~3;
  if (W >= 8 * kLceRun) p += (96 - p % 64) % 64;
  return p;
}
__host__ __device__ inline size_t lce_stage_bytes(int rows, int W) {
  return (size_t)2 * (rows + 4) * kLceCh * lce_pitch(W) * 2;
}
__host__ __device__ inline int lce_rows(int H, int W) {
  return H <= kLceRowsWhole && lce_stage_bytes(H, W) <= kLceStageMax ? H : kLceRowsTall;
}
__host__ __device__ inline int lce_groups(int W) { return W >= 8 * kLceRun ? 64 : 32; }
__host__ __device__ inline size_t lce_grad_lds(int H, int W) {
  const size_t stage = lce_stage_bytes(lce_rows(H, W), W);
  const size_t red = (size_t)lce_groups(W) * kLceCh * 26 * sizeof(float);
  return stage > red ? stage : red;
}

struct LceArgs {
  const uint16_t* v;
  const uint16_t* g;
  const uint16_t* lw;
  int N, H, W, C, rows;  // rows: output rows of a block
  FastDiv dpp;           // staged pixel pairs a row (lce_pitch / 2)
  FastDiv druns;         // runs of kLceRun columns a row
  float* part;
  float* dv_lce;
};

// row blocks of an image
__host__ __device__ inline int lce_blocks(int H, int W) { return (H + lce_rows(H, W) - 1) / lce_rows(H, W); }

template <int XG>
__global__ __launch_bounds__(XG * kLceCh) void lce_grad_rows_kernel(LceArgs a) {
  constexpr int NT = XG * kLceCh;
  extern __shared__ __attribute__((aligned(16))) char sm[];
  const int H = a.H, W = a.W, C = a.C, BR = a.rows;
  const int YB = (H + BR - 1) / BR, CB = C / kLceCh;
  // consecutive units -- the CB channel blocks of one row block, which read
  // the same 128-byte pixel lines 16 bytes each -- share an XCD and its L2
  int u = xcd_unit((int)blockIdx.x, (int)gridDim.x);
  const int cb = u % CB;
  u /= CB;
  const int yb = u % YB, n = u / YB;
  const int y0 = yb * BR, tid = threadIdx.x;
  const int WP = lce_pitch(W), PP = WP / 2, SR = BR + 4;
  uint32_t* vs = reinterpret_cast<uint32_t*>(sm);  // [SR][kLceCh][PP] pixel pairs
  uint32_t* gs = vs + (size_t)SR * kLceCh * PP;
  const size_t img = (size_t)n * H * W * C;
  const uint32_t img_bytes = (uint32_t)((size_t)H * W * C * 2);
  const Rsrc vr = rsrc(a.v + img, img_bytes), gr = rsrc(a.g + img, img_bytes);
  const uint32_t cofs = (uint32_t)cb * kLceCh * 2;
  const int c = tid % kLceCh, xg = tid / kLceCh;
  // the channel's weights as dot2 operands for each window row ta: taps
  // (4, 3) and (2, 1) against the pairs (x-2, x-1) and (x, x+1) of an output
  // x, and tap 0 alone against (x+2, x+3) or (x+1, x+2)
  uint32_t w43[5], w21[5], w0l[5], w0h[5];
  {
    const uint16_t* wc = a.lw + (size_t)(cb * kLceCh + c) * 25;
#pragma unroll
    for (int ta = 0; ta < 5; ++ta) {
      const uint32_t t0 = wc[5 * ta], t1 = wc[5 * ta + 1], t2 = wc[5 * ta + 2], t3 = wc[5 * ta + 3],
                     t4 = wc[5 * ta + 4];
      w43[ta] = t4 | (t3 << 16);
      w21[ta] = t2 | (t1 << 16);
      w0l[ta] = t0;
      w0h[ta] = t0 << 16;
    }
  }
  // staging: pixel pairs (2p - 2, 2p - 1) of staged row ry (image row
  // y0 + ry - 2), both tensors; the eight channels of the two 16-byte
  // pieces become eight channel pairs
  const int units = SR * PP;
  for (int e0 = tid; e0 < units; e0 += NT * kLceBatch) {
    uint4 va[kLceBatch], vb[kLceBatch], ga[kLceBatch], gb[kLceBatch];
#pragma unroll
    for (int i = 0; i < kLceBatch; ++i) {
      const int e = e0 + NT * i, ry = (int)fdiv(a.dpp, (uint32_t)e), p = e - ry * PP;
      const int y = y0 + ry - 2, xa = 2 * p - 2;
      const bool row_in = e < units && y >= 0 && y < H;
      const uint32_t oa = row_in && xa >= 0 && xa < W ? (uint32_t)((y * W + xa) * C * 2) + cofs : kOut;
      const uint32_t ob = row_in && xa + 1 >= 0 && xa + 1 < W ? (uint32_t)((y * W + xa + 1) * C * 2) + cofs : kOut;
      va[i] = ld16(vr, oa);
      vb[i] = ld16(vr, ob);
      ga[i] = ld16(gr, oa);
      gb[i] = ld16(gr, ob);
    }
#pragma unroll
    for (int i = 0; i < kLceBatch; ++i) {
      const int e = e0 + NT * i;
      if (e < units) {
        const int ry = (int)fdiv(a.dpp, (uint32_t)e), p = e - ry * PP;
        uint32_t* vd = vs + (size_t)ry * kLceCh * PP + p;
        uint32_t* gd = gs + (size_t)ry * kLceCh * PP + p;
        const uint32_t av[4] = {va[i].x, va[i].y, va[i].z, va[i].w}, bv[4] = {vb[i].x, vb[i].y, vb[i].z, vb[i].w};
        const uint32_t ag[4] = {ga[i].x, ga[i].y, ga[i].z, ga[i].w}, bg[4] = {gb[i].x, gb[i].y, gb[i].z, gb[i].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          vd[(2 * k) * PP] = __builtin_amdgcn_perm(bv[k], av[k], 0x05040100u);
          vd[(2 * k + 1) * PP] = __builtin_amdgcn_perm(bv[k], av[k], 0x07060302u);
          gd[(2 * k) * PP] = __builtin_amdgcn_perm(bg[k], ag[k], 0x05040100u);
          gd[(2 * k + 1) * PP] = __builtin_amdgcn_perm(bg[k], ag[k], 0x07060302u);
        }
      }
    }
  }
  __syncthreads();
  // the four even pairs of staged columns x0 .. x0 + 7 of row ry, channel c
  auto pairs4 = [&](const uint32_t* base, int ry, int x0, uint32_t* o) {
    const uint2* p = reinterpret_cast<const uint2*>(base + ((size_t)ry * kLceCh + c) * PP + x0 / 2);
    const uint2 l = p[0], h = p[1];
    o[0] = l.x; o[1] = l.y; o[2] = h.x; o[3] = h.y;
  };
  float acc[26];
#pragma unroll
  for (int i = 0; i < 26; ++i) acc[i] = 0.f;
  const int runs = (int)a.druns.d;
  const uint32_t ones = 0x3f803f80u;  // bf16 (1, 1)
  for (int item = xg; item < BR * runs; item += XG) {  // (row, run) items over the column groups
    const int ry = (int)fdiv(a.druns, (uint32_t)item), x0 = (item - ry * runs) * kLceRun, y = y0 + ry;
    // dout[y][x0 .. x0+3] as pairs (staged row ry + 2, columns x0 + 2 ..)
    const uint32_t* gcp = gs + ((size_t)(ry + 2) * kLceCh + c) * PP + x0 / 2 + 1;  // 4-byte aligned
    const uint2 gc = make_uint2(gcp[0], gcp[1]);
    acc[25] = dot2(gc.y, ones, dot2(gc.x, ones, acc[25]));
    float dl[kLceRun] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ta = 0; ta < 5; ++ta) {
      uint32_t P[4], Q[4];
      pairs4(vs, ry + ta, x0, P);      // v[y+ta-2][x0-2 .. x0+5]
      pairs4(gs, ry + 4 - ta, x0, Q);  // dout[y+2-ta][x0-2 .. x0+5]
      const uint32_t O0 = __builtin_amdgcn_alignbyte(P[1], P[0], 2), O1 = __builtin_amdgcn_alignbyte(P[2], P[1], 2),
                     O2 = __builtin_amdgcn_alignbyte(P[3], P[2], 2);
      const uint32_t R0 = __builtin_amdgcn_alignbyte(Q[1], Q[0], 2), R1 = __builtin_amdgcn_alignbyte(Q[2], Q[1], 2),
                     R2 = __builtin_amdgcn_alignbyte(Q[3], Q[2], 2);
      // tap (ta, te): dout pairs (x0, x0+1), (x0+2, x0+3) against v pairs
      // starting at x0 + te - 2 and x0 + te
      acc[5 * ta + 0] = dot2(gc.y, P[1], dot2(gc.x, P[0], acc[5 * ta + 0]));
      acc[5 * ta + 1] = dot2(gc.y, O1, dot2(gc.x, O0, acc[5 * ta + 1]));
      acc[5 * ta + 2] = dot2(gc.y, P[2], dot2(gc.x, P[1], acc[5 * ta + 2]));
      acc[5 * ta + 3] = dot2(gc.y, O2, dot2(gc.x, O1, acc[5 * ta + 3]));
      acc[5 * ta + 4] = dot2(gc.y, P[3], dot2(gc.x, P[2], acc[5 * ta + 4]));
      // output x0 + j: dout at x0 + j - 2 .. x0 + j + 2 against taps 4 .. 0
      dl[0] = dot2(Q[2], w0l[ta], dot2(Q[1], w21[ta], dot2(Q[0], w43[ta], dl[0])));
      dl[1] = dot2(Q[2], w0h[ta], dot2(R1, w21[ta], dot2(R0, w43[ta], dl[1])));
      dl[2] = dot2(Q[3], w0l[ta], dot2(Q[2], w21[ta], dot2(Q[1], w43[ta], dl[2])));
      dl[3] = dot2(Q[3], w0h[ta], dot2(R2, w21[ta], dot2(R1, w43[ta], dl[3])));
    }
    if (y < H)
#pragma unroll
      for (int j = 0; j < kLceRun; ++j)
        if (x0 + j < W) a.dv_lce[((((size_t)n * CB + cb) * H + y) * W + x0 + j) * kLceCh + c] = dl[j];
  }
  __syncthreads();  // the staging area becomes the reduction area
  float* red = reinterpret_cast<float*>(sm);  // [XG][kLceCh][26]
#pragma unroll
  for (int i = 0; i < 26; ++i) red[((size_t)xg * kLceCh + c) * 26 + i] = acc[i];
  __syncthreads();
  for (int e = tid; e < kLceCh * 26; e += NT) {
    float sum = 0.f;
    for (int j = 0; j < XG; ++j) sum += red[(size_t)j * kLceCh * 26 + e];
    a.part[((size_t)(n * YB + yb) * C + cb * kLceCh) * 26 + e] = sum;
  }
}

// dw[c][tap] and db[c]: 32 threads per (c, tap) element add the blocks j,
// j + 32, ... in order, then a fixed butterfly adds the 32 partial sums
__global__ __launch_bounds__(256) void lce_grad_sum_kernel(const float* __restrict__ part, int blocks, int C,
                                                           float* __restrict__ dw, float* __restrict__ db) {
  const int e = blockIdx.x * 8 + (threadIdx.x >> 5), j = threadIdx.x & 31;
  const bool live = e < C * 26;
  float acc = 0.f;
  if (live)
    for (int b = j; b < blocks; b += 32) acc += part[(size_t)b * C * 26 + e];
#pragma unroll
  for (int m = 16; m >= 1; m >>= 1) acc += __shfl_xor(acc, m, 32);
  if (!live || j != 0) return;
  const int c = e / 26, tap = e - c * 26;
  if (tap < 25) dw[(size_t)c * 25 + tap] = acc;
  else if (db) db[c] = acc;
}

template <int WAVES, int TK, int TQ, int BPW>
hipError_t launch_sides(const BwdArgs& a, hipStream_t st) {
  const unsigned units = (unsigned)(a.N * a.R * a.heads * (a.T / 16 / (WAVES * BPW)));
  if (a.L % TK == 0)
    launch(bwd_query_kernel<WAVES, TK, BPW, true>, dim3(units), dim3(64 * WAVES), 0, st, a);
  else
    launch(bwd_query_kernel<WAVES, TK, BPW, false>, dim3(units), dim3(64 * WAVES), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.T % TQ == 0)
    launch(bwd_key_kernel<WAVES, TQ, BPW, true>, dim3(units), dim3(64 * WAVES), 0, st, a);
  else
    launch(bwd_key_kernel<WAVES, TQ, BPW, false>, dim3(units), dim3(64 * WAVES), 0, st, a);
  return hipGetLastError();
}

// A region's 16-token blocks two to a wave when there are at least two, the
// waves of one workgroup covering up to 256 tokens; key tiles of 64 keys for
// workgroups of 4 or 8 waves (so the query side stays within 128 registers
// and two workgroups share a CU), else 128 (64, 32 for short gathered
// sequences); query tiles of up to 128 by T.
hipError_t launch_sides_for(const BwdArgs& a, hipStream_t st) {
  const int blocks = a.T / 16;
  const bool big = a.L >= 128;
  if (blocks % 2) {  // odd block counts: one block a wave, one wave a workgroup
    return big ? launch_sides<1, 128, 32, 1>(a, st)
               : a.L >= 64 ? launch_sides<1, 64, 32, 1>(a, st) : launch_sides<1, 32, 32, 1>(a, st);
  }
  const int pairs = blocks / 2;
  int waves = pairs % 8 == 0 ? 8 : pairs % 4 == 0 ? 4 : pairs % 2 == 0 ? 2 : 1;
  if (waves > kBwdMaxWaves) waves = kBwdMaxWaves;
  switch (waves) {
    case 8: return launch_sides<8, 64, 128, 2>(a, st);  // <= 128 VGPRs: two workgroups a CU
    case 4: return launch_sides<4, 64, 128, 2>(a, st);
    case 2: return big ? launch_sides<2, 128, 64, 2>(a, st) : launch_sides<2, 64, 64, 2>(a, st);
    default: return big ? launch_sides<1, 128, 32, 2>(a, st) : launch_sides<1, 64, 32, 2>(a, st);
  }
}

}  // namespace

bool backward_supports(const Shape& s, int dtype) {
  return dtype == 1 && s.hd == 32 && s.T % 16 == 0 && s.topk <= 16 && s.R <= 1024 &&
         lce_grad_lds(s.H, s.W) <= 96 * 1024 && (size_t)s.H * s.W * s.C * 2 < (1ull << 31);
}

size_t backward_workspace_bytes(const Shape& s) {
  const size_t stats = (size_t)s.N * s.H * s.W * s.heads * sizeof(float);
  auto al = [](size_t x) { return (x + 255) & ~(size_t)255; };
  return 2 * al(stats) + al((size_t)s.N * s.R * 4) + al((size_t)s.N * s.R * s.R * 4) +
         al((size_t)s.N * lce_blocks(s.H, s.W) * s.C * 26 * sizeof(float)) +
         al((size_t)s.N * s.H * s.W * s.C * sizeof(float));
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
  int32_t* cnt = reinterpret_cast<int32_t*>(p);
  p += al((size_t)s.N * s.R * 4);
  int32_t* ent = reinterpret_cast<int32_t*>(p);
  p += al((size_t)s.N * s.R * s.R * 4);
  float* part = reinterpret_cast<float*>(p);
  p += al((size_t)s.N * lce_blocks(s.H, s.W) * s.C * 26 * sizeof(float));
  float* dvl = reinterpret_cast<float*>(p);
  a.dv_lce = dvl;
  a.inv_cnt = cnt;
  a.inv_ent = ent;
  a.dq = (uint16_t*)dq;
  a.dk = (uint16_t*)dk;
  a.dv = (uint16_t*)dv;
  a.N = s.N; a.H = s.H; a.W = s.W; a.C = s.C; a.heads = s.heads; a.S = s.S; a.topk = s.topk;
  a.R = s.R; a.rh = s.rh; a.rw = s.rw; a.T = s.T; a.L = s.L;

  launch(inv_route_kernel, dim3((unsigned)(s.N * s.R)), dim3(64), 0, st, route, s.R, s.topk, cnt, ent);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int lblocks = s.N * lce_blocks(s.H, s.W);
  LceArgs la;
  la.v = (const uint16_t*)v;
  la.g = (const uint16_t*)dout;
  la.lw = (const uint16_t*)w;
  la.N = s.N; la.H = s.H; la.W = s.W; la.C = s.C;
  la.rows = lce_rows(s.H, s.W);
  la.dpp = make_fastdiv((uint32_t)(lce_pitch(s.W) / 2));
  la.druns = make_fastdiv((uint32_t)((s.W + kLceRun - 1) / kLceRun));
  la.part = part;
  la.dv_lce = dvl;
  const dim3 lgrid((unsigned)(lblocks * (s.C / kLceCh)));
  if (lce_groups(s.W) == 64)
    launch(lce_grad_rows_kernel<64>, lgrid, dim3(64 * kLceCh), lce_grad_lds(s.H, s.W), st, la);
  else
    launch(lce_grad_rows_kernel<32>, lgrid, dim3(32 * kLceCh), lce_grad_lds(s.H, s.W), st, la);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  launch(lce_grad_sum_kernel, dim3((unsigned)((s.C * 26 + 7) / 8)), dim3(256), 0, st, (const float*)part, lblocks,
         s.C, dw, db);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  e = launch_sides_for(a, st);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace bra
