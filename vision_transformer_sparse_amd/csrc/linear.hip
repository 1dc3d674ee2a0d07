// The projections around the BRA operator: y = x W^T + b, a Linear layer over
// the channels of every token. The walk-through at
// TRANSFORMER.niftyadmin.cn/n/347023.html, section BRA模块, projects the
// tokens to q and kv with one Linear(C, 3C) and splits the result (q first,
// then k, then v; the module print in section 网络结构 shows QKVLinear's
// Linear(64, 192)), and ends the block with the output Linear(C, C) (wo).
//
// y's features are written in consecutive blocks of `split` features to up
// to three outputs (y0: features [0, split), y1: [split, 2 split), y2:
// [2 split, 3 split)), each a row-major [M][split] matrix, so the q, k and v
// of the qkv projection come out as three NHWC tensors. The host checks
// K % 32 == 0, split % 8 == 0, Nout = split * (1, 2 or 3), that both
// operands stay under 2 GiB, and 16-byte aligned outputs.
//
// bf16: the matrix cores. A wave computes 64 tokens x 64 features as 4 x 4
// tiles of v_mfma_f32_16x16x32_bf16 with D = W_tile . X_tile^T: the A operand
// is 16 bytes of a weight row (from LDS, where the workgroup puts its 64
// weight rows once for its four waves) and the B operand 16 bytes of a token
// row (straight from memory, channels contiguous); a lane's D column is four
// consecutive features of one token. The wave stages its tile in LDS and
// stores it back as 16-byte pieces of the tile's 128-byte rows (64 features
// of a token), so the stores fill whole cache lines (when split is a multiple
// of 64 and the outputs 128-byte aligned, as torch allocates them). The next k step's
// operands load while the current step's products run. A workgroup of
// four waves takes 256 tokens x 64 features; the feature blocks of one token
// block are consecutive units on one XCD, so its L2 serves the token rows to
// all of them and they come from HBM once. K is at most 256.
// fp32: a lane computes four features of one token with fma chains.
//
// The qkv projection fused with the region pooling (POOL): the same tiles
// over the tokens taken region by region (a region's T tokens row-major, the
// regions of an image in order, T a multiple of 64, so a wave's 64 tokens
// lie in one region). Each wave sums its staged bf16 q or k tile over its
// tokens (one lane a feature, tokens in order), and for k it also takes the
// largest squared norm of each 32-channel head slice over its tokens (one
// lane a token); the waves of a region are combined in order and written as
// the region means Q^r, K^r (fp32, [N][S*S][C]) and max |k|^2 per (image,
// region, head) ([N][S*S][C/32]) -- what the pooling kernel gives the
// router and the large-region attention kernel, here without reading q and
// k back from memory. Means are taken over the values as stored (bf16).
#include "bra_internal.h"

namespace bra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float sq2(uint32_t v, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v), __builtin_bit_cast(bf16x2, v), acc, false);
}

constexpr int kLinTok = 256;  // tokens per workgroup (64 per wave)
constexpr int kLinFeat = 64;  // features per workgroup

struct LinArgs {
  const uint16_t* x;
  const uint16_t* w;
  const uint16_t* b;  // or null
  uint16_t* y[3];
  int M, K, Nout, split;
  // POOL only: the image layout and the pooled outputs (region sides are
  // powers of two: rw = 1 << lrw)
  int H, W, S, rh, rw, lrw;
  float* qr;  // [N][S*S][split] region means of y[0]
  float* kr;  // [N][S*S][split] region means of y[1]
  float* kn;  // [N][S*S][split/32] max |k|^2 of each head slice of y[1]
  const uint16_t* lw;  // the LCE weights [split][25], repacked (as the pooling
  uint32_t* wpk;       // kernel does) into wpk for the attention kernels
};

// Where the wave's 64 tokens sit: without POOL, rows t0 .. t0 + 63 of x / y.
// With POOL, tokens t0 .. t0 + 63 of the region-major order (region t / T of
// image t / (S*S*T), token t % T row-major inside the region) lie in one
// region (T % 64 == 0): its first pixel and the wave's first token inside it
// are found once, and token t0 + l is pixel base + (tt >> lrw) * W +
// (tt & (rw - 1)) with tt = tt0 + l.
struct TokenMap {
  int base, tt0;
};
template <bool POOL>
__device__ __forceinline__ TokenMap token_map(const LinArgs& a, int t0) {
  if constexpr (!POOL) {
    return {t0, 0};
  } else {
    const int T = a.rh * a.rw, R = a.S * a.S;
    const int nr = t0 / T, tt0 = t0 - nr * T;
    const int n = nr / R, r = nr - n * R;
    const int jr = r / a.S, ir = r - jr * a.S;
    return {(n * a.H + jr * a.rh) * a.W + ir * a.rw, tt0};
  }
}
template <bool POOL>
__device__ __forceinline__ int token_row(const LinArgs& a, const TokenMap& m, int l) {
  if constexpr (!POOL) {
    return m.base + l;
  } else {
    const int tt = m.tt0 + l;
    return m.base + (tt >> a.lrw) * a.W + (tt & (a.rw - 1));
  }
}

template <bool POOL>
__global__ __launch_bounds__(256) void linear_bf16_kernel(LinArgs a) {
  // LDS: first the workgroup's 64 weight rows (row pitch 2K + 16 bytes, so a
  // tile column's 16 rows fall in distinct bank groups), shared by its four
  // waves; after the products, each wave's 64 x 64 output tile, staged for
  // row-contiguous stores (row pitch 72 elements = 144 bytes: rows stay
  // 16-byte aligned and a tile column's 16 tokens spread over the banks).
  // K <= 256 keeps the weight rows inside the same 36 KiB.
  constexpr int kPitch = 72;
  __shared__ __align__(16) uint8_t lds[4 * 64 * kPitch * 2];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int nfb = (a.Nout + kLinFeat - 1) / kLinFeat;
  const int u = xcd_unit((int)blockIdx.x, (int)gridDim.x);
  const int tb = u / nfb, fb = u - tb * nfb;
  const int t0 = tb * kLinTok + wave * 64, f0 = fb * kLinFeat;
  const uint32_t xbytes = (uint32_t)a.M * a.K * 2, wbytes = (uint32_t)a.Nout * a.K * 2;
  const Rsrc xr = rsrc(a.x, xbytes), wr = rsrc(a.w, wbytes);
  const int wpitch = 2 * a.K + 16;
  const TokenMap tmap = token_map<POOL>(a, t0);
  if constexpr (POOL) {  // the LCE weight repacking, a grid-stride side job
    for (int e = (int)blockIdx.x * 256 + tid; e < lce_pack_items(a.split); e += (int)gridDim.x * 256)
      pack_lce_item(a.lw, a.split, e, a.wpk);
  }
  // operand rows of this lane: tokens t0 + 16 i + col (HBM), features
  // f0 + 16 j + col (LDS)
  uint32_t xo[4], wl[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int t = t0 + 16 * i + col;
    // rows past the end read zeros: kOut plus an in-range k offset (< 2^31)
    // stays past the buffer
    xo[i] = t < a.M ? (uint32_t)token_row<POOL>(a, tmap, 16 * i + col) * a.K * 2 + (uint32_t)grp * 16 : kOut;
    wl[i] = (uint32_t)((16 * i + col) * wpitch + grp * 16);
  }
  // two operand sets: one k step's products run while the next step's
  // operands load. A load at or past K reads zero token rows (their offsets
  // moved past the buffer) and is never multiplied: when K % 64 == 32 the
  // loop's second half-step is skipped (a wave-uniform branch), so weights
  // are only ever multiplied by real token values.
  bf16x8 xa[4], wa[4], xb[4], wb[4];
  auto load_x = [&](bf16x8* xs, int k) {
    const uint32_t kb = k < a.K ? (uint32_t)k * 2 : kOut;
#pragma unroll
    for (int i = 0; i < 4; ++i) xs[i] = __builtin_bit_cast(bf16x8, ld16(xr, xo[i] + kb));
  };
  auto load_w = [&](bf16x8* ws, int k) {
    const uint32_t kw = k < a.K ? (uint32_t)k * 2 : 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      ws[i] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(lds + wl[i] + kw));
  };
  // the first two k steps' token rows are requested before the weights, so
  // the two latencies overlap
  load_x(xa, 0);
  load_x(xb, 32);
  {
    // the weight rows f0 .. f0 + 63 in 16-byte chunks (at most 8 a thread for
    // K <= 256), all loads issued before the first LDS write; rows past Nout
    // and chunks past the tile read zeros
    const int cpr = a.K / 8, chunks = 64 * cpr;
    uint4 v[8];
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int c = tid + 256 * n, r = c / cpr, q = c - r * cpr, f = f0 + r;
      v[n] = ld16(wr, c < chunks && f < a.Nout ? (uint32_t)f * a.K * 2 + (uint32_t)q * 16 : kOut);
    }
#pragma unroll
    for (int n = 0; n < 8; ++n) {
      const int c = tid + 256 * n, r = c / cpr, q = c - r * cpr;
      if (c < chunks) *reinterpret_cast<uint4*>(lds + r * wpitch + q * 16) = v[n];
    }
  }
  // this lane's bias words (features f0 + 16 j + 4 grp .. + 3), loaded before
  // the products so their latency hides behind them; Nout % 8 == 0, so the
  // four features are all in range or all out
  uint32_t bw[4][2];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int f = f0 + 16 * j + 4 * grp;
    const bool has = a.b && f < a.Nout;
    const uint32_t* bp = reinterpret_cast<const uint32_t*>(a.b + (has ? f : 0));
    bw[j][0] = has ? bp[0] : 0u;
    bw[j][1] = has ? bp[1] : 0u;
  }
  f32x4 acc[4][4];  // [feature tile j][token tile i]
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[j][i] = f32x4{0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  auto mma = [&](const bf16x8* xs, const bf16x8* ws) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[j][i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ws[j], xs[i], acc[j][i], 0, 0, 0);
  };
  // (the scheduling barriers keep each load batch ahead of the products
  // that overlap it)
  load_w(wa, 0);
  load_w(wb, 32);
  for (int k0 = 0; k0 < a.K; k0 += 64) {
    __builtin_amdgcn_sched_barrier(0);
    mma(xa, wa);
    __builtin_amdgcn_sched_barrier(0);
    if (k0 + 64 < a.K) {
      load_x(xa, k0 + 64);
      load_w(wa, k0 + 64);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (k0 + 32 < a.K) mma(xb, wb);
    __builtin_amdgcn_sched_barrier(0);
    if (k0 + 96 < a.K) {
      load_x(xb, k0 + 96);
      load_w(wb, k0 + 96);
    }
  }
  __syncthreads();  // every wave is done with the weight rows
  // lane (col, grp) of tile (j, i) holds features 16 j + 4 grp .. + 3 (of
  // the block) of token 16 i + col: bias, round, and stage 8 bytes
  uint16_t* tw = reinterpret_cast<uint16_t*>(lds) + wave * 64 * kPitch;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int fl = 16 * j + 4 * grp;
    const float bias[4] = {bf16_lo(bw[j][0]), bf16_hi(bw[j][0]), bf16_lo(bw[j][1]), bf16_hi(bw[j][1])};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t v[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] = float_to_bf16_bits(acc[j][i][e] + bias[e]);
      *reinterpret_cast<uint2*>(tw + (16 * i + col) * kPitch + fl) =
          make_uint2(v[0] | (v[1] << 16), v[2] | (v[3] << 16));
    }
  }
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // 16-byte chunks: lane -> row 8 p + lane / 8, features 8 (lane % 8) .. + 7;
  // split % 8 == 0 keeps a chunk inside one output
  const int c8 = (lane & 7) * 8, f = f0 + c8;
  if (f < a.Nout) {
    const int part = f / a.split, fo = f - part * a.split;
    uint16_t* ybase = a.y[part] + fo;
#pragma unroll
    for (int p = 0; p < 8; ++p) {
      const int r = 8 * p + (lane >> 3), t = t0 + r;
      const uint4 v = *reinterpret_cast<const uint4*>(tw + r * kPitch + c8);
      if (t < a.M) *reinterpret_cast<uint4*>(ybase + (size_t)token_row<POOL>(a, tmap, r) * a.split) = v;
    }
  }
  if constexpr (POOL) {
    // the host checks split % 64 == 0: the 64 features are one part's
    // features fo0 .. fo0 + 63, two whole heads
    __shared__ float red_sum[4][64];
    __shared__ float red_kn[4][2];
    const int part = f0 / a.split, fo0 = f0 - part * a.split;
    const bool live = part < 2 && t0 < a.M;  // a wave's tokens are all in range or all out
    if (live) {
      // the sums over the wave's 64 tokens: lane l adds features
      // 8 (l % 8) .. + 7 of tokens l / 8, l / 8 + 8, ..., then the eight
      // token groups are added by lane swaps (a fixed order)
      float sum[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) sum[e] = 0.f;
#pragma unroll
      for (int m = 0; m < 8; ++m) {
        const uint4 w4 = *reinterpret_cast<const uint4*>(tw + (8 * m + (lane >> 3)) * kPitch + 8 * (lane & 7));
        const uint32_t wv[4] = {w4.x, w4.y, w4.z, w4.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sum[2 * e] += bf16_lo(wv[e]);
          sum[2 * e + 1] += bf16_hi(wv[e]);
        }
      }
#pragma unroll
      for (int d = 8; d <= 32; d <<= 1)
#pragma unroll
        for (int e = 0; e < 8; ++e) sum[e] += __shfl_xor(sum[e], d);
      if (lane < 8) {
#pragma unroll
        for (int e = 0; e < 8; ++e) red_sum[wave][8 * lane + e] = sum[e];
      }
      if (part == 1) {
        // lane = token: the squared norms of the two head slices
        const uint16_t* row = tw + lane * kPitch;
        float n2[2];
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          float acc = 0.f;
#pragma unroll
          for (int c = 0; c < 4; ++c) {
            const uint4 w4 = *reinterpret_cast<const uint4*>(row + 32 * hh + 8 * c);
            acc = sq2(w4.w, sq2(w4.z, sq2(w4.y, sq2(w4.x, acc))));
          }
#pragma unroll
          for (int d = 32; d >= 1; d >>= 1) acc = fmaxf(acc, __shfl_xor(acc, d));
          n2[hh] = acc;
        }
        if (lane == 0) {
          red_kn[wave][0] = n2[0];
          red_kn[wave][1] = n2[1];
        }
      }
    }
    __syncthreads();
    // the first wave of each region adds its region's waves in order
    const int T = a.rh * a.rw, wpr = T >= 256 ? 4 : T / 64;
    if (live && wave % wpr == 0) {
      float sum = 0.f;
      for (int w2 = wave; w2 < wave + wpr; ++w2) sum += red_sum[w2][lane];
      const int nr = t0 / T;  // image * S*S + region
      float* means = part == 0 ? a.qr : a.kr;
      means[(size_t)nr * a.split + fo0 + lane] = sum / (float)T;
      if (part == 1 && lane < 2) {
        float m = 0.f;
        for (int w2 = wave; w2 < wave + wpr; ++w2) m = fmaxf(m, red_kn[w2][lane]);
        a.kn[(size_t)nr * (a.split / 32) + fo0 / 32 + lane] = m;
      }
    }
  }
}

struct LinArgsF {
  const float* x;
  const float* w;
  const float* b;
  float* y[3];
  int M, K, Nout, split;
};

// fp32: a thread computes features f .. f+3 of one token
__global__ __launch_bounds__(256) void linear_f32_kernel(LinArgsF a) {
  const int nq = a.Nout / 4;
  const long long g = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (g >= (long long)a.M * nq) return;
  const int t = (int)(g / nq), f = (int)(g - (long long)t * nq) * 4;
  const float* xr = a.x + (size_t)t * a.K;
  float acc[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) acc[e] = 0.f;
  for (int k = 0; k < a.K; ++k) {
    const float xv = xr[k];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = fmaf(xv, a.w[(size_t)(f + e) * a.K + k], acc[e]);
  }
  const int part = f / a.split;
  float* yrow = a.y[part] + (size_t)t * a.split + (f - part * a.split);
#pragma unroll
  for (int e = 0; e < 4; ++e) yrow[e] = acc[e] + (a.b ? a.b[f + e] : 0.f);
}

}  // namespace

hipError_t launch_linear(const void* x, const void* w, const void* b, int M, int K, int Nout,
                         int split, int dtype, void* y0, void* y1, void* y2, hipStream_t st) {
  if (dtype == 1) {
    LinArgs a;
    a.x = (const uint16_t*)x; a.w = (const uint16_t*)w; a.b = (const uint16_t*)b;
    a.y[0] = (uint16_t*)y0; a.y[1] = (uint16_t*)y1; a.y[2] = (uint16_t*)y2;
    a.M = M; a.K = K; a.Nout = Nout; a.split = split;
    const unsigned blocks = (unsigned)((M + kLinTok - 1) / kLinTok) * (unsigned)((Nout + kLinFeat - 1) / kLinFeat);
    launch(linear_bf16_kernel<false>, dim3(blocks), dim3(256), 0, st, a);
  } else {
    LinArgsF a;
    a.x = (const float*)x; a.w = (const float*)w; a.b = (const float*)b;
    a.y[0] = (float*)y0; a.y[1] = (float*)y1; a.y[2] = (float*)y2;
    a.M = M; a.K = K; a.Nout = Nout; a.split = split;
    const long long n = (long long)M * (Nout / 4);
    launch(linear_f32_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a);
  }
  return hipGetLastError();
}

bool qkv_pool_supports(const Shape& s) {
  const int T = s.rh * s.rw;
  return s.C % 64 == 0 && s.C <= 256 && T % 64 == 0 && T <= 256 && 256 % T == 0 &&
         (s.rw & (s.rw - 1)) == 0 &&
         (long long)s.N * s.H * s.W * s.C * 2 < (1ll << 31) &&
         (long long)3 * s.C * s.C * 2 < (1ll << 31);
}

hipError_t launch_qkv_pool(const void* x, const void* w, const void* b, const void* lw, const Shape& s,
                           void* q, void* k, void* v, float* qr, float* kr, float* kn, uint32_t* wpk,
                           hipStream_t st) {
  LinArgs a;
  a.x = (const uint16_t*)x; a.w = (const uint16_t*)w; a.b = (const uint16_t*)b;
  a.y[0] = (uint16_t*)q; a.y[1] = (uint16_t*)k; a.y[2] = (uint16_t*)v;
  a.M = s.N * s.H * s.W; a.K = s.C; a.Nout = 3 * s.C; a.split = s.C;
  a.H = s.H; a.W = s.W; a.S = s.S; a.rh = s.rh; a.rw = s.rw;
  a.lrw = 0;
  while ((1 << a.lrw) < s.rw) ++a.lrw;
  a.qr = qr; a.kr = kr; a.kn = kn; a.lw = (const uint16_t*)lw; a.wpk = wpk;
  const unsigned blocks = (unsigned)((a.M + kLinTok - 1) / kLinTok) * (unsigned)(a.Nout / kLinFeat);
  launch(linear_bf16_kernel<true>, dim3(blocks), dim3(256), 0, st, a);
  return hipGetLastError();
}

}  // namespace bra
