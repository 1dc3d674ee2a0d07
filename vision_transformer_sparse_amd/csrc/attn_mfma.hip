// Token-to-token attention over the routed regions plus LCE for bf16 tensors,
// on gfx950 matrix cores (v_mfma_f32_16x16x32_bf16). Eq. 6-7 of the BRA
// walk-through at TRANSFORMER.niftyadmin.cn/n/347023.html, section BRA模块:
// the keys/values of a query region are the tokens of its topk routed
// regions; per head (channels [h*32, h*32+32)) a softmax over all topk*T of
// them jointly; out = attention + LCE(V) (5x5 depthwise conv, zero padding
// 2, bias; the module print's Conv2d(C, C, 5, padding=2, groups=C)).
//
// Tiling. A wave owns 16 queries of one (image, region, head) unit and walks
// the unit's gathered keys in chunks of 64 (four 16-key tiles), fetching each
// key row by route index straight from NHWC memory -- the routed K/V copy is
// never materialised. With hd = 32 one 16x16x32 MFMA covers a whole head:
//
//   S^T(16 keys x 16 queries) = K_tile (A: lane = key row, 8 dims)
//                             x Q^T   (B: lane = query col, 8 dims)
//
// so a lane (query q = lane%16, group g = lane/16) receives the scores of
// keys 4g..4g+3 of every tile for ITS query: the softmax max/sum need only
// the lane's own values plus two cross-lane steps (xor 16, xor 32).
//
// P V needs V with keys along the contraction, i.e. transposed. The
// transpose is done on the matrix cores: V_tile (A, lane = key row) times a
// 0/1 selector (B) returns V^T in the accumulator layout -- lane (dim j,
// group g) holds keys 4g..4g+3 of the tile -- which is exactly the key order
// the score accumulator gives P^T. So
//
//   O^T(16 dims x 16 queries) += V^T (A: keys of tiles 2b, 2b+1)
//                              x P^T (B: same keys, same order)
//
// with no LDS traffic and no shuffles. The softmax is online across chunks,
// in base 2 with head_dim^-1/2 * log2(e) folded into one fma, in fp32; P is
// rounded to bf16 for the product.
#include "bra_internal.h"

namespace bra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kChunk = 64;  // keys per online-softmax step (4 tiles of 16)

__device__ __forceinline__ bf16x8 load8(const uint16_t* p) {
  uint4 w = *reinterpret_cast<const uint4*>(p);
  return __builtin_bit_cast(bf16x8, w);
}

__device__ __forceinline__ bf16x4 to_bf16x4(f32x4 x) {
  bf16x4 r;
  r[0] = (__bf16)x[0]; r[1] = (__bf16)x[1]; r[2] = (__bf16)x[2]; r[3] = (__bf16)x[3];
  return r;
}

__device__ __forceinline__ bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

struct Geo {
  int H, W, C, S, rh, rw, T, L, topk;
};

// NHWC element offset of token tt of region s (image n, channel c).
__device__ __forceinline__ size_t tok_off(const Geo& g, int n, int s, int tt, int c) {
  const int js = s / g.S, is = s - js * g.S;
  const int y = js * g.rh + tt / g.rw, x = is * g.rw + tt % g.rw;
  return (((size_t)n * g.H + y) * g.W + x) * g.C + c;
}

// SMALL: one wave per (image, region, head) unit, T <= 16 (one query block).
// !SMALL: one workgroup per unit, the waves share out its 16-query blocks.
template <bool SMALL>
__global__ __launch_bounds__(256) void attn_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ w,
    const uint16_t* __restrict__ b, const int32_t* __restrict__ route, Geo g,
    int heads, long long units, float qscale, uint16_t* __restrict__ out) {
  __shared__ float wl[kWaves][25][32];  // LCE weights of the wave's head, tap-major
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int col = lane & 15, grp = lane >> 4;
  const long long unit = SMALL ? (long long)blockIdx.x * kWaves + wave : (long long)blockIdx.x;
  const bool live = unit < units;
  const long long uu = live ? unit : 0;
  const int h = (int)(uu % heads);
  const long long nr = uu / heads;
  const int R = g.S * g.S;
  const int r = (int)(nr % R);
  const int n = (int)(nr / R);
  const int c0 = h * 32;
  const int32_t* rt = route + nr * g.topk;

  // LCE weights of this head into LDS as fp32 [tap][channel].
  {
    float* dst = &wl[SMALL ? wave : 0][0][0];
    const int first = SMALL ? lane : threadIdx.x, step = SMALL ? 64 : 256;
    for (int e = first; e < 25 * 32; e += step) {
      const int d = e / 25, tap = e - d * 25;
      dst[tap * 32 + d] = bf16_bits_to_float(w[(size_t)(c0 + d) * 25 + tap]);
    }
  }
  __syncthreads();
  if (!live) return;
  const float* wt = &wl[SMALL ? wave : 0][0][0];

  // 0/1 selectors that turn a V tile into V^T (dims 0-15 and 16-31).
  bf16x8 sel[2];
#pragma unroll
  for (int half = 0; half < 2; ++half)
#pragma unroll
    for (int e = 0; e < 8; ++e)
      sel[half][e] = (__bf16)((grp == 2 * half + (col >> 3) && e == (col & 7)) ? 1.0f : 0.0f);

  const int nqb = SMALL ? 1 : (g.T + 15) / 16;
  for (int qb = SMALL ? 0 : wave; qb < nqb; qb += SMALL ? 1 : kWaves) {
    const int qt = qb * 16 + col;             // this lane's query token
    const bool qvalid = qt < g.T;
    const int qtc = qvalid ? qt : g.T - 1;    // clamp: duplicate columns are not stored
    const bf16x8 bq = load8(q + tok_off(g, n, r, qtc, c0 + 8 * grp));

    float m = -INFINITY, l = 0.f;
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = {0.f, 0.f, 0.f, 0.f};
    for (int base = 0; base < g.L; base += kChunk) {
      f32x4 s[4];
      bf16x4 vt[4][2];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int u = base + 16 * t + col;   // key row this lane loads for tile t
        const int uc = u < g.L ? u : g.L - 1;
        const int p = uc / g.T, tt = uc - p * g.T;
        const size_t off = tok_off(g, n, rt[p], tt, c0 + 8 * grp);
        const bf16x8 ak = load8(k + off);
        const bf16x8 av = load8(v + off);
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        s[t] = mfma(ak, bq, z);
        vt[t][0] = to_bf16x4(mfma(av, sel[0], z));
        vt[t][1] = to_bf16x4(mfma(av, sel[1], z));
      }
      // scores -> log2 domain, mask keys past L
      float cm = -INFINITY;
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int key = base + 16 * t + 4 * grp + e;
          float x = s[t][e] * qscale;
          x = key < g.L ? x : -INFINITY;
          s[t][e] = x;
          cm = fmaxf(cm, x);
        }
      cm = fmaxf(cm, __shfl_xor(cm, 16, 64));
      cm = fmaxf(cm, __shfl_xor(cm, 32, 64));
      const float mn = fmaxf(m, cm);
      const float corr = __builtin_amdgcn_exp2f(m - mn);
      m = mn;
      l *= corr;
      o0 *= corr;
      o1 *= corr;
      bf16x4 pb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(s[t][e] - mn);
          l += pv[e];
        }
        pb[t] = to_bf16x4(pv);
      }
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        const bf16x8 pt = cat(pb[2 * bb], pb[2 * bb + 1]);
        o0 = mfma(cat(vt[2 * bb][0], vt[2 * bb + 1][0]), pt, o0);
        o1 = mfma(cat(vt[2 * bb][1], vt[2 * bb + 1][1]), pt, o1);
      }
    }
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.0f / l;
    if (!qvalid) continue;

    // LCE for this lane's query and channels c0+4g..+3, c0+16+4g..+3.
    const int jr = r / g.S, ir = r - jr * g.S;
    const int y = jr * g.rh + qt / g.rw, x = ir * g.rw + qt % g.rw;
    float acc[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      acc[e] = b ? bf16_bits_to_float(b[c0 + 4 * grp + e]) : 0.f;
      acc[4 + e] = b ? bf16_bits_to_float(b[c0 + 16 + 4 * grp + e]) : 0.f;
    }
    for (int a = 0; a < 5; ++a) {
      const int yy = y + a - 2;
      if (yy < 0 || yy >= g.H) continue;
      for (int e2 = 0; e2 < 5; ++e2) {
        const int xx = x + e2 - 2;
        if (xx < 0 || xx >= g.W) continue;
        const uint16_t* pv = v + (((size_t)n * g.H + yy) * g.W + xx) * g.C + c0;
        const uint2 lo = *reinterpret_cast<const uint2*>(pv + 4 * grp);
        const uint2 hi = *reinterpret_cast<const uint2*>(pv + 16 + 4 * grp);
        const float* wr = wt + (a * 5 + e2) * 32;
        acc[0] = fmaf(wr[4 * grp + 0], bf16_lo(lo.x), acc[0]);
        acc[1] = fmaf(wr[4 * grp + 1], bf16_hi(lo.x), acc[1]);
        acc[2] = fmaf(wr[4 * grp + 2], bf16_lo(lo.y), acc[2]);
        acc[3] = fmaf(wr[4 * grp + 3], bf16_hi(lo.y), acc[3]);
        acc[4] = fmaf(wr[16 + 4 * grp + 0], bf16_lo(hi.x), acc[4]);
        acc[5] = fmaf(wr[16 + 4 * grp + 1], bf16_hi(hi.x), acc[5]);
        acc[6] = fmaf(wr[16 + 4 * grp + 2], bf16_lo(hi.y), acc[6]);
        acc[7] = fmaf(wr[16 + 4 * grp + 3], bf16_hi(hi.y), acc[7]);
      }
    }
    uint16_t* po = out + (((size_t)n * g.H + y) * g.W + x) * g.C + c0;
    uint2 wlo, whi;
    wlo.x = pack_bf16x2(fmaf(o0[0], inv, acc[0]), fmaf(o0[1], inv, acc[1]));
    wlo.y = pack_bf16x2(fmaf(o0[2], inv, acc[2]), fmaf(o0[3], inv, acc[3]));
    whi.x = pack_bf16x2(fmaf(o1[0], inv, acc[4]), fmaf(o1[1], inv, acc[5]));
    whi.y = pack_bf16x2(fmaf(o1[2], inv, acc[6]), fmaf(o1[3], inv, acc[7]));
    *reinterpret_cast<uint2*>(po + 4 * grp) = wlo;
    *reinterpret_cast<uint2*>(po + 16 + 4 * grp) = whi;
  }
}

}  // namespace

bool mfma_supports(const Shape& s) { return s.hd == 32; }

hipError_t launch_attend_mfma(const void* q, const void* k, const void* v,
                              const void* w, const void* b, const int32_t* route,
                              const Shape& s, void* out, hipStream_t st) {
  Geo g{s.H, s.W, s.C, s.S, s.rh, s.rw, s.T, s.L, s.topk};
  const long long units = (long long)s.N * s.R * s.heads;
  const float qscale = (float)(1.4426950408889634 / __builtin_sqrt((double)s.hd));
  if (s.T <= 16) {
    const unsigned blocks = (unsigned)((units + kWaves - 1) / kWaves);
    launch(attn_mfma_kernel<true>, dim3(blocks), dim3(256), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                       (const uint16_t*)w, (const uint16_t*)b, route, g, s.heads, units,
                       qscale, (uint16_t*)out);
  } else {
    launch(attn_mfma_kernel<false>, dim3((unsigned)units), dim3(256), 0, st,
                       (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                       (const uint16_t*)w, (const uint16_t*)b, route, g, s.heads, units,
                       qscale, (uint16_t*)out);
  }
  return hipGetLastError();
}

}  // namespace bra
