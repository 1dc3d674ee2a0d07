// Gathered attention + LCE for fp32 tensors on the fp32 matrix cores
// (v_mfma_f32_16x16x4_f32: fp32 operands, fp32 accumulation) -- the first
// classification stage of BiFormer in fp32 (8x8 regions of a 56x56 map,
// topk 1). Eqs. 6-7 of the BRA walk-through at
// TRANSFORMER.niftyadmin.cn/n/347023.html, section BRA模块: per head, a
// softmax over the tokens of the routed regions jointly, plus LCE(V).
//
// One workgroup per (image, query region, head), one wave per 16 queries
// (T / 16 waves). Per 64-key chunk:
//   S^T (16 keys x 16 queries) = K_tile Q^T, eight k-steps of 4: at step s a
//     lane (row i, group g) gives dim 8g + s of its key row / query column,
//     so its operands are two contiguous float4 per row;
//   softmax in base 2 (log2(e) / sqrt(32) folded into Q), a query's scores
//     in one lane column: its max and sum need only the two group swaps;
//   O^T (16 dims x 16 queries) += V^T P^T, k-step e of tile t = keys
//     16t + 4g + e: the P operand is the lane's own score register, V^T
//     comes from the chunk's V staged in LDS.
// The LCE of the lane's 8 output channels runs from the V halo of the region
// in LDS ((RH+4) x (RW+4) pixels x the head's 32 channels, zero outside the
// image) with the head's weights staged tap-major.
#include "bra_internal.h"
#include "route_common.h"

namespace bra {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  const float* w;       // LCE weights [C][25]
  const float* b;       // LCE bias [C] or null
  const int32_t* route; // [N][S*S][topk]
  float* out;
  int N, H, W, C, heads, S, topk, rh, rw;
  float qscale;         // head_dim^-1/2 * log2(e)
  // routes chosen in the kernel (f32_kernel_routes): the region means
  // [N][S*S][C], where the first head's workgroups report the routes, C^-1/2
  const float* qr;
  const float* kr;
  int32_t* route_out;
  float rscale;
};

constexpr int kHaloStride = 36;  // floats per halo pixel: 32 channels + 4 (banks)
constexpr int kVStride = 33;     // floats per staged V row: 32 dims + 1 (banks)

__host__ __device__ constexpr size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }
struct F32Lds {
  size_t halo, vs, wt, rt, total;
};
// (the in-kernel routing borrows the V staging area for its logits and keys
// before the key loop; the chosen routes keep rt, up to 64 of them)
__host__ __device__ inline F32Lds f32_lds(int rh, int rw) {
  F32Lds l;
  size_t o = 0;
  l.halo = o; o += align16((size_t)(rh + 4) * (rw + 4) * kHaloStride * 4);
  l.vs = o; o += align16((size_t)64 * kVStride * 4);
  l.wt = o; o += (size_t)25 * 32 * 4;
  l.rt = o; o += (size_t)64 * 4;
  l.total = o;
  return l;
}

__global__ __launch_bounds__(1024) void attn_f32_kernel(F32Args a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int H = a.H, W = a.W, C = a.C, S = a.S, R = S * S, topk = a.topk;
  const int rh = a.rh, rw = a.rw, T = rh * rw, L = topk * T;
  const int HP = rh + 4, WP = rw + 4;
  const F32Lds lay = f32_lds(rh, rw);
  float* halo = reinterpret_cast<float*>(smem + lay.halo);  // [HP * WP][36]
  float* vs = reinterpret_cast<float*>(smem + lay.vs);      // [64][33]
  float* wt = reinterpret_cast<float*>(smem + lay.wt);      // [25][32]

  const int tid = threadIdx.x, nthreads = blockDim.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  int u = blockIdx.x;
  const int h = u % a.heads;
  u /= a.heads;
  const int r = u % R, n = u / R;
  const int jr = r / S, ir = r - jr * S;
  const int y0 = jr * rh, x0 = ir * rw;
  const int c0 = h * 32;
  const float* qi = a.q + (size_t)n * H * W * C;
  const float* ki = a.k + (size_t)n * H * W * C;
  const float* vi = a.v + (size_t)n * H * W * C;
  const int32_t* rt = a.route + ((size_t)n * R + r) * topk;
  if (a.qr) {
    // routes chosen here from the region means (the route kernel's logits
    // and ranking, route_common.h), kept in LDS for the key loop
    int32_t* sel = reinterpret_cast<int32_t*>(smem + lay.rt);
    route::route_region(a.qr + (size_t)n * R * C, a.kr + (size_t)n * R * C, R, C, 0, C, a.rscale, r, topk,
                        wave, lane, vs, reinterpret_cast<uint64_t*>(smem + lay.vs + 256), sel, h == 0,
                        a.route_out + ((size_t)n * R + r) * topk);
    rt = sel;
  }

  // ---- stage the V halo and the head's LCE weights
  for (int e = tid; e < HP * WP * 8; e += nthreads) {
    const int pix = e >> 3, pc = e & 7;
    const int y = y0 - 2 + pix / WP, x = x0 - 2 + pix % WP;
    float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
    if (y >= 0 && y < H && x >= 0 && x < W)
      val = *reinterpret_cast<const float4*>(vi + ((size_t)y * W + x) * C + c0 + 4 * pc);
    *reinterpret_cast<float4*>(halo + pix * kHaloStride + 4 * pc) = val;
  }
  for (int e = tid; e < 25 * 32; e += nthreads) {
    const int tap = e >> 5, d = e & 31;
    wt[e] = a.w[(size_t)(c0 + d) * 25 + tap];
  }

  // ---- this wave's queries: tokens 16 * wave + col of the region
  const int qt = 16 * wave + col;
  const int qy = y0 + qt / rw, qx = x0 + qt % rw;
  float qv[8];
  {
    const float* qp = qi + ((size_t)qy * W + qx) * C + c0 + 8 * grp;
    const float4 q0 = *reinterpret_cast<const float4*>(qp);
    const float4 q1 = *reinterpret_cast<const float4*>(qp + 4);
    qv[0] = q0.x * a.qscale; qv[1] = q0.y * a.qscale; qv[2] = q0.z * a.qscale; qv[3] = q0.w * a.qscale;
    qv[4] = q1.x * a.qscale; qv[5] = q1.y * a.qscale; qv[6] = q1.z * a.qscale; qv[7] = q1.w * a.qscale;
  }
  // pixel of key kk (token kk % T of routed region kk / T)
  auto key_pix = [&](int kk) {
    const int s = rt[kk / T], tt = kk % T;
    const int js = s / S, is = s - js * S;
    return (size_t)(js * rh + tt / rw) * W + (size_t)(is * rw + tt % rw);
  };

  float m = -INFINITY, lsum = 0.f;
  f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0;
  for (int base = 0; base < L; base += 64) {
    __syncthreads();  // the previous chunk's V is consumed (first pass: halo staged)
    for (int e = tid; e < 64 * 8; e += nthreads) {  // this chunk's V -> LDS
      const int key = e >> 3, pc = e & 7;
      float4 val = make_float4(0.f, 0.f, 0.f, 0.f);
      if (base + key < L) val = *reinterpret_cast<const float4*>(vi + key_pix(base + key) * C + c0 + 4 * pc);
      float* dst = vs + key * kVStride + 4 * pc;
      dst[0] = val.x; dst[1] = val.y; dst[2] = val.z; dst[3] = val.w;
    }
    // the K rows of this lane: key base + 16t + col, dims 8grp..8grp+7
    float kv[4][8];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int kk = base + 16 * t + col;
      float4 k0 = make_float4(0.f, 0.f, 0.f, 0.f), k1 = k0;
      if (kk < L) {
        const float* kp = ki + key_pix(kk) * C + c0 + 8 * grp;
        k0 = *reinterpret_cast<const float4*>(kp);
        k1 = *reinterpret_cast<const float4*>(kp + 4);
      }
      kv[t][0] = k0.x; kv[t][1] = k0.y; kv[t][2] = k0.z; kv[t][3] = k0.w;
      kv[t][4] = k1.x; kv[t][5] = k1.y; kv[t][6] = k1.z; kv[t][7] = k1.w;
    }
    // S^T tiles: lane (col, grp) gets keys 16t + 4grp + e for query col
    f32x4 sc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sc[t] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < 8; ++s) sc[t] = mfma4(kv[t][s], qv[s], sc[t]);
    }
    if (base + 64 > L) {  // ragged last chunk
#pragma unroll
      for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (base + 16 * t + 4 * grp + e >= L) sc[t][e] = -INFINITY;
    }
    float cm = -INFINITY;
#pragma unroll
    for (int t = 0; t < 4; ++t) cm = max3(cm, max3(sc[t][0], sc[t][1], sc[t][2]), sc[t][3]);
    const float mn = fmaxf(m, group_max(cm));
    const float corr = __builtin_amdgcn_exp2f(m - mn);  // 0 on the first chunk
    o0 *= corr;
    o1 *= corr;
    lsum *= corr;
    m = mn;
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        sc[t][e] = __builtin_amdgcn_exp2f(sc[t][e] - mn);
        lsum += sc[t][e];
      }
    __syncthreads();  // the chunk's V staged
    // O^T += V^T P^T: k-step (t, e) = keys 16t + 4g + e; A' row col = dim col (+16)
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float* vr = vs + (16 * t + 4 * grp + e) * kVStride;
        o0 = mfma4(vr[col], sc[t][e], o0);
        o1 = mfma4(vr[16 + col], sc[t][e], o1);
      }
  }
  const float inv = 1.0f / group_sum(lsum);

  // ---- LCE of query col, channels c0 + 4grp + e and c0 + 16 + 4grp + e
  float l0[4], l1[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    l0[e] = a.b ? a.b[c0 + 4 * grp + e] : 0.f;
    l1[e] = a.b ? a.b[c0 + 16 + 4 * grp + e] : 0.f;
  }
  const int hy = qt / rw, hx = qt % rw;  // window top-left in halo coordinates
  for (int ay = 0; ay < 5; ++ay) {
#pragma unroll
    for (int ax = 0; ax < 5; ++ax) {
      const float* hp = halo + ((hy + ay) * WP + hx + ax) * kHaloStride;
      const float* wp = wt + (5 * ay + ax) * 32;
      const float4 v0 = *reinterpret_cast<const float4*>(hp + 4 * grp);
      const float4 v1 = *reinterpret_cast<const float4*>(hp + 16 + 4 * grp);
      const float4 w0 = *reinterpret_cast<const float4*>(wp + 4 * grp);
      const float4 w1 = *reinterpret_cast<const float4*>(wp + 16 + 4 * grp);
      l0[0] = fmaf(w0.x, v0.x, l0[0]); l0[1] = fmaf(w0.y, v0.y, l0[1]);
      l0[2] = fmaf(w0.z, v0.z, l0[2]); l0[3] = fmaf(w0.w, v0.w, l0[3]);
      l1[0] = fmaf(w1.x, v1.x, l1[0]); l1[1] = fmaf(w1.y, v1.y, l1[1]);
      l1[2] = fmaf(w1.z, v1.z, l1[2]); l1[3] = fmaf(w1.w, v1.w, l1[3]);
    }
  }
  float* op = a.out + (size_t)n * H * W * C + ((size_t)qy * W + qx) * C + c0;
  *reinterpret_cast<float4*>(op + 4 * grp) =
      make_float4(fmaf(o0[0], inv, l0[0]), fmaf(o0[1], inv, l0[1]), fmaf(o0[2], inv, l0[2]), fmaf(o0[3], inv, l0[3]));
  *reinterpret_cast<float4*>(op + 16 + 4 * grp) =
      make_float4(fmaf(o1[0], inv, l1[0]), fmaf(o1[1], inv, l1[1]), fmaf(o1[2], inv, l1[2]), fmaf(o1[3], inv, l1[3]));
}

}  // namespace

bool f32_kernel_supports(const Shape& s) {
  if (s.hd != 32 || s.T % 16 != 0 || s.T > 256) return false;  // one wave per 16 queries, <= 16 waves
  return f32_lds(s.rh, s.rw).total <= 160 * 1024;
}

// Can the kernel choose the routes itself: S*S <= 64 candidates, and at
// least one wave per 16 of them (a wave per 16 queries)?
bool f32_kernel_routes(const Shape& s) {
  return f32_kernel_supports(s) && s.R <= 64 && s.T / 16 >= (s.R + 15) / 16 && s.C % 32 == 0;
}

// Routes given (route), or with qr and kr (the region means;
// f32_kernel_routes) chosen in the kernel and written to route_out.
hipError_t launch_attend_f32(const void* q, const void* k, const void* v, const void* w,
                             const void* b, const int32_t* route, const Shape& s, void* out,
                             hipStream_t st, const float* qr, const float* kr, int32_t* route_out) {
  F32Args a;
  a.q = (const float*)q; a.k = (const float*)k; a.v = (const float*)v;
  a.w = (const float*)w; a.b = (const float*)b; a.route = route; a.out = (float*)out;
  a.qr = qr; a.kr = kr; a.route_out = route_out;
  a.rscale = (float)(1.0 / __builtin_sqrt((double)s.C));
  a.N = s.N; a.H = s.H; a.W = s.W; a.C = s.C; a.heads = s.heads; a.S = s.S; a.topk = s.topk;
  a.rh = s.rh; a.rw = s.rw;
  a.qscale = (float)(1.4426950408889634 / __builtin_sqrt((double)s.hd));
  const unsigned blocks = (unsigned)(s.N * s.R * s.heads);
  launch(attn_f32_kernel, dim3(blocks), dim3(4 * s.T), f32_lds(s.rh, s.rw).total, st, a);
  return hipGetLastError();
}

}  // namespace bra
