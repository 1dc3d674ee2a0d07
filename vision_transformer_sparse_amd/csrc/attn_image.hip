// Gathered attention + LCE for small images with 2x2-token regions, bf16
// tensors -- the third classification stage of BiFormer (a 14x14 map, S = 7,
// topk = 16). Eqs. 6-7 of the BRA walk-through at
// TRANSFORMER.niftyadmin.cn/n/347023.html, section BRA模块.
//
// With 4-token regions a region's own work is tiny next to the latency of
// fetching its 64 routed keys, so this kernel makes the image, not the
// region, the unit: one workgroup owns one (image, head). It stages that
// head's K and V for the whole image in LDS once (V inside a 2-pixel zero
// border, which is the LCE padding), plus the image's route table, and then
// its waves walk the query regions, gathering every routed key from LDS:
//
//   K tile      16 keys x 32 dims per ds_read_b128 (lane = key row)
//   V^T tile    ds_read_b64_tr_b16: the transposing read hands each lane one
//               dim of four keys, the A operand of O^T = V^T P^T
//   LCE         the 5x5 window of the query pixel, read from the bordered V
//               without bounds checks
//
// Scores use the column-stacked layout of the small-region kernel: a 16x16
// score tile holds 4 key tiles x 4 queries (column j = query j % 4 against
// key tile j / 4), so every score computed is a real one; each P.V column
// sums its own tile's keys and the four column partials of a query are added
// after the last chunk. A lane then owns one (query, channel pair): the four
// copies of a query's 32 dims are split into 16 channel pairs, and the lane
// adds the LCE of its pair and stores it.
#include "bra_internal.h"

namespace bra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

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
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}
// Transposing LDS read: within each group of 16 lanes, lanes 4r..4r+3 give
// the address of row r's 16 consecutive bf16 (4 each); lane i gets element i
// of rows 0..3.
__device__ __forceinline__ bf16x4 ld_tr(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(bf16x4, v);
}

struct ImageArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint32_t* wpk;     // packed LCE weights; the tap-major part is used
  const uint16_t* b;       // LCE bias or null
  const int32_t* route;    // [N][S*S][topk]
  uint16_t* out;
  int N, H, W, C, heads, S, topk;
  float qscale;            // head_dim^-1/2 * log2(e)
};

__host__ __device__ constexpr size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

struct ImgLds {
  size_t k, v, rb, sink, total;
};
// K [H*W][32] and bordered V [(H+4)*(W+4)][32] bf16 of one head, the route
// table as packed token bases [S*S*topk], a sink for out-of-range stores.
__host__ __device__ inline ImgLds img_lds(int H, int W, int R, int topk) {
  ImgLds l;
  size_t o = 0;
  l.k = o; o += (size_t)H * W * 64;
  l.v = o; o += (size_t)(H + 4) * (W + 4) * 64;
  l.rb = o; o += align16((size_t)R * topk * 4);
  l.sink = o; o += 16;
  l.total = o;
  return l;
}

template <int NW>
__global__ __launch_bounds__(64 * NW) void attn_image_kernel(ImageArgs a) {
  constexpr int RH = 2, RW = 2, T = RH * RW;  // 2x2 regions: 4 key tiles x 4 queries
  constexpr int nthreads = 64 * NW;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int H = a.H, W = a.W, C = a.C, S = a.S, R = S * S, topk = a.topk;
  const int L = topk * T, WP = W + 4;
  const ImgLds lay = img_lds(H, W, R, topk);
  uint16_t* kh = reinterpret_cast<uint16_t*>(smem + lay.k);
  uint16_t* vh = reinterpret_cast<uint16_t*>(smem + lay.v);
  uint32_t* rb = reinterpret_cast<uint32_t*>(smem + lay.rb);
  uint16_t* sink = reinterpret_cast<uint16_t*>(smem + lay.sink);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;

  const int u = xcd_unit((int)blockIdx.x, (int)gridDim.x);  // heads of one image share an XCD
  const int n = u / a.heads, h = u - n * a.heads;
  const size_t img = (size_t)n * H * W * C;
  const uint32_t img_bytes = (uint32_t)H * W * C * 2;
  const Rsrc qb = rsrc(a.q + img, img_bytes), kb = rsrc(a.k + img, img_bytes);
  const Rsrc vb = rsrc(a.v + img, img_bytes);
  const uint32_t pixb = (uint32_t)C * 2;   // bytes per pixel
  const uint32_t hoff = (uint32_t)h * 64;  // byte offset of the head in a pixel

  // ---- stage K, bordered V and the routes ----------------------------------
  {
    const int kp = H * W * 4, vp = (H + 4) * WP * 4;  // 16-byte pieces
    // each pass: up to 4 K and 6 V pieces per thread in flight
    for (int i0 = 0, j0 = 0; i0 < kp || j0 < vp; i0 += 4 * nthreads, j0 += 6 * nthreads) {
      uint4 kbuf[4], vbuf[6];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + j * nthreads + tid;
        kbuf[j] = ld16(kb, i < kp ? (uint32_t)(i >> 2) * pixb + hoff + (uint32_t)(i & 3) * 16 : kOut);
      }
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        const int i = j0 + j * nthreads + tid;
        const int pix = i >> 2;
        const int y = pix / WP - 2, x = pix % WP - 2;
        const bool in = i < vp && y >= 0 && y < H && x >= 0 && x < W;  // border: zero
        vbuf[j] = ld16(vb, in ? (uint32_t)(y * W + x) * pixb + hoff + (uint32_t)(i & 3) * 16 : kOut);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + j * nthreads + tid;
        *reinterpret_cast<uint4*>(i < kp ? kh + (size_t)i * 8 : sink) = kbuf[j];
      }
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        const int i = j0 + j * nthreads + tid;
        *reinterpret_cast<uint4*>(i < vp ? vh + (size_t)i * 8 : sink) = vbuf[j];
      }
    }
    // route p of region r -> K token base | bordered-V token base << 16
    const int32_t* rt = a.route + (size_t)n * R * topk;
    for (int p = tid; p < R * topk; p += nthreads) {
      const int rr = rt[p];
      const int js = rr / S, is = rr - js * S;
      const uint32_t kbase = (uint32_t)(js * RH * W + is * RW);
      const uint32_t vbase = (uint32_t)((js * RH + 2) * WP + is * RW + 2);
      rb[p] = kbase | (vbase << 16);
    }
  }

  // ---- per-lane constants ---------------------------------------------------
  const int tq = col >> 2;   // key tile of this score column
  const int qt = col & 3;    // query (token of the region) of this score column
  const uint32_t offK = (uint32_t)((qt / RW) * W + qt % RW);     // K row token: col % 4
  const uint32_t offV = (uint32_t)((tq / RW) * WP + tq % RW);    // V^T row token: col >> 2
  // this lane's output: query qt, channel pair cp of the head
  const int cp = 2 * grp + (tq & 1) + 8 * (tq >> 1);
  const int gpair = h * 16 + cp;  // channel pair index in the image (channels 2gpair, +1)
  // LCE weights of the pair as dot2 operands, per kernel row: pixels (0,1)
  // and (2,3) paired per channel, pixel 4 alone (the other half zero)
  uint32_t w01c[5], w01d[5], w23c[5], w23d[5], w4c[5], w4d[5];
  {
    const uint32_t* wt = a.wpk + 30 * C + gpair;  // tap-major pairs, [25][C/2]
    uint32_t d[25];
#pragma unroll
    for (int t = 0; t < 25; ++t) d[t] = wt[t * (C / 2)];
#pragma unroll
    for (int ay = 0; ay < 5; ++ay) {
      const uint32_t* e = d + 5 * ay;
      w01c[ay] = __builtin_amdgcn_perm(e[1], e[0], 0x05040100u);
      w01d[ay] = __builtin_amdgcn_perm(e[1], e[0], 0x07060302u);
      w23c[ay] = __builtin_amdgcn_perm(e[3], e[2], 0x05040100u);
      w23d[ay] = __builtin_amdgcn_perm(e[3], e[2], 0x07060302u);
      w4c[ay] = e[4] & 0xffffu;
      w4d[ay] = e[4] & 0xffff0000u;
    }
  }
  const uint32_t bias2 = a.b ? reinterpret_cast<const uint32_t*>(a.b)[gpair] : 0u;

  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  const bf16x8 zero8 = {};
  const bf16x4 zero4 = {};

  // query pixel of column qt in region r, and its Q load (prefetched a region ahead)
  auto qpix = [&](int r, int& y, int& x) {
    const int js = r / S, is = r - js * S;
    y = js * RH + qt / RW;
    x = is * RW + qt % RW;
  };
  auto qload = [&](int r) {
    int y, x;
    qpix(r, y, x);
    const uint32_t off = r < R ? (uint32_t)(y * W + x) * pixb + hoff + (uint32_t)grp * 16 : kOut;
    return __builtin_bit_cast(bf16x8, ld16(qb, off));
  };
  bf16x8 bq_next = qload(wave);
  __syncthreads();  // K, V, routes staged

  for (int r = wave; r < R; r += NW) {
    const bf16x8 bq = bq_next;
    bq_next = qload(r + NW);
    const uint32_t* rbr = rb + r * topk;

    float m = -INFINITY;  // running max of the scaled (base-2) logits
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0, ls = o0;
    for (int base = 0; base < L; base += 64) {
      // K rows: key base + 16t + col; V^T rows: key base + 16t + 4grp + (col >> 2)
      bf16x8 ak[4];
      const uint16_t* vrow[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int pk = (base >> 2) + 4 * t + (col >> 2);
        const int pv = (base >> 2) + 4 * t + grp;
        const uint32_t ek = rbr[pk < topk ? pk : 0];  // keys past L: any row, masked below
        const uint32_t ev = rbr[pv < topk ? pv : 0];
        ak[t] = *reinterpret_cast<const bf16x8*>(kh + ((ek & 0xffffu) + offK) * 32 + 8 * grp);
        vrow[t] = vh + ((ev >> 16) + offV) * 32 + 4 * (col & 3);
      }
      f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int g = 0; g < 4; ++g) s = mfma(ak[g], tq == g ? bq : zero8, s);
      if (base + 64 > L) {  // ragged last chunk
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (base + 16 * tq + 4 * grp + e >= L) s[e] = -INFINITY;
      }
      float cm = max3(max3(s[0], s[1], s[2]), s[3], -INFINITY);
      cm = row_class_max<T>(group_max(cm));     // over the key rows, then the tiles of a query
      const float mn = fmaxf(m, cm * a.qscale);  // qscale > 0 commutes with max
      if (base > 0) {                            // rescale what earlier chunks summed
        const float corr = __builtin_amdgcn_exp2f(m - mn);
        o0 *= corr;
        o1 *= corr;
        ls *= corr;
      }
      m = mn;
      f32x4 pv;
#pragma unroll
      for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(s[e], a.qscale, -mn));
      const bf16x4 pb = to_bf16x4(pv);
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        // k slots: keys 4g..4g+3 of tiles 2bb and 2bb+1; a column takes P only for its own tile
        const bf16x8 pt = cat(tq == 2 * bb ? pb : zero4, tq == 2 * bb + 1 ? pb : zero4);
        o0 = mfma(cat(ld_tr(vrow[2 * bb]), ld_tr(vrow[2 * bb + 1])), pt, o0);
        o1 = mfma(cat(ld_tr(vrow[2 * bb] + 16), ld_tr(vrow[2 * bb + 1] + 16)), pt, o1);
        ls = mfma(ones, pt, ls);  // every row of ones x P^T is the row sum of P
      }
    }
    // add the tile partials of each query
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      o0[e] = row_class_sum<T>(o0[e]);
      o1[e] = row_class_sum<T>(o1[e]);
    }
    const float inv = 1.0f / row_class_sum<T>(ls[0]);
    // this lane's pair: channels 4grp + 2(tq & 1) (+16 if tq >= 2), +1
    const f32x4 oh = tq >= 2 ? o1 : o0;
    const float at0 = ((tq & 1) ? oh[2] : oh[0]) * inv;
    const float at1 = ((tq & 1) ? oh[3] : oh[1]) * inv;

    // LCE of (query pixel, pair): 5x5 window of the bordered V
    int y, x;
    qpix(r, y, x);
    float acc0 = bf16_lo(bias2), acc1 = bf16_hi(bias2);
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(vh) + (size_t)(y * WP + x) * 16 + cp;
#pragma unroll
    for (int ay = 0; ay < 5; ++ay) {
      const uint32_t* vr = vw + ay * WP * 16;
      const uint32_t p0 = vr[0], p1 = vr[16], p2 = vr[32], p3 = vr[48], p4 = vr[64];
      acc0 = dot2(__builtin_amdgcn_perm(p1, p0, 0x05040100u), w01c[ay], acc0);
      acc1 = dot2(__builtin_amdgcn_perm(p1, p0, 0x07060302u), w01d[ay], acc1);
      acc0 = dot2(__builtin_amdgcn_perm(p3, p2, 0x05040100u), w23c[ay], acc0);
      acc1 = dot2(__builtin_amdgcn_perm(p3, p2, 0x07060302u), w23d[ay], acc1);
      acc0 = dot2(p4, w4c[ay], acc0);
      acc1 = dot2(p4, w4d[ay], acc1);
    }
    const uint32_t packed = float_to_bf16_bits(at0 + acc0) | (float_to_bf16_bits(at1 + acc1) << 16);
    *reinterpret_cast<uint32_t*>(a.out + img + (size_t)(y * W + x) * C + 2 * gpair) = packed;
  }
}

}  // namespace

bool image_kernel_supports(const Shape& s) {
  if (s.hd != 32 || s.rh != 2 || s.rw != 2) return false;
  if ((long long)s.H * s.W * s.C >= (1ll << 30)) return false;  // 32-bit byte offsets in an image
  if ((long long)(s.H + 4) * (s.W + 4) >= 65536) return false;   // 16-bit token bases
  return img_lds(s.H, s.W, s.R, s.topk).total <= 40 * 1024;      // four workgroups per CU
}

hipError_t launch_attend_image(const void* q, const void* k, const void* v, const uint32_t* wpk,
                               const void* b, const int32_t* route, const Shape& s, void* out,
                               hipStream_t st) {
  ImageArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.wpk = wpk; a.b = (const uint16_t*)b; a.route = route; a.out = (uint16_t*)out;
  a.N = s.N; a.H = s.H; a.W = s.W; a.C = s.C; a.heads = s.heads; a.S = s.S; a.topk = s.topk;
  a.qscale = (float)(1.4426950408889634 / __builtin_sqrt((double)s.hd));
  const size_t lds = img_lds(s.H, s.W, s.R, s.topk).total;
  const unsigned blocks = (unsigned)(s.N * s.heads);
  launch(attn_image_kernel<4>, dim3(blocks), dim3(256), lds, st, a);
  return hipGetLastError();
}

}  // namespace bra
