// Gathered attention + LCE for small images, bf16 tensors: 2x2-token regions
// -- the third classification stage of BiFormer (a 14x14 map, S = 7, topk =
// 16) -- and 4x4-token regions -- the second stage (28x28, S = 7, topk = 4),
// where one kernel also pools the region means and routes (Eqs. 3-7 of the
// BRA walk-through at TRANSFORMER.niftyadmin.cn/n/347023.html, section
// BRA模块). The 2x2 kernel first:
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
// Scores are column-stacked: a 16x16 score tile holds 4 key tiles x 4
// queries (column j = key tile j % 4 for query j / 4; each lane keeps its
// column's tile from the four K x Q^T products), so every exponential is a
// real one and a query's four columns form a lane quad. For P.V each tile's
// P is broadcast over the quad (quad_perm DPP), so every column sums all the
// keys of its query and the quad holds four copies of the result. A lane
// then owns one (query, channel pair) -- the copies split the query's 32
// dims into 16 channel pairs -- and adds the LCE of its pair and stores it.
#include "bra_internal.h"
#include "route_common.h"

#include <type_traits>

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

// the 4 bf16 of quad lane FROM (0..3), in every lane of the quad
template <int FROM>
__device__ __forceinline__ bf16x4 quad_bcast(bf16x4 x) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_bit_cast(u32x2, x);
  constexpr int ctrl = FROM * 0x55;  // quad_perm [FROM, FROM, FROM, FROM]
  u32x2 r;
  r[0] = __builtin_amdgcn_update_dpp(v[0], v[0], ctrl, 0xf, 0xf, false);
  r[1] = __builtin_amdgcn_update_dpp(v[1], v[1], ctrl, 0xf, 0xf, false);
  return __builtin_bit_cast(bf16x4, r);
}
// one of four values by the two bits of i
__device__ __forceinline__ float pick4(bool b0, bool b1, float v0, float v1, float v2, float v3) {
  return b1 ? (b0 ? v3 : v2) : (b0 ? v1 : v0);
}

// LDS bank swizzles (16-byte piece index XOR). K token (y, x): piece ^ (y & 1
// | ((x >> 1) & 1) << 1) -- the eight K rows an 8-lane group reads (two
// routed 2x2 regions) spread over the banks. Bordered V row py: piece ^ 3 on
// odd rows -- a region's two token rows, and the LCE windows of vertically
// adjacent queries, fall on different banks.
__device__ __forceinline__ int kswz(int y, int x) { return (y & 1) | (((x >> 1) & 1) << 1); }
__device__ __forceinline__ int vswz(int py) { return 3 * (py & 1); }

struct ImageArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint32_t* wpk;     // packed LCE weights; the tap-major part is used
  const uint16_t* b;       // LCE bias or null
  const int32_t* route;    // [N][S*S][topk] (null: the kernel routes itself)
  uint16_t* out;
  int N, H, W, C, heads, S, topk;
  float qscale;            // head_dim^-1/2 * log2(e)
  // the whole forward inside the kernel (4x4 regions): the raw LCE weights
  // [C][5][5], where the routes are reported, and C^-1/2
  const uint16_t* lw;
  int32_t* route_out;
  float rscale;
  // divisions of staging indices (all below 2^16) by W, W + 4, S and the
  // route stride, as multiply-highs
  FastDiv dw, dwp, ds, drs;
};

__host__ __device__ constexpr size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// route slots per region in LDS: topk rounded up to whole 64-key chunks
// (64 / T slots per chunk)
__host__ __device__ constexpr int route_stride(int topk, int T) {
  return (topk + 64 / T - 1) / (64 / T) * (64 / T);
}

struct ImgLds {
  size_t k, v, rk, rv, w, x, sink, total;
};
// K [H*W][32] and bordered V [(H+4)*(W+4)][32] bf16 of one head; the routes
// as byte offsets of each routed region's first K and V token within those
// arrays [S*S][route_stride] (16-bit: each array stays under 64 KB); the
// head's LCE weights as dot2 operands [16 pairs][5 rows][8 dwords]; for 4x4
// regions each wave's hand-over of the attention output [16 queries][36]
// fp32; a sink for unused stores.
// Bordered-V row pitch in pixels: W + 4, or for 4x4 regions a fixed 32 (the
// LCE window then sits at constant offsets from one address).
constexpr int kVRow4 = 32;
__host__ __device__ constexpr int vrow(int RS, int W) { return RS == 4 ? kVRow4 : W + 4; }
__host__ __device__ inline ImgLds img_lds(int RS, int NW, int H, int W, int R, int topk) {
  ImgLds l;
  size_t o = 0;
  l.k = o; o += (size_t)H * W * 64;
  l.v = o; o += (size_t)(H + 4) * vrow(RS, W) * 64;
  l.rk = o; o += align16((size_t)R * route_stride(topk, RS * RS) * 2);
  l.rv = o; o += align16((size_t)R * route_stride(topk, RS * RS) * 2);
  l.w = o; o += RS == 4 ? (size_t)kLceToepDwords * 4 : 16 * 5 * 32;  // Toeplitz LCE blocks / dot2 operands
  l.x = o; o += RS == 4 ? (size_t)NW * 16 * 36 * 4 : 0;
  l.sink = o; o += 16;
  l.total = o;
  return l;
}

// FULL: every 64-key chunk is whole (topk * 4 a multiple of 64), so no key
// is masked
template <int NW, bool FULL>
__global__ __launch_bounds__(64 * NW) void attn_image2_kernel(ImageArgs a) {
  constexpr int RS = 2, RH = RS, RW = RS, T = RS * RS;  // 2x2 regions
  constexpr int nthreads = 64 * NW;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int H = a.H, W = a.W, C = a.C, S = a.S, R = S * S, topk = a.topk;
  const int L = topk * T, WP = W + 4, RSTR = route_stride(topk, T);
  const ImgLds lay = img_lds(RS, NW, H, W, R, topk);
  uint16_t* kh = reinterpret_cast<uint16_t*>(smem + lay.k);
  uint16_t* vh = reinterpret_cast<uint16_t*>(smem + lay.v);
  uint16_t* rk = reinterpret_cast<uint16_t*>(smem + lay.rk);
  uint16_t* rv = reinterpret_cast<uint16_t*>(smem + lay.rv);
  uint32_t* wl = reinterpret_cast<uint32_t*>(smem + lay.w);
  uint16_t* sink = reinterpret_cast<uint16_t*>(smem + lay.sink);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;

  const int u = xcd_unit((int)blockIdx.x, (int)gridDim.x);  // heads of one image share an XCD
  const int n = u / a.heads, h = u - n * a.heads;
  const size_t img = (size_t)n * H * W * C;
  const uint32_t img_bytes = (uint32_t)H * W * C * 2;
  const Rsrc qb = rsrc(a.q + img, img_bytes), kb = rsrc(a.k + img, img_bytes);
  const Rsrc ob = rsrc(a.out + img, img_bytes);
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
        const int pix = i >> 2, py = (int)fdiv(a.dwp, (uint32_t)pix);
        const int y = py - 2, x = pix - py * WP - 2;
        const bool in = i < vp && y >= 0 && y < H && x >= 0 && x < W;  // border: zero
        vbuf[j] = ld16(vb, in ? (uint32_t)(y * W + x) * pixb + hoff + (uint32_t)(i & 3) * 16 : kOut);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + j * nthreads + tid;
        const int tok = i >> 2, y = (int)fdiv(a.dw, (uint32_t)tok), x = tok - y * W;
        const int pc = (i & 3) ^ kswz(y, x);
        *reinterpret_cast<uint4*>(i < kp ? kh + (size_t)(4 * tok + pc) * 8 : sink) = kbuf[j];
      }
#pragma unroll
      for (int j = 0; j < 6; ++j) {
        const int i = j0 + j * nthreads + tid;
        const int pix = i >> 2, py = (int)fdiv(a.dwp, (uint32_t)pix);
        const int pc = (i & 3) ^ vswz(py);
        *reinterpret_cast<uint4*>(i < vp ? vh + (size_t)(4 * pix + pc) * 8 : sink) = vbuf[j];
      }
    }
    // route slot p of region r -> offsets of the routed region's first K and
    // bordered-V token (slots past topk: region 0, their keys are masked)
    const int32_t* rt = a.route + (size_t)n * R * topk;
    for (int i = tid; i < R * RSTR; i += nthreads) {
      const int r = (int)fdiv(a.drs, (uint32_t)i), p = i - r * RSTR;
      const int rr = p < topk ? rt[r * topk + p] : 0;
      const int js = (int)fdiv(a.ds, (uint32_t)rr), is = rr - js * S;
      // 2x2 regions: bit 5 carries the region-column parity of the K swizzle
      // (token offsets are 64-byte aligned)
      rk[i] = (uint16_t)(((size_t)(js * RH * W + is * RW) * 64) | (size_t)(RS == 2 ? (is & 1) << 5 : 0));
      rv[i] = (uint16_t)((size_t)((js * RH + 2) * WP + is * RW + 2) * 64);
    }
    // LCE weights of the head's 16 channel pairs as dot2 operands, per kernel
    // row: pixels (0,1) and (2,3) paired per channel (c, then c+1), pixel 4
    // alone with the other half zero
    if (tid < 80) {
      const int cp = tid / 5, ay = tid - cp * 5;
      const uint32_t* wt = a.wpk + 30 * C + h * 16 + cp + 5 * ay * (C / 2);  // tap-major pairs
      uint32_t e[5];
#pragma unroll
      for (int ax = 0; ax < 5; ++ax) e[ax] = wt[ax * (C / 2)];
      uint4 w0, w1;
      w0.x = __builtin_amdgcn_perm(e[1], e[0], 0x05040100u);
      w0.y = __builtin_amdgcn_perm(e[1], e[0], 0x07060302u);
      w0.z = __builtin_amdgcn_perm(e[3], e[2], 0x05040100u);
      w0.w = __builtin_amdgcn_perm(e[3], e[2], 0x07060302u);
      w1.x = e[4] & 0xffffu;
      w1.y = e[4] & 0xffff0000u;
      w1.z = 0u;
      w1.w = 0u;
      *reinterpret_cast<uint4*>(wl + tid * 8) = w0;
      *reinterpret_cast<uint4*>(wl + tid * 8 + 4) = w1;
    }
  }

  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);

  // ---- per-lane constants ---------------------------------------------------
  const int tq = col & 3;    // key tile of this score column
  const int qt = col >> 2;   // query (token of the region) of this score column
  // K row of this lane: token col % 4 of a routed region, piece grp; address
  // = (route entry ^ kx) + kt (the entry carries the region-column bit of the
  // piece swizzle, kx the row bit and the piece)
  const uint32_t kx = 16u * (uint32_t)(grp ^ ((col & 3) >> 1));
  const uint32_t kt = (uint32_t)lay.k + (uint32_t)(((col & 3) / RW) * W + (col & 3) % RW) * 64;
  // V^T row of this lane: token col / 4 (padded row parity col / 8), dims
  // 16hh + 4(col % 4) .. +3 = dwords 8hh + 2(col % 4), +1
  const int vpar = col >> 3, c4 = col & 3;
  const uint32_t vt = (uint32_t)lay.v + (uint32_t)(((col >> 2) / RW) * WP + (col >> 2) % RW) * 64;
  const uint32_t offV0 = vt + 16u * (uint32_t)((c4 >> 1) ^ (3 * vpar)) + 8u * (uint32_t)(c4 & 1);
  const uint32_t offV1 = vt + 16u * (uint32_t)((2 + (c4 >> 1)) ^ (3 * vpar)) + 8u * (uint32_t)(c4 & 1);
  // this lane's output: query qt, channel pair cp of the head
  const int cp = 2 * grp + (tq & 1) + 8 * (tq >> 1);
  const uint32_t bias2 = a.b ? reinterpret_cast<const uint32_t*>(a.b)[h * 16 + cp] : 0u;

  // query pixel of this lane's column in region r (r wave-uniform), and the
  // head's Q row there, prefetched a region ahead
  auto qpix = [&](int r, int& y, int& x) {
    const int js = (int)fdiv(a.ds, (uint32_t)r), is = r - js * S;
    y = js * RH + qt / RW;
    x = is * RW + qt % RW;
  };
  auto qload = [&](int r) {
    int y, x;
    qpix(r, y, x);
    const uint32_t off = r < R ? (uint32_t)(y * W + x) * pixb + hoff + (uint32_t)grp * 16 : kOut;
    return __builtin_bit_cast(bf16x8, ld16(qb, off));
  };
  bf16x8 bq_next = qload(wave_u);
  __syncthreads();  // K, V, routes, weights staged

  // this lane's LCE weights, kept in registers for all its regions
  uint4 wr0[5];
  uint2 wr1[5];
#pragma unroll
  for (int ay = 0; ay < 5; ++ay) {
    wr0[ay] = *reinterpret_cast<const uint4*>(wl + cp * 40 + 8 * ay);
    wr1[ay] = *reinterpret_cast<const uint2*>(wl + cp * 40 + 8 * ay + 4);
  }

  for (int r = wave_u; r < R; r += NW) {
    const bf16x8 bq = bq_next;
    bq_next = qload(r + NW);
    const uint16_t* rkr = rk + r * RSTR;
    const uint16_t* rvr = rv + r * RSTR;

    float m = -INFINITY;  // running max of the scaled (base-2) logits
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0, ls = o0;
    for (int base = 0; base < L; base += 64) {
      // K rows: key base + 16t + col; V^T rows: key base + 16t + 4grp + col / 4
      bf16x8 ak[4];
      uint32_t va[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const uint32_t ka = ((uint32_t)rkr[(base >> 2) + 4 * t + (col >> 2)] ^ kx) + kt;
        va[t] = rvr[(base >> 2) + 4 * t + grp];
        ak[t] = *reinterpret_cast<const bf16x8*>(smem + ka);
      }
      auto vtr = [&](int t, uint32_t off) { return ld_tr(reinterpret_cast<const uint16_t*>(smem + va[t] + off)); };
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      f32x4 st[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) st[g] = mfma(ak[g], bq, z);
      f32x4 s;
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] = pick4(tq & 1, tq & 2, st[0][e], st[1][e], st[2][e], st[3][e]);
      if (!FULL && base + 64 > L) {  // ragged last chunk
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (base + 16 * tq + 4 * grp + e >= L) s[e] = -INFINITY;
      }
      float cm = max3(max3(s[0], s[1], s[2]), s[3], -INFINITY);
      cm = group_max(cm);                        // over the key rows
      cm = dpp_max<0x4e, 0xf>(dpp_max<0xb1, 0xf>(cm));  // over the quad's tiles
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
      // k slots: keys 4g..4g+3 of tiles 2bb and 2bb+1, their P broadcast
      // from the quad lanes that hold them
      const bf16x8 pt0 = cat(quad_bcast<0>(pb), quad_bcast<1>(pb));
      const bf16x8 pt1 = cat(quad_bcast<2>(pb), quad_bcast<3>(pb));
      o0 = mfma(cat(vtr(0, offV0), vtr(1, offV0)), pt0, o0);
      o1 = mfma(cat(vtr(0, offV1), vtr(1, offV1)), pt0, o1);
      ls = mfma(ones, pt0, ls);  // every row of ones x P^T is the row sum of P
      o0 = mfma(cat(vtr(2, offV0), vtr(3, offV0)), pt1, o0);
      o1 = mfma(cat(vtr(2, offV1), vtr(3, offV1)), pt1, o1);
      ls = mfma(ones, pt1, ls);
    }
    // this lane's pair: channels 4grp + 2(tq & 1) (+16 if tq >= 2), +1
    const float inv = __builtin_amdgcn_rcpf(ls[0]);
    const float at0 = pick4(tq & 1, tq & 2, o0[0], o0[2], o1[0], o1[2]) * inv;
    const float at1 = pick4(tq & 1, tq & 2, o0[1], o0[3], o1[1], o1[3]) * inv;

    // LCE of (query pixel, pair): 5x5 window of the bordered V
    int y, x;
    qpix(r, y, x);
    float acc0 = bf16_lo(bias2), acc1 = bf16_hi(bias2), acc2 = 0.f, acc3 = 0.f;
    // window row ay is padded row y + ay; its dwords are swizzled by 12 on odd rows
    const uint32_t* vw = reinterpret_cast<const uint32_t*>(vh) + (size_t)(y * WP + x) * 16;
    const int cpe = cp ^ (12 * (y & 1)), cpo = cp ^ (12 * ((y + 1) & 1));
#pragma unroll
    for (int ay = 0; ay < 5; ++ay) {
      const uint4 w0 = wr0[ay];
      const uint2 w1 = wr1[ay];
      const uint32_t* vr = vw + ay * WP * 16 + ((ay & 1) ? cpo : cpe);
      const uint32_t p0 = vr[0], p1 = vr[16], p2 = vr[32], p3 = vr[48], p4 = vr[64];
      acc0 = dot2(__builtin_amdgcn_perm(p1, p0, 0x05040100u), w0.x, acc0);
      acc1 = dot2(__builtin_amdgcn_perm(p1, p0, 0x07060302u), w0.y, acc1);
      acc2 = dot2(__builtin_amdgcn_perm(p3, p2, 0x05040100u), w0.z, acc2);
      acc3 = dot2(__builtin_amdgcn_perm(p3, p2, 0x07060302u), w0.w, acc3);
      acc0 = dot2(p4, w1.x, acc0);
      acc1 = dot2(p4, w1.y, acc1);
    }
    const uint32_t packed = pack_bf16x2(at0 + (acc0 + acc2), at1 + (acc1 + acc3));
    st_nt(ob, (uint32_t)((y * W + x) * C + 32 * h + 2 * cp) * 2, packed);
  }
}

// ---- 4x4 regions: persistent workgroups ------------------------------------
// One workgroup per CU walks (image, head) units with sixteen waves. While
// the waves work on one unit's regions, every lane holds seven 16-byte pieces
// of the next unit's K, V and LCE weights (and one route entry) in registers,
// loaded right after the lane's own query rows; at the end of the unit, between
// two barriers, they are written to LDS. A unit's staging thus overlaps the
// previous unit's arithmetic instead of following it. (Loads complete in issue
// order as far as the wait counter goes, so the query rows of all of a wave's
// regions are requested first: no query wait ever waits for the prefetch.)
//
// A score tile is one routed region (16 keys) against the region's 16
// queries (lane column = query); P.V reads V^T straight from LDS, where the
// bordered V is stored as horizontal pixel pairs per channel. The LCE runs on
// the matrix cores: a 4x4x4 product with 16 independent blocks gives each
// block one channel's 4x4 output tile, each window row adding its 8 pixels
// (two chunks of 4) times a Toeplitz block of that row's 5 weights; the
// attention output, handed over through LDS, is the accumulator's start.
//
// The whole forward in one kernel (FUSE): a workgroup takes heads h and
// h + heads/2 of one image. It pools the image's q and k into the region
// means -- in the pool kernel's summation order, so the means, and so the
// routes, are the stage-by-stage path's bit for bit -- and routes: waves 0-3
// take 16 rows each (logit tiles with the route kernel's split-bf16 steps,
// then the top k of every row as fp64 codes through sorting networks, merged
// across lane quads) with no workgroup barrier, while the other waves already
// issue the first unit's prefetch. The LCE weights come as given and are built
// into the Toeplitz blocks in LDS for each unit.
constexpr int kNW4 = 16;                       // waves
constexpr int kThreads4 = 64 * kNW4;
constexpr int kPF = 7;                         // prefetch pieces per lane
constexpr int kPFA = 4;                        // of which issued at a unit's start
constexpr int kWPieces = kLceToepDwords / 4;   // a head's Toeplitz LCE blocks in 16-byte pieces
constexpr int kWRawPieces = 32 * 25 * 2 / 16;  // a head's 5x5 weights as given, in 16-byte pieces
constexpr int kVPitch4 = kVRow4 / 2 * 128;     // bytes per bordered-V row: 16 pixel pairs x 32 channels

// Bordered V row Y, pixel pair P, channel c: the dword (pixel 2P, pixel 2P+1)
// at byte (Y * 16 + P) * 128 + 4 * (c ^ vsw(Y)). The swizzle flips channel
// bits 4 and 3 by row: the two rows of a P.V read's 32-lane pass (16 dims
// each) and the four rows of a window read's 16-lane pass (8 dwords each)
// fall on different banks.
__host__ __device__ constexpr int vsw(int Y) { return 16 * (Y & 1) + 8 * ((Y >> 1) & 1); }

__device__ __forceinline__ f32x4 mfma4(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x4bf16_1k(a, b, c, 0, 0, 0);
}

// LDS-only workgroup barrier: orders LDS accesses across it without waiting
// for global loads and stores still in flight
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Routing inside the kernel (C <= 128): the region means, as split bf16 rows
// in LDS
constexpr int kRouteMaxC = 128;
// LDS the in-kernel routing borrows from the weight and hand-over areas: the
// logits [R][16 ceil(R/16) + 1] fp32
__host__ __device__ inline size_t route_logits_bytes(int R) { return align16((size_t)R * (16 * ((R + 15) / 16) + 1) * 4); }

// FK: whole K/V slot pairs of the prefetch (4 H W / 1024, rounded down);
// FUSE: the kernel computes its units' routes from the region means (a
// workgroup then has at most two units)
template <int FK, bool FUSE>
__global__ __launch_bounds__(kThreads4) void attn_image4_kernel(ImageArgs a) {
  constexpr int RH = 4, RW = 4, T = 16;
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int H = a.H, W = a.W, C = a.C, S = a.S, R = S * S, topk = a.topk;
  const int L = topk * T, HW = H * W, RSTR = route_stride(topk, T);
  const ImgLds lay = img_lds(4, kNW4, H, W, R, topk);
  uint16_t* rk = reinterpret_cast<uint16_t*>(smem + lay.rk);
  uint16_t* rv = reinterpret_cast<uint16_t*>(smem + lay.rv);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  const int units = a.N * a.heads, G = (int)gridDim.x;
  const uint32_t pixb = (uint32_t)C * 2;  // bytes per pixel
  const uint32_t img_bytes = (uint32_t)HW * C * 2;
  const int nroute = R * RSTR;
  const float inv_w = 1.0f / (float)W;

  // ---- the next unit's K, V, weights and routes ------------------------------
  // Slots 2jj and 2jj+1 (jj < FK) hold K and V of pixel tid / 4 + 256jj, chunk
  // tid % 4: whole slots of one tensor at a fixed pixel stride, so a load is a
  // per-lane base plus a uniform offset. The remaining slots are mixed: the
  // last remK K pieces, the same V pieces, then the head's LCE blocks. Route
  // slot tid rides along. (A V pixel's horizontal partner is always in lane
  // tid ^ 4 of the same slot: pixel pairs are even-aligned, remK is a multiple
  // of 8.)
  u32x4 pf[kPF];
  uint32_t rq = 0;
  const int remK = 4 * HW - FK * kThreads4;
  constexpr int kWP = FUSE ? kWRawPieces : kWPieces;  // weight pieces
  auto route_off = [&](int i) {  // byte offset of route slot i's entry, or kOut
    const int r = i / RSTR, p = i - r * RSTR;
    return i < nroute && p < topk ? (uint32_t)(r * topk + p) * 4 : kOut;
  };
  // The lane's piece indices are rederived from an opaque copy of its thread
  // index in each call: hoisted out of the unit loop, the addresses would
  // hold dozens of registers next to the prefetched data.
  auto opaque_tid = [&]() {
    int t = tid;
    asm volatile("" : "+v"(t));
    return t;
  };
  // (real == false: the same loads, past the buffers or all of one address,
  // discarded: every path issues the same loads)
  auto prefetch = [&](int u, bool real, int j0 = 0, int j1 = kPF) {  // slots [j0, j1)
    const int tid = opaque_tid();
    const int n = u / a.heads, h = u - n * a.heads;
    const size_t img = (size_t)n * HW * C;
    const Rsrc kb = rsrc(a.k + img, img_bytes), vb = rsrc(a.v + img, img_bytes);
    const char* kp = reinterpret_cast<const char*>(a.k + img);
    const char* vp = reinterpret_cast<const char*>(a.v + img);
    // the head's LCE weights: as given (built into Toeplitz blocks in LDS), or
    // packed beforehand
    const char* wp = FUSE ? reinterpret_cast<const char*>(a.lw + (size_t)h * 32 * 25)
                          : reinterpret_cast<const char*>(a.wpk + lce_toep_offset(C) + (size_t)h * kLceToepDwords);
    int keep = real ? 1 : 0;  // a lane value: the selects below stay selects, not branches
    asm volatile("" : "+v"(keep));
    const uint32_t lb = keep ? (uint32_t)(tid >> 2) * pixb + (uint32_t)(tid & 3) * 16 : kOut;
#pragma unroll
    for (int j = 0; j < kPF; ++j) {
      if (j < j0 || j >= j1) continue;
      if (j < 2 * FK) {
        const uint32_t so = (uint32_t)h * 64 + (uint32_t)(j >> 1) * 256 * pixb;
        pf[j] = __builtin_bit_cast(u32x4, ld16s((j & 1) ? vb : kb, lb, so));
      } else {
        const int m = tid + kThreads4 * (j - 2 * FK);
        const bool isk = m < remK, isv = !isk && m < 2 * remK;
        const int i2 = FK * kThreads4 + (isk ? m : m - remK);  // piece of K or V
        const size_t po = (size_t)(i2 >> 2) * pixb + (size_t)h * 64 + (size_t)(i2 & 3) * 16;
        const int iw = m - 2 * remK;
        // one load from a per-lane address (a tensor per lane); pieces past
        // the operands, and every piece of a discarded prefetch, re-read the
        // first K piece of the unit
        const char* src = !keep ? kp : isk ? kp + po : isv ? vp + po : iw < kWP ? wp + (size_t)iw * 16 : kp;
        pf[j] = *reinterpret_cast<const u32x4*>(src);
      }
    }
    if (!FUSE && j0 == 0) {  // (routed in the kernel: rq already holds the routes)
      const Rsrc rrs = rsrc(a.route + (size_t)n * R * topk, (uint32_t)(R * topk) * 4);
      rq = __builtin_amdgcn_raw_buffer_load_b32(rrs, keep ? route_off(tid) : kOut, 0, 0);
    }
    asm volatile("" ::: "memory");  // issued here: not sunk toward their use
  };
  auto route_put = [&](int i, int rr) {  // slot i -> the routed region's first K token, first V pixel pair
    const int js = rr / S, is = rr - js * S;
    rk[i] = (uint16_t)((js * RH * W + is * RW) * 64);
    rv[i] = (uint16_t)(((js * RH + 2) * 16 + is * (RW / 2) + 1) * 128);
  };
  // K piece (pixel, chunk c) -> its swizzled 16 bytes
  auto k_put = [&](int pix, int c, u32x4 d) {
    const int y = (int)(((float)pix + 0.5f) * inv_w), x = pix - y * W;  // exact: pix < 2^12
    *reinterpret_cast<u32x4*>(smem + lay.k + (4 * pix + (c ^ ((((x >> 1) & 1) << 1) | (y & 1)))) * 16) = d;
  };
  // V piece (pixel, chunk c: channels 8c..8c+7), its partner pixel's same
  // piece in lane ^ 4: the even pixel's lane writes channels 8c..8c+3 of the
  // pair, the odd one 8c+4..8c+7 (each as four (even, odd) dwords)
  auto v_put = [&](int pix, int c, u32x4 d) {
    const bool odd = pix & 1;
    const uint32_t s0 = odd ? d[0] : d[2], s1 = odd ? d[1] : d[3];
    const uint32_t r0 = (uint32_t)__shfl_xor((int)s0, 4), r1 = (uint32_t)__shfl_xor((int)s1, 4);
    const uint32_t a0 = odd ? r0 : d[0], a1 = odd ? r1 : d[1];  // even pixel's dwords
    const uint32_t b0 = odd ? d[2] : r0, b1 = odd ? d[3] : r1;  // odd pixel's
    const int y = (int)(((float)pix + 0.5f) * inv_w), x = pix - y * W;
    const int Y = y + 2, P = (x + 2) >> 1, sw = vsw(Y);
    u32x4 o;
    o[0] = __builtin_amdgcn_perm(b0, a0, 0x05040100u);
    o[1] = __builtin_amdgcn_perm(b0, a0, 0x07060302u);
    o[2] = __builtin_amdgcn_perm(b1, a1, 0x05040100u);
    o[3] = __builtin_amdgcn_perm(b1, a1, 0x07060302u);
    const int cg = (8 * c + 4 * (int)odd) ^ sw;  // the swizzle moves whole 4-dword groups
    *reinterpret_cast<u32x4*>(smem + lay.v + (Y * 16 + P) * 128 + cg * 4) = o;
  };
  auto commit = [&](int u, bool with_routes) {
    const int tid = opaque_tid();
    const int c = tid & 3;
#pragma unroll
    for (int jj = 0; 2 * jj + 1 < kPF; ++jj) {
      if (jj < FK) {
        const int pix = (tid >> 2) + 256 * jj;
        k_put(pix, c, pf[2 * jj]);
        v_put(pix, c, pf[2 * jj + 1]);
      }
    }
#pragma unroll
    for (int j = 0; j < kPF; ++j) {
      if (j >= 2 * FK) {
        const int m = tid + kThreads4 * (j - 2 * FK);
        const bool isk = m < remK, isv = !isk && m < 2 * remK;
        const int i2 = FK * kThreads4 + (isk ? m : m - remK);
        const int iw = m - 2 * remK;
        if (isk) k_put(i2 >> 2, c, pf[j]);
        if (isv) v_put(i2 >> 2, c, pf[j]);  // partners share the branch (8-aligned pairs)
        if (!isk && !isv && iw < kWP) *reinterpret_cast<u32x4*>(smem + (FUSE ? lay.x : lay.w) + iw * 16) = pf[j];
        if (FUSE && iw == kWP) *reinterpret_cast<uint32_t*>(smem + lay.x + kWP * 16) = 0u;  // the zero weight
      }
    }
    if (with_routes && tid < nroute) route_put(tid, (int)rq);
    // retire the prefetch registers on every path (the writes above are
    // guarded; left pending on the path that skips them, they would make the
    // next unit's first load wait on its own query rows)
#pragma unroll
    for (int j = 0; j < kPF; ++j) asm volatile("" : "+v"(pf[j]));
    asm volatile("" : "+v"(rq));
    if (!FUSE && nroute > kThreads4) {  // large route tables: the rest read here
      const int n = u / a.heads;
      const Rsrc rrs = rsrc(a.route + (size_t)n * R * topk, (uint32_t)(R * topk) * 4);
      for (int i = tid + kThreads4; i < nroute; i += kThreads4)
        route_put(i, (int)__builtin_amdgcn_raw_buffer_load_b32(rrs, route_off(i), 0, 0));
    }
  };


  // FUSE: the head's Toeplitz LCE blocks, built from the weights that commit
  // left in the hand-over area (between two barriers). Which two weights a
  // lane's dwords e = tid + 1024 i take is the same for every head, so it is
  // worked out once (u16 indices into the weights; 800 is a zero just past
  // them).
  constexpr int kToepPer = (kLceToepDwords + kThreads4 - 1) / kThreads4;  // 3
  uint32_t tsrc[kToepPer];
  if constexpr (FUSE) {
#pragma unroll
    for (int i = 0; i < kToepPer; ++i) {
      const int e = tid + kThreads4 * i, f = 2 * (e < kLceToepDwords ? e : 0);
      const int k = f & 3, j = (f >> 2) & 3, b = (f >> 4) & 15, ch = (f >> 8) & 1;
      const int dy = (f >> 9) % 5, hh = (f >> 9) / 5;
      const int c = 2 * b + hh, tap = 4 * ch + k - j, base = c * 25 + dy * 5;
      const uint32_t lo = tap >= 0 && tap < 5 ? (uint32_t)(base + tap) : 800u;
      const uint32_t hi = tap + 1 >= 0 && tap + 1 < 5 ? (uint32_t)(base + tap + 1) : 800u;
      tsrc[i] = lo | (hi << 16);
    }
  }
  auto toep_build = [&]() {
    const uint16_t* raw = reinterpret_cast<const uint16_t*>(smem + lay.x);
    uint32_t* wl = reinterpret_cast<uint32_t*>(smem + lay.w);
    uint32_t v[kToepPer];
#pragma unroll
    for (int i = 0; i < kToepPer; ++i)
      v[i] = (uint32_t)raw[tsrc[i] & 0xffffu] | ((uint32_t)raw[tsrc[i] >> 16] << 16);
#pragma unroll
    for (int i = 0; i < kToepPer; ++i)
      if (tid + kThreads4 * i < kLceToepDwords) wl[tid + kThreads4 * i] = v[i];
  };

  // the V border (two pixels around the image) stays zero for every unit:
  // rows 0, 1, H + 2, H + 3 whole, and pixel pairs 0 and W / 2 + 1 of the rest
  // (written once, just before the first unit is staged)
  auto zero_border = [&]() {
    const int top = 4 * 16 * 8;  // 16-byte pieces
    const uint4 z4 = make_uint4(0u, 0u, 0u, 0u);
    for (int i = tid; i < top + H * 16; i += kThreads4) {
      int Y, P;
      if (i < top) {
        const int rr = i >> 7;
        Y = rr < 2 ? rr : H + rr;
        P = (i >> 3) & 15;
      } else {
        const int i2 = i - top;
        Y = 2 + (i2 >> 4);
        P = (i2 & 8) ? W / 2 + 1 : 0;
      }
      *reinterpret_cast<uint4*>(smem + lay.v + (Y * 16 + P) * 128 + (i & 7) * 16) = z4;
    }
  };

  // ---- the query rows and LCE bias of a unit --------------------------------
  // A wave takes regions first, first + 16, ... (at most four: R <= 64); the
  // start rotates with the unit so the waves that take an extra region change.
  // The loads are issued a unit ahead, before that unit's staging is written.
  const int lb4 = lane >> 2, lq = lane & 3;  // LCE: matrix block (channels 2lb4, +1), row / column lq
  bf16x8 q0, q1, q2, q3;
  uint32_t bias2;
  auto qrows = [&](int u, int it) {
    const int n = u / a.heads, h = u - n * a.heads;
    const Rsrc qb = rsrc(a.q + (size_t)n * HW * C, img_bytes);
    const int first = (wave + kNW4 - it % kNW4) % kNW4;
    auto qload = [&](int r) {
      const int js = r / S, is = r - js * S;
      const int y = js * RH + (col >> 2), x = is * RW + (col & 3);
      const uint32_t off = r < R ? (uint32_t)(y * W + x) * pixb + (uint32_t)h * 64 + (uint32_t)grp * 16 : kOut;
      return __builtin_bit_cast(bf16x8, ld16(qb, off));
    };
    q0 = qload(first);
    q1 = qload(first + kNW4);
    q2 = qload(first + 2 * kNW4);
    q3 = qload(first + 3 * kNW4);
    bias2 = a.b ? reinterpret_cast<const uint32_t*>(a.b)[h * 16 + lb4] : 0u;
  };

  // ---- the units of this workgroup: unit_of(it), it < nits. Routing in the
  // kernel, a workgroup takes heads h and h + heads/2 of one image (the image
  // is routed once for both; the workgroups of heads h, h + 1 run side by
  // side on one XCD and share the cache lines of their channels); else units
  // b, b + G, ... Either way neighbouring units share an XCD.
  const int nits = FUSE ? 2 : (units - (int)blockIdx.x + G - 1) / G;
  auto unit_of = [&](int it) {
    if constexpr (FUSE) {
      const int hh = a.heads / 2, pi = xcd_unit((int)blockIdx.x, units / 2);
      const int n = pi / hh;
      return n * a.heads + (pi - n * hh) + it * hh;
    } else {
      return xcd_unit((int)blockIdx.x + it * G, units);
    }
  };
  const int u0 = unit_of(0);
  if constexpr (FUSE) {
    // ---- the image's routes, from q and k. The region means Q^r and K^r
    // are computed here and written to the K/V area as bf16 hi and lo rows,
    // split as the route kernel splits them (rows C + 8 apart to spread the
    // banks); the logits (the route kernel's split-bf16 steps, so the same
    // logits) and the top k follow below, and pick what the route kernel's
    // ranks pick. The routes go straight to the route table (both units share
    // it); the workgroup with head 0 reports them. The logits use the weight
    // and hand-over areas; the means and logits are overwritten when the
    // first unit is staged.
    const int CT = (R + 15) / 16, RP = 16 * CT + 1;  // odd pitch: a lane per row reads without conflicts
    float* logits = reinterpret_cast<float*>(smem + lay.w);            // [R][RP]
    const int n0 = u0 / a.heads;
    const int RS = C + 8;                      // bf16 per LDS row
    // matrix m (0: Q^r, 1: K^r), part 0 (hi) / 1 (lo): R rows of RS bf16
    auto mat_lds = [&](int m, int part) { return (__bf16*)(smem + lay.k) + (size_t)(2 * m + part) * R * RS; };
    // The means over all C channels, from q and k: a task is one region of
    // q (task < R) or of k (task - R); the lane sums 16-byte chunk pc
    // (channels 8 pc..8 pc + 7) of tasks psl and psl + slots in fp32, in the
    // pool kernel's order: each region column top to bottom, then the four
    // column sums left to right (so both give the same means, bit for bit).
    // Its 32 loads go out as eight batches of four (one region column),
    // three batches in flight. (Lanes without a task read the image's first
    // piece and drop it.)
    const int nch = C / 8, slots = kThreads4 / nch;
    const int pc = tid % nch, psl = tid / nch;
    const char* qimg = reinterpret_cast<const char*>(a.q + (size_t)n0 * HW * C);
    const char* kimg = reinterpret_cast<const char*>(a.k + (size_t)n0 * HW * C);
    const char* tb[2];
    uint32_t rstep[2], cstep[2];
    bool tok[2];
    int tmat[2], treg[2];
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int tk = psl + slots * p;
      tok[p] = psl < slots && tk < 2 * R;
      tmat[p] = tk >= R ? 1 : 0;
      treg[p] = tk - tmat[p] * R;
      const int js = treg[p] / S, is = treg[p] - js * S;
      tb[p] = tok[p] ? (tmat[p] ? kimg : qimg) + (size_t)(4 * js * W + 4 * is) * pixb + (size_t)pc * 16 : qimg;
      rstep[p] = tok[p] ? (uint32_t)W * pixb : 0u;
      cstep[p] = tok[p] ? pixb : 0u;
    }
    float acc[2][8];
#pragma unroll
    for (int p = 0; p < 2; ++p)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[p][e] = 0.f;
    auto pool_issue = [&](int i, u32x4* b) {  // batch i: task i / 4, region column i % 4
      const int p = i >> 2;
      const char* src = tb[p] + (i & 3) * cstep[p];
#pragma unroll
      for (int py = 0; py < 4; ++py) b[py] = *reinterpret_cast<const u32x4*>(src + py * rstep[p]);
    };
    auto pool_add = [&](int i, const u32x4* b) {
      float col[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) col[e] = 0.f;
#pragma unroll
      for (int py = 0; py < 4; ++py)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          col[2 * e] += bf16_lo(b[py][e]);
          col[2 * e + 1] += bf16_hi(b[py][e]);
        }
      float* sm = acc[i >> 2];
#pragma unroll
      for (int e = 0; e < 8; ++e) sm[e] += col[e];
    };
    auto pool_put = [&](int p) {  // mean -> hi and lo bf16 rows (as route::split_bf16)
      // (the sums taken on every path: sunk into the branch below, they
      // would leave the task's loads unretired for lanes without a task)
#pragma unroll
      for (int e = 0; e < 8; ++e) asm volatile("" : "+v"(acc[p][e]));
      if (tok[p]) {
        typedef __bf16 b8 __attribute__((ext_vector_type(8)));
        b8 hi, lo;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float x = acc[p][e] * (1.0f / (RH * RW));  // exact: a power of two
          hi[e] = (__bf16)x;
          lo[e] = (__bf16)(x - (float)hi[e]);
        }
        *reinterpret_cast<b8*>(mat_lds(tmat[p], 0) + treg[p] * RS + 8 * pc) = hi;
        *reinterpret_cast<b8*>(mat_lds(tmat[p], 1) + treg[p] * RS + 8 * pc) = lo;
      }
    };
    u32x4 pbuf[3][4];
    pool_issue(0, pbuf[0]);
    pool_issue(1, pbuf[1]);
    pool_issue(2, pbuf[2]);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      asm volatile("" ::: "memory");  // each batch issued where it stands
      pool_add(i, pbuf[i % 3]);
      if (i == 3) pool_put(0);
      if (i + 3 < 8) pool_issue(i + 3, pbuf[i % 3]);
    }
    pool_put(1);
    lds_barrier();  // the means in LDS
    // Wave rb < 4 routes rows 16 rb .. 16 rb + 15 on its own -- logit tiles
    // (rb, 0..3), then the top k of its rows -- so the routing needs no
    // workgroup barrier, and waves 4.. issue their share of the first unit's
    // prefetch at once (a wave blocked issuing loads holds up no other);
    // waves 0..3 issue theirs when their rows are routed.
    if (wave < 4 && 16 * wave < R) {
      const int rb = wave;
      // logit tiles (rb, ct): each the route kernel's steps in its order (C a
      // multiple of 32); the A rows serve all four tiles, and the next
      // step's operands are read while this step's products run
      const int qrow = min(16 * rb + col, R - 1);
      const __bf16* ah = mat_lds(0, 0) + qrow * RS + 8 * grp;
      const __bf16* al = mat_lds(0, 1) + qrow * RS + 8 * grp;
      uint32_t boff[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) boff[ct] = (uint32_t)(min(16 * ct + col, R - 1) * RS + 8 * grp);
      const __bf16* bh = mat_lds(1, 0);
      const __bf16* bl = mat_lds(1, 1);
      typedef route::rbf16x8 R8;
      f32x4 acc[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4{0.f, 0.f, 0.f, 0.f};
      R8 xah = *reinterpret_cast<const R8*>(ah), xal = *reinterpret_cast<const R8*>(al);
      R8 xbh[4], xbl[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        xbh[ct] = *reinterpret_cast<const R8*>(bh + boff[ct]);
        xbl[ct] = *reinterpret_cast<const R8*>(bl + boff[ct]);
      }
      for (int k0 = 0; k0 < C; k0 += 32) {
        const int kn = k0 + 32 < C ? k0 + 32 : k0;  // (the last step re-reads its own operands)
        const R8 nah = *reinterpret_cast<const R8*>(ah + kn), nal = *reinterpret_cast<const R8*>(al + kn);
        R8 nbh[4], nbl[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          nbh[ct] = *reinterpret_cast<const R8*>(bh + boff[ct] + kn);
          nbl[ct] = *reinterpret_cast<const R8*>(bl + boff[ct] + kn);
        }
        // route::logit_step_x3 for the four tiles, its products interleaved
        // across them
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xah, xbl[ct], acc[ct], 0, 0, 0);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xal, xbh[ct], acc[ct], 0, 0, 0);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xah, xbh[ct], acc[ct], 0, 0, 0);
        xah = nah;
        xal = nal;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          xbh[ct] = nbh[ct];
          xbl[ct] = nbl[ct];
        }
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int row = 16 * rb + 4 * grp + e;
          if (row < R && ct < CT) logits[row * RP + 16 * ct + col] = acc[ct][e] * a.rscale;
        }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // top k (k <= 4) of row 16 rb + lane / 4: lane q = lane % 4 keeps the
      // top 4 of candidates [q cq, (q + 1) cq) (cq <= 16: R <= 64) as rank
      // codes, then the quad merges its four lists (DPP exchanges)
      const int cq = (R + 3) / 4, q = lane & 3, row = 16 * rb + (lane >> 2);
      const float* lg = logits + min(row, R - 1) * RP + q * cq;
      const int nc = min(R, (q + 1) * cq) - q * cq;
      uint32_t kv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float x = lg[min(j, nc - 1)];  // all reads first
        kv[j] = j < nc ? route::key_u32(x) : 0u;
      }
      double g[4][4];
#pragma unroll
      for (int j = 0; j < 16; ++j) g[j >> 2][j & 3] = route::rank_code(kv[j], q * cq + j);
#pragma unroll
      for (int i = 0; i < 4; ++i) route::sort4_code(g[i]);
      route::merge4_code(g[0], g[1]);
      route::merge4_code(g[2], g[3]);
      route::merge4_code(g[0], g[2]);
      auto quad_merge = [&](auto ctrl) {  // merge with the list of the quad lane ctrl names
        double o[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          const uint64_t u = __builtin_bit_cast(uint64_t, g[0][k]);
          const uint32_t lo = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)u, decltype(ctrl)::value, 0xF, 0xF, false);
          const uint32_t hi = (uint32_t)__builtin_amdgcn_mov_dpp((int)(uint32_t)(u >> 32), decltype(ctrl)::value, 0xF, 0xF, false);
          o[k] = __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
        }
        route::merge4_code(g[0], o);
      };
      quad_merge(std::integral_constant<int, 0xB1>{});  // quad_perm [1,0,3,2]
      quad_merge(std::integral_constant<int, 0x4E>{});  // quad_perm [2,3,0,1]
      if (row < R) {  // lane q writes slot q (slots past topk: region 0, masked)
        double tq = g[0][0];
#pragma unroll
        for (int k = 1; k < 4; ++k) tq = q == k ? g[0][k] : tq;
        route_put(row * RSTR + q, q < topk ? route::rank_code_index(tq) : 0);
      }
    }
    asm volatile("" ::: "memory");
    prefetch(u0, true);
    qrows(u0, 0);
    asm volatile("" ::: "memory");
    lds_barrier();  // routed; every read of the means and logits done before staging
    zero_border();
    commit(u0, false);
    lds_barrier();
    toep_build();
  } else {
    zero_border();
    prefetch(u0, true);
    qrows(u0, 0);
    asm volatile("" ::: "memory");
    commit(u0, true);
  }
  lds_barrier();  // the first unit staged
  if constexpr (FUSE) {
    // the workgroup with head 0 reports the image's routes, read back from
    // the route table (K offset 256 (j W + i) for region (j, i)); stores
    // issued now, not while the prefetch still fills the memory queues
    const int n0 = u0 / a.heads;
    if (u0 - n0 * a.heads == 0) {
      for (int i = tid; i < R * topk; i += kThreads4) {
        const int r = i / topk, k = i - r * topk;
        const int ji = rk[r * RSTR + k] >> 8, js = ji / W;
        a.route_out[(size_t)n0 * R * topk + i] = js * S + (ji - js * W);
      }
    }
  }

  // ---- per-lane constants -----------------------------------------------------
  // K row of this lane: token (col / 4, col % 4) of a routed region (whose
  // origin is a multiple of 4, so its swizzle depends on col only)
  const int f = ((col >> 2) & 1) | (((col & 3) >> 1) << 1);
  const uint32_t kt = (uint32_t)lay.k + (uint32_t)((col >> 2) * W + (col & 3)) * 64 + 16u * (uint32_t)(grp ^ f);
  // V^T of P.V: dim col (+16) at routed-region row grp (bordered row 2 + grp
  // modulo 4), pixel pairs 0 and 1 of the region 128 bytes apart
  const uint32_t offV0 = (uint32_t)lay.v + (uint32_t)grp * kVPitch4 + 4u * (uint32_t)(col ^ vsw(2 + grp));
  const uint32_t offV1 = (uint32_t)lay.v + (uint32_t)grp * kVPitch4 + 4u * (uint32_t)((16 + col) ^ vsw(2 + grp));
  // LCE window rows dy = 0..4 of this lane's output row lq: the dword pair of
  // channels 2lb4, 2lb4 + 1 in bordered row lq + dy (modulo 4) of the region
  uint32_t offA[5];
#pragma unroll
  for (int dy = 0; dy < 5; ++dy) offA[dy] = (uint32_t)(lq + dy) * kVPitch4 + 4u * (uint32_t)((2 * lb4) ^ vsw(lq + dy));
  const uint32_t offB = (uint32_t)lay.w + (uint32_t)(lb4 * 4 + lq) * 8;  // Toeplitz block of (lb4, column lq)
  float* xw = reinterpret_cast<float*>(smem + lay.x) + wave * (16 * 36);  // this wave's hand-over
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;

  for (int it = 0; it < nits; ++it) {
    const int u = unit_of(it);
    const int n = u / a.heads, h = u - n * a.heads;
    const Rsrc ob = rsrc(a.out + (size_t)n * HW * C, img_bytes);
    const int first = (wave + kNW4 - it % kNW4) % kNW4;
    const bool more = it + 1 < nits;
    // The next unit's prefetch goes out in two parts, the second after the
    // wave's first region: a wave blocks while the memory queues take its
    // loads, and split this way the waves of a SIMD block at different times.
    // (The first region is peeled so the second part has one definition.)
    const int un = more ? unit_of(it + 1) : u;
    prefetch(un, more, 0, kPFA);
    // Take delivery of the query rows and the bias right after the prefetch
    // was issued: the wait covers just these loads, and the region loop holds
    // no value still in flight (a loop that used one would have the compiler
    // wait for every outstanding load, the prefetch too, before entering it).
    asm volatile("" : "+v"(q0), "+v"(q1), "+v"(q2), "+v"(q3), "+v"(bias2));

    auto region = [&](const int r) {
      const bf16x8 bq = q0;
      q0 = q1;
      q1 = q2;
      q2 = q3;
      const uint16_t* rkr = rk + r * RSTR;
      const uint16_t* rvr = rv + r * RSTR;

      float m = -INFINITY;  // running max of the scaled (base-2) logits
      f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0, ls = o0;
      // one 64-key chunk (four routed regions); ragged: the last, partly past L
      auto chunk = [&](const int base, auto ragged) {
        bf16x8 ak[4];
        uint32_t va[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {  // tile t = route slot base / 16 + t
          const int slot = (base >> 4) + t;
          ak[t] = *reinterpret_cast<const bf16x8*>(smem + rkr[slot] + kt);
          va[t] = rvr[slot];
        }
        // V^T operand: tile t's keys 4grp..4grp+3 (region row grp) for one dim
        auto vtr = [&](int t, uint32_t off) {
          const uint32_t* p = reinterpret_cast<const uint32_t*>(smem + va[t] + off);
          u32x2 d;
          d[0] = p[0];
          d[1] = p[32];
          return __builtin_bit_cast(bf16x4, d);
        };
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4 sc[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) sc[t] = mfma(ak[t], bq, z);
        if constexpr (decltype(ragged)::value) {
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (base + 16 * t + 4 * grp + e >= L) sc[t][e] = -INFINITY;
        }
        float cm = -INFINITY;
#pragma unroll
        for (int t = 0; t < 4; ++t) cm = max3(cm, max3(sc[t][0], sc[t][1], sc[t][2]), sc[t][3]);
        cm = group_max(cm);                        // over the key rows
        const float mn = fmaxf(m, cm * a.qscale);  // qscale > 0 commutes with max
        if (base > 0) {                            // rescale what earlier chunks summed
          const float corr = __builtin_amdgcn_exp2f(m - mn);
          o0 *= corr;
          o1 *= corr;
          ls *= corr;
        }
        m = mn;
        bf16x4 pb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          f32x4 pv;
#pragma unroll
          for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(sc[t][e], a.qscale, -mn));
          pb[t] = to_bf16x4(pv);
        }
#pragma unroll
        for (int bb = 0; bb < 2; ++bb) {
          // k slots: keys 4g..4g+3 of tiles 2bb and 2bb+1
          const bf16x8 pt = cat(pb[2 * bb], pb[2 * bb + 1]);
          o0 = mfma(cat(vtr(2 * bb, offV0), vtr(2 * bb + 1, offV0)), pt, o0);
          o1 = mfma(cat(vtr(2 * bb, offV1), vtr(2 * bb + 1, offV1)), pt, o1);
          ls = mfma(ones, pt, ls);  // every row of ones x P^T is the row sum of P
        }
      };
      int base = 0;
      for (; base + 64 <= L; base += 64) chunk(base, std::false_type{});
      if (base < L) chunk(base, std::true_type{});  // a separate path: whole chunks select nothing

      // hand the output of query col (dims 4grp.., 16 + 4grp..) to the LCE layout
      const float inv = __builtin_amdgcn_rcpf(ls[0]);
      *reinterpret_cast<f32x4*>(xw + col * 36 + 4 * grp) = o0 * inv;
      *reinterpret_cast<f32x4*>(xw + col * 36 + 16 + 4 * grp) = o1 * inv;
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // LCE accumulators start at attention output + bias: block lb4, column
      // lq, rows 0..3 (query 4 row + lq), channels 2lb4 (d0) and 2lb4 + 1 (d1)
      f32x4 d0, d1;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const float2 at = *reinterpret_cast<const float2*>(xw + (4 * p + lq) * 36 + 2 * lb4);
        d0[p] = at.x + bf16_lo(bias2);
        d1[p] = at.y + bf16_hi(bias2);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();  // read before the next region's hand-over
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

      // window: bordered rows 4js + lq + dy, pixel pairs 2is + 2ch, + 1
      const int js = r / S, is = r - js * S;
      const uint32_t rb = (uint32_t)lay.v + (uint32_t)(4 * js * 16 + 2 * is) * 128;
#pragma unroll
      for (int dy = 0; dy < 5; ++dy) {
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          const uint32_t* pa = reinterpret_cast<const uint32_t*>(smem + rb + offA[dy] + ch * 256);
          const u32x2 x0 = *reinterpret_cast<const u32x2*>(pa);       // pair 2is + 2ch: (c, c + 1)
          const u32x2 x1 = *reinterpret_cast<const u32x2*>(pa + 32);  // pair + 1
          u32x2 a0, a1;
          a0[0] = x0[0]; a0[1] = x1[0];
          a1[0] = x0[1]; a1[1] = x1[1];
          const bf16x4 b0 = *reinterpret_cast<const bf16x4*>(smem + offB + ((0 * 5 + dy) * 2 + ch) * 512);
          const bf16x4 b1 = *reinterpret_cast<const bf16x4*>(smem + offB + ((1 * 5 + dy) * 2 + ch) * 512);
          d0 = mfma4(__builtin_bit_cast(bf16x4, a0), b0, d0);
          d1 = mfma4(__builtin_bit_cast(bf16x4, a1), b1, d1);
        }
      }
      const uint32_t oo = (uint32_t)((4 * js) * W + 4 * is + lq) * pixb + (uint32_t)h * 64 + (uint32_t)lb4 * 4;
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        bf16x2 o2;
        o2[0] = (__bf16)d0[p];  // round to nearest even
        o2[1] = (__bf16)d1[p];
        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, o2), ob, oo, (uint32_t)p * W * pixb, 2);  // nt: streamed, not kept in L2
      }
    };
    if (first < R) region(first);
    asm volatile("" ::: "memory");
    prefetch(un, more, kPFA, kPF);
    asm volatile("" ::: "memory");
    for (int r = first + kNW4; r < R; r += kNW4) region(r);
    if (more) {
      qrows(unit_of(it + 1), it + 1);
      asm volatile("" ::: "memory");  // issued here, ahead of the staging below
      lds_barrier();  // every wave is done with this unit's LDS
      commit(unit_of(it + 1), !FUSE);  // (two heads of one image share the routes)
      if constexpr (FUSE) {
        lds_barrier();
        toep_build();
      }
      lds_barrier();  // the next unit staged
    } else {
      // the discarded loads of the last unit retired as well: no path around
      // the loop leaves a prefetch register in flight
#pragma unroll
      for (int j = 0; j < kPF; ++j) asm volatile("" : "+v"(pf[j]));
      asm volatile("" : "+v"(rq));
    }
  }
}

}  // namespace

// 2x2 regions: four waves, four workgroups per CU (the LDS budget)
constexpr int kImage2Waves = 4;

bool image_kernel_supports(const Shape& s) {
  if (s.hd != 32 || s.rh != s.rw || (s.rh != 2 && s.rh != 4)) return false;
  if ((long long)s.H * s.W * s.C >= (1ll << 30)) return false;    // 32-bit byte offsets in an image
  if ((long long)(s.H + 4) * (s.W + 4) * 64 > 65536) return false;  // 16-bit token offsets
  if (s.rh == 2) return img_lds(2, kImage2Waves, s.H, s.W, s.R, s.topk).total <= 40 * 1024;  // four per CU
  {  // prefetch slots: whole K/V pairs, then the mixed remainder
    const int fk = 4 * s.H * s.W / kThreads4, rem = 4 * s.H * s.W - fk * kThreads4;
    if (2 * fk + (2 * rem + kWPieces + kThreads4 - 1) / kThreads4 > kPF) return false;
  }
  if (s.R > 4 * kNW4) return false;  // regions per wave
  if (s.W + 4 > kVRow4 || (long long)(s.H + 4) * kVRow4 * 64 > 65536) return false;  // row pitch, 16-bit offsets
  return img_lds(4, kNW4, s.H, s.W, s.R, s.topk).total <= 160 * 1024;
}

// one persistent workgroup per CU (a multiple of 8, so a workgroup's units
// stay on its XCD), at most one per unit
static int image4_grid(int units) {
  int cus = device_cu_count();
  cus = cus >= 8 ? cus / 8 * 8 : 8;
  return units < cus ? units : cus;
}

bool image_kernel_routes(const Shape& s) {
  if (s.rh != 4 || !image_kernel_supports(s)) return false;
  if (s.heads % 2) return false;                           // head pairs
  if (s.C > kRouteMaxC || s.C % 32 || s.R > 64) return false;  // split steps, 64 candidates
  if (s.topk > 4) return false;                            // top 4 by insertion
  const int units = s.N * s.heads;
  if (units / 2 > image4_grid(units)) return false;        // a workgroup per head pair, in one round
  if (2 * s.R > 2 * (kThreads4 / (s.C / 8))) return false;  // the pooling's two tasks a lane
  const ImgLds l = img_lds(4, kNW4, s.H, s.W, s.R, s.topk);
  if ((size_t)4 * s.R * (s.C + 8) * 2 > l.rk - l.k) return false;  // the split means in the K/V area
  if ((size_t)kWRawPieces * 16 > l.sink - l.x) return false;        // the raw weights in the hand-over area
  return route_logits_bytes(s.R) <= l.sink - l.w;          // the logits in the weight and hand-over areas
}

static ImageArgs image_args(const void* q, const void* k, const void* v, const void* b,
                            const Shape& s, void* out) {
  ImageArgs a = {};
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.b = (const uint16_t*)b; a.out = (uint16_t*)out;
  a.N = s.N; a.H = s.H; a.W = s.W; a.C = s.C; a.heads = s.heads; a.S = s.S; a.topk = s.topk;
  a.qscale = (float)(1.4426950408889634 / __builtin_sqrt((double)s.hd));
  a.rscale = (float)(1.0 / __builtin_sqrt((double)s.C));  // as the route kernels
  a.dw = make_fastdiv((uint32_t)s.W);
  a.dwp = make_fastdiv((uint32_t)s.W + 4);
  a.ds = make_fastdiv((uint32_t)s.S);
  a.drs = make_fastdiv((uint32_t)route_stride(s.topk, s.T));
  return a;
}

#define BRA_IMG4(FKV, FU) launch(attn_image4_kernel<FKV, FU>, g, blk, lds, st, a)
#define BRA_IMG4_FK(FU)                  \
  switch (4 * s.H * s.W / kThreads4) {   \
    case 0: BRA_IMG4(0, FU); break;      \
    case 1: BRA_IMG4(1, FU); break;      \
    case 2: BRA_IMG4(2, FU); break;      \
    default: BRA_IMG4(3, FU); break;     \
  }

hipError_t launch_attend_image(const void* q, const void* k, const void* v, const uint32_t* wpk,
                               const void* b, const int32_t* route, const Shape& s, void* out,
                               hipStream_t st) {
  ImageArgs a = image_args(q, k, v, b, s, out);
  a.wpk = wpk; a.route = route;
  const int units = s.N * s.heads;
  if (s.rh == 2) {
    const size_t lds = img_lds(2, kImage2Waves, s.H, s.W, s.R, s.topk).total;
    if (s.L % 64 == 0)
      launch(attn_image2_kernel<kImage2Waves, true>, dim3((unsigned)units), dim3(64 * kImage2Waves), lds, st, a);
    else
      launch(attn_image2_kernel<kImage2Waves, false>, dim3((unsigned)units), dim3(64 * kImage2Waves), lds, st, a);
  } else {
    const size_t lds = img_lds(4, kNW4, s.H, s.W, s.R, s.topk).total;
    const dim3 g((unsigned)image4_grid(units)), blk(kThreads4);
    BRA_IMG4_FK(false)
  }
  return hipGetLastError();
}

hipError_t launch_forward_image(const void* q, const void* k, const void* v, const void* lce_w,
                                const void* b, const Shape& s, void* out, int32_t* route_out,
                                hipStream_t st) {
  ImageArgs a = image_args(q, k, v, b, s, out);
  a.lw = (const uint16_t*)lce_w; a.route_out = route_out;
  const size_t lds = img_lds(4, kNW4, s.H, s.W, s.R, s.topk).total;
  const dim3 g((unsigned)(s.N * s.heads / 2)), blk(kThreads4);  // a workgroup per head pair
  BRA_IMG4_FK(true)
  return hipGetLastError();
}
#undef BRA_IMG4_FK
#undef BRA_IMG4

}  // namespace bra
