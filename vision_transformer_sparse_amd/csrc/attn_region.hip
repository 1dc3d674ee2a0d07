// Gathered attention + LCE for small regions (T = RH*RW <= 16 tokens), bf16
// tensors -- the classification stages of BiFormer (4x4 and 2x2 regions of a
// 7x7 grid). Eqs. 6-7 of the BRA walk-through at
// TRANSFORMER.niftyadmin.cn/n/347023.html, section BRA模块.
//
// One workgroup owns one query region (n, r) and all its heads, one wave per
// head (64 * HEADS threads, C = 32 * HEADS channels, both compile-time, as
// are the region sides RH x RW). Every global load it needs is issued up
// front, so a workgroup pays about one memory latency:
//
//   A. each wave reads the region's route indices with scalar loads and,
//      as soon as they land, issues its head's gathered K and V rows (the
//      16-key tiles of the MFMA, 16 bytes per lane); meanwhile the V halo
//      (RH+4 x RW+4 pixels, zero outside the image) is staged in LDS as
//      horizontal pixel pairs per channel ([row][pair][C] dwords), the LCE
//      weights (pre-packed as dot2 pairs) are staged in LDS and the head's
//      16 query columns are loaded;
//   B. per head, S^T = K Q^T and O^T = V^T P^T on 16x16x32 bf16 MFMAs (V^T
//      produced on the matrix cores by a 0/1 selector; the softmax row sums
//      by an all-ones operand, so they sum exactly the bf16 P that multiplies
//      V), fp32 online softmax in base 2; the head output goes to LDS;
//   C. LCE on packed bf16 dot products: a thread owns a channel pair and a
//      region column; each halo row gives three pixel-pair dot2s per channel
//      to each of the (up to five) output rows it touches. Added to the
//      attention output and stored as bf16 pairs.
//
// Workgroups are numbered so that all regions of one image go to the same
// XCD (dispatch is round-robin over the 8 XCDs), keeping an image's K/V in
// that XCD's L2 while its regions gather from each other.
#include "bra_internal.h"

namespace bra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ bf16x8 load8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
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
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}
// Buffer loads (rsrc, ld16) read offsets past the image (kOut) as zero:
// used for pixels outside the image.
__device__ __forceinline__ bf16x8 ld16_bf16(Rsrc r, uint32_t off) {
  return __builtin_bit_cast(bf16x8, ld16(r, off));
}

struct RegionArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint32_t* wpk;     // LCE weights packed for dot2: [2 parity][5 rows][3 pairs][C]
  const uint16_t* b;
  const int32_t* route;    // [N][S*S][topk]
  uint16_t* out;
  int N, H, W, S, topk;
  float qscale;            // head_dim^-1/2 * log2(e) (attention, base 2)
  float inv_s;             // 1 / S
};

__host__ __device__ constexpr size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

struct Lds {
  size_t halo, wts, att, sink, total;
};
__host__ __device__ inline Lds lds_layout(int RH, int RW, int C) {
  Lds l;
  size_t o = 0;
  l.halo = o; o += align16((size_t)(RH + 4) * ((RW + 5) / 2) * C * 4);
  l.wts = o; o += align16((size_t)25 * (C / 2) * 4);
  l.att = o; o += align16((size_t)RH * RW * C * 4);
  l.sink = o; o += 32;  // target of the stores of out-of-range slots; never read
  l.total = o;
  return l;
}

template <int RH, int RW, int HEADS>
__global__ __launch_bounds__(64 * HEADS, 4) void attn_region_kernel(RegionArgs a) {
  constexpr int C = 32 * HEADS;  // channels (head_dim 32)
  constexpr int T = RH * RW;     // divides 16: a 16-key tile holds whole regions
  constexpr int HP = RH + 4, WP = RW + 4;
  constexpr int NPAIR = (WP + 1) / 2;  // halo column pairs (an odd width gets a zero column)
  constexpr int nthreads = 2 * C;      // one wave per head
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int W = a.W, H = a.H, S = a.S, R = S * S, topk = a.topk;
  const int L = topk * T;
  const Lds lay = lds_layout(RH, RW, C);
  uint32_t* halo = reinterpret_cast<uint32_t*>(smem + lay.halo);  // [HP][NPAIR][C]
  uint32_t* wts = reinterpret_cast<uint32_t*>(smem + lay.wts);    // [25 taps][C/2] channel pairs
  float* lce = reinterpret_cast<float*>(smem + lay.att);          // [T][C] fp32: LCE or attention
  uint32_t* sink = reinterpret_cast<uint32_t*>(smem + lay.sink);  // [8]

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;

  // XCD-aware numbering: consecutive units (one image's regions) share blockIdx % 8.
  const int units = a.N * R;
  const int per = (units + 7) / 8;
  const int u = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (u >= units) return;  // the whole workgroup leaves together
  const int n = u / R, r = u - n * R;
  const int jr = r / S, ir = r - jr * S;
  const int y0 = jr * RH, x0 = ir * RW;
  const size_t img = (size_t)n * H * W * C;
  const uint32_t img_bytes = (uint32_t)H * W * C * 2;
  const Rsrc qb = rsrc(a.q + img, img_bytes), kbuf = rsrc(a.k + img, img_bytes);
  const Rsrc vbuf = rsrc(a.v + img, img_bytes);
  const Rsrc ob = rsrc(a.out + img, img_bytes);
  const uint32_t rowb = (uint32_t)W * C * 2;  // bytes per image row
  constexpr uint32_t pixb = C * 2;            // bytes per pixel
  const int c0 = wave * 32;                   // this wave's head
  const uint32_t chb = (uint32_t)(c0 + 8 * grp) * 2;  // this lane's 8 channels

  // ---- A: every load of the workgroup ------------------------------------
  // Route indices first (one 4-byte load per lane and key tile: the index of
  // the region that holds this lane's key), then the loads that do not depend
  // on them (V halo, LCE weights, queries), then the gathered K/V rows they
  // address.
  const Rsrc rtb = rsrc(a.route + (size_t)u * topk, (uint32_t)topk * 4);
  constexpr int NR = 16 / T;  // regions per 16-key tile
  int rv[4];
  auto read_routes = [&](int base) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int p = base / T + t * NR + (int)(col / T);  // past topk: read as 0, masked below
      rv[t] = (int)__builtin_amdgcn_raw_buffer_load_b32(rtb, (uint32_t)p * 4, 0, 0);
    }
  };
  read_routes(0);

  constexpr int NSLOT = HP * NPAIR, NIT = (NSLOT + 15) / 16;
  constexpr uint32_t chunks = C / 8;
  const uint32_t hch = tid % chunks, slot0 = tid / chunks;  // 16 threads per 8-channel chunk
  uint4 va[NIT], vb[NIT];
#pragma unroll
  for (int i = 0; i < NIT; ++i) {
    const int pp = slot0 + 16 * i;
    const int pr = pp % NPAIR, py = pp / NPAIR;
    const int y = y0 - 2 + py, x = x0 - 2 + 2 * pr;
    const bool rowok = pp < NSLOT && y >= 0 && y < H;
    const uint32_t hbase = (uint32_t)y * rowb + hch * 16;
    va[i] = ld16(vbuf, rowok && x >= 0 && x < W ? hbase + (uint32_t)x * pixb : kOut);
    vb[i] = ld16(vbuf, rowok && x + 1 >= 0 && x + 1 < W && 2 * pr + 1 < WP ? hbase + (uint32_t)(x + 1) * pixb : kOut);
  }
  // the LCE weights, tap-major channel pairs (after the pixel-pair layout)
  constexpr int pieces = 25 * C / 8;  // 16-byte pieces, < 2 * nthreads
  const Rsrc wb = rsrc(a.wpk + 30 * C, (uint32_t)pieces * 16);
  uint4 wv[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) wv[i] = ld16(wb, (uint32_t)(tid + i * nthreads) * 16);
  const uint32_t qt = col % T;  // the query of this lane's score column
  const bf16x8 bq = ld16_bf16(qb, (y0 + qt / RW) * rowb + (x0 + qt % RW) * pixb + chb);
  // LCE bias of this thread's channel pair (no bias: zeros)
  const uint32_t bias2 = __builtin_amdgcn_raw_buffer_load_b32(
      rsrc(a.b, a.b ? (uint32_t)C * 2 : 0u), (uint32_t)(tid % (C / 2)) * 4, 0, 0);
  // keep this issue order: the gathered loads below wait for the routes only
  __builtin_amdgcn_sched_barrier(0);

  const uint32_t ltok = (uint32_t)(col % T);  // token of this lane's key row within its region
  const uint32_t toff = (ltok / RW) * rowb + (ltok % RW) * pixb + chb;
  bf16x8 ak[4], av[4];
  auto fetch = [&](int base) {  // rv holds the routes of keys base .. base + 63
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      // region (js, is) of index rv[t]: (rv + 1/2) / S is at least 1/(2S) away
      // from an integer, so the float quotient floors exactly
      const int js = (int)(((float)rv[t] + 0.5f) * a.inv_s), is = rv[t] - js * S;
      const uint32_t rb = (uint32_t)(js * RH) * rowb + (uint32_t)(is * RW) * pixb;
      // keys past L read as zero (their scores are masked)
      const bool live = base + 16 * t + (int)(col / T) * T < L;
      ak[t] = ld16_bf16(kbuf, live ? rb + toff : kOut);
      av[t] = ld16_bf16(vbuf, live ? rb + toff : kOut);
    }
  };
  fetch(0);
  __builtin_amdgcn_sched_barrier(0);  // all loads issued before the first LDS store waits

  // V halo as horizontal pixel pairs per channel, weights -> LDS
  // (stores of slots past the end go to `sink`, not behind a branch: a
  // guarded store lets the compiler sink its load under the guard and then
  // wait there for every load issued before it)
#pragma unroll
  for (int i = 0; i < NIT; ++i) {
    const int pp = slot0 + 16 * i;
    // channel c of the pair: low half = left pixel, high half = right pixel
    uint4 lo, hi;
    lo.x = (va[i].x & 0xffffu) | (vb[i].x << 16); lo.y = (va[i].x >> 16) | (vb[i].x & 0xffff0000u);
    lo.z = (va[i].y & 0xffffu) | (vb[i].y << 16); lo.w = (va[i].y >> 16) | (vb[i].y & 0xffff0000u);
    hi.x = (va[i].z & 0xffffu) | (vb[i].z << 16); hi.y = (va[i].z >> 16) | (vb[i].z & 0xffff0000u);
    hi.z = (va[i].w & 0xffffu) | (vb[i].w << 16); hi.w = (va[i].w >> 16) | (vb[i].w & 0xffff0000u);
    uint32_t* dst = NSLOT % 16 == 0 || pp < NSLOT ? halo + (size_t)pp * C + 8 * hch : sink;
    *reinterpret_cast<uint4*>(dst) = lo;
    *reinterpret_cast<uint4*>(dst + 4) = hi;
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int e = tid + i * nthreads;
    *reinterpret_cast<uint4*>(e < pieces ? wts + 4 * e : sink) = wv[i];
  }

  // The LCE of this thread's item: (C/2) channel pairs x RW columns <= 2C,
  // so at most one item per thread; acc0/acc1 get its channels c and c+1 for
  // the RH rows of column xcol.
  const bool has_item = tid < (C / 2) * RW;
  const int cp = tid % (C / 2), xcol = has_item ? tid / (C / 2) : 0;
  const int c = 2 * cp;
  auto lce_item = [&](float* acc0, float* acc1) {
#pragma unroll
    for (int i = 0; i < RH; ++i) { acc0[i] = bf16_lo(bias2); acc1[i] = bf16_hi(bias2); }
    // One weight row at a time (few live registers while the gathered K/V
    // are in flight). Pixel-pair weights from the tap weights: an even
    // column pairs taps (0,1) (2,3) (4,-); an odd one starts a pixel earlier:
    // (-,0) (1,2) (3,4). x: channel c (low halves), y: channel c+1.
    const bool even = (xcol & 1) == 0;
    const uint32_t* hc = halo + (xcol >> 1) * C + c;
#pragma unroll
    for (int ay = 0; ay < 5; ++ay) {
      uint32_t d[5];
#pragma unroll
      for (int ax = 0; ax < 5; ++ax) d[ax] = wts[(5 * ay + ax) * (C / 2) + cp];
      const uint32_t e6[6] = {even ? d[0] : 0u, even ? d[1] : d[0], even ? d[2] : d[1],
                              even ? d[3] : d[2], even ? d[4] : d[3], even ? 0u : d[4]};
      uint2 wv[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        wv[j].x = __builtin_amdgcn_perm(e6[2 * j + 1], e6[2 * j], 0x05040100u);
        wv[j].y = __builtin_amdgcn_perm(e6[2 * j + 1], e6[2 * j], 0x07060302u);
      }
#pragma unroll
      for (int yo = 0; yo < RH; ++yo) {
        const uint32_t* hr = hc + (yo + ay) * NPAIR * C;
        const uint2 h0 = *reinterpret_cast<const uint2*>(hr);
        const uint2 h1 = *reinterpret_cast<const uint2*>(hr + C);
        const uint2 h2 = *reinterpret_cast<const uint2*>(hr + 2 * C);
        acc0[yo] = dot2(h0.x, wv[0].x, acc0[yo]);
        acc0[yo] = dot2(h1.x, wv[1].x, acc0[yo]);
        acc0[yo] = dot2(h2.x, wv[2].x, acc0[yo]);
        acc1[yo] = dot2(h0.y, wv[0].y, acc1[yo]);
        acc1[yo] = dot2(h1.y, wv[1].y, acc1[yo]);
        acc1[yo] = dot2(h2.y, wv[2].y, acc1[yo]);
      }
    }
  };

  // Two orders of the phases, fixed per shape. With eight heads (512
  // threads, two workgroups per CU) the LCE runs first, while the gathered
  // K/V are still in flight, and the attention waves add it to their output;
  // with fewer heads (four workgroups per CU, which already cover each
  // other's latency) the attention runs first and the LCE threads merge.
  constexpr bool kLceFirst = HEADS >= 8;
  if constexpr (kLceFirst) {
    __syncthreads();  // halo and weights staged
    if (has_item) {
      float acc0[RH], acc1[RH];
      lce_item(acc0, acc1);
#pragma unroll
      for (int yo = 0; yo < RH; ++yo)
        *reinterpret_cast<float2*>(lce + (yo * RW + xcol) * C + c) = make_float2(acc0[yo], acc1[yo]);
    }
    __syncthreads();  // the LCE of every channel staged
  }

  // ---- B: attention, head = wave -----------------------------------------
  // A 16-column score tile holds only T queries, so for T < 16 it carries
  // G = min(16 / T, 4) key tiles side by side: column j is query j % T
  // against key tile j / T of its group (the K tiles multiply copies of Q^T
  // masked to their own columns, summed into one accumulator), and every
  // score computed is a real one. P keeps that layout through P.V -- each
  // column sums the keys of its own tile -- and the G column partials of a
  // query are added after the last chunk.
  {
    constexpr int NR = 16 / T;
    constexpr int G = NR < 4 ? NR : 4;  // key tiles per score tile
    constexpr int NO = 4 / G;           // score tiles per 64-key chunk
    const int tq = col / T;             // this column's tile in its group (>= G: no tile)
    bf16x8 sel0, sel1, ones;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      sel0[e] = (__bf16)((grp == (col >> 3) && e == (col & 7)) ? 1.0f : 0.0f);
      sel1[e] = (__bf16)((grp == 2 + (col >> 3) && e == (col & 7)) ? 1.0f : 0.0f);
      ones[e] = (__bf16)1.0f;
    }
    const bf16x8 zero8 = {};
    float m = -INFINITY;  // running max of the scaled (base-2) logits
    f32x4 o0 = {0.f, 0.f, 0.f, 0.f}, o1 = o0, ls = o0;
    for (int base = 0; base < L; base += 64) {
      // keys past the first 64 (topk * T > 64): their routes, then their
      // rows, loaded in turn (prefetching them during the softmax would cost
      // about 30 more registers per lane in every shape)
      if (base > 0) {
        read_routes(base);
        fetch(base);
      }
      f32x4 s[NO];
      bf16x4 vt[4][2];
#pragma unroll
      for (int o = 0; o < NO; ++o) {
        s[o] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int g = 0; g < G; ++g) s[o] = mfma(ak[o * G + g], G == 1 || tq == g ? bq : zero8, s[o]);
      }
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        vt[t][0] = to_bf16x4(mfma(av[t], sel0, z));
        vt[t][1] = to_bf16x4(mfma(av[t], sel1, z));
      }
      // mask keys past L (ragged last chunk) and columns of no tile (T < 4)
      if (T < 4 || base + 64 > L) {
#pragma unroll
        for (int o = 0; o < NO; ++o)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (tq >= G || base + 16 * (o * G + tq) + 4 * grp + e >= L) s[o][e] = -INFINITY;
      }
      float cm = -INFINITY;
#pragma unroll
      for (int o = 0; o < NO; ++o) cm = max3(cm, max3(s[o][0], s[o][1], s[o][2]), s[o][3]);
      cm = row_class_max<T>(group_max(cm));     // over the key rows, then the tiles of a query
      const float mn = fmaxf(m, cm * a.qscale);  // qscale > 0 commutes with max
      if (base > 0) {                            // rescale what earlier chunks summed
        const float corr = __builtin_amdgcn_exp2f(m - mn);
        o0 *= corr;
        o1 *= corr;
        ls *= corr;
      }
      m = mn;
      bf16x4 pb[NO];
#pragma unroll
      for (int o = 0; o < NO; ++o) {
        f32x4 pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(s[o][e], a.qscale, -mn));
        pb[o] = to_bf16x4(pv);
      }
#pragma unroll
      for (int bb = 0; bb < 2; ++bb) {
        // k slots: keys of tiles 2bb and 2bb+1; a column takes P only for its own tile
        const int t0 = 2 * bb;
        bf16x8 pt;
        if constexpr (G == 1) {
          pt = cat(pb[t0], pb[t0 + 1]);
        } else {
          const bf16x4 zero4 = {};
          const bf16x4 p = pb[t0 / G];
          pt = cat(tq == t0 % G ? p : zero4, tq == (t0 + 1) % G ? p : zero4);
        }
        o0 = mfma(cat(vt[t0][0], vt[t0 + 1][0]), pt, o0);
        o1 = mfma(cat(vt[t0][1], vt[t0 + 1][1]), pt, o1);
        ls = mfma(ones, pt, ls);  // every row of ones x P^T is the row sum of P
      }
    }
    if constexpr (G > 1) {  // add the tile partials of each query
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o0[e] = row_class_sum<T>(o0[e]);
        o1[e] = row_class_sum<T>(o1[e]);
      }
      ls[0] = row_class_sum<T>(ls[0]);
    }
    const float inv = 1.0f / ls[0];
    if (col < T) {
      if constexpr (kLceFirst) {
        // out = attention + LCE for query col, channels c0+4grp.. and c0+16+4grp..
        const float* lp = lce + col * C + c0 + 4 * grp;
        const float4 l0 = *reinterpret_cast<const float4*>(lp);
        const float4 l1 = *reinterpret_cast<const float4*>(lp + 16);
        uint2 p0, p1;
        p0.x = pack_bf16x2(fmaf(o0[0], inv, l0.x), fmaf(o0[1], inv, l0.y));
        p0.y = pack_bf16x2(fmaf(o0[2], inv, l0.z), fmaf(o0[3], inv, l0.w));
        p1.x = pack_bf16x2(fmaf(o1[0], inv, l1.x), fmaf(o1[1], inv, l1.y));
        p1.y = pack_bf16x2(fmaf(o1[2], inv, l1.z), fmaf(o1[3], inv, l1.w));
        const uint32_t oo = (uint32_t)(((y0 + col / RW) * W + x0 + col % RW) * C + c0 + 4 * grp) * 2;
        st_nt(ob, oo, p0);
        st_nt(ob, oo + 32, p1);
      } else {
        // the head's output -> LDS, for the LCE threads to merge
        float* ap = lce + col * C + c0;
        *reinterpret_cast<float4*>(ap + 4 * grp) = make_float4(o0[0] * inv, o0[1] * inv, o0[2] * inv, o0[3] * inv);
        *reinterpret_cast<float4*>(ap + 16 + 4 * grp) = make_float4(o1[0] * inv, o1[1] * inv, o1[2] * inv, o1[3] * inv);
      }
    }
  }

  if constexpr (!kLceFirst) {
    __syncthreads();  // every head's output staged
    // ---- C: LCE, merged with the attention output, stored as bf16 pairs
    if (has_item) {
      float acc0[RH], acc1[RH];
      lce_item(acc0, acc1);
#pragma unroll
      for (int yo = 0; yo < RH; ++yo) {
        const float2 at = *reinterpret_cast<const float2*>(lce + (yo * RW + xcol) * C + c);
        const uint32_t packed = pack_bf16x2(at.x + acc0[yo], at.y + acc1[yo]);
        st_nt(ob, (uint32_t)(((y0 + yo) * W + x0 + xcol) * C + c) * 2, packed);
      }
    }
  }
}

__global__ __launch_bounds__(256) void lce_pack_kernel(const uint16_t* __restrict__ w, int C,
                                                       uint32_t* __restrict__ wpk) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e < lce_pack_items(C)) pack_lce_item(w, C, e, wpk);
}

template <int RH, int RW, int HEADS>
hipError_t launch_shape(const RegionArgs& a, int R, size_t lds, hipStream_t st) {
  const int units = a.N * R;
  const unsigned blocks = (unsigned)(((units + 7) / 8) * 8);
  launch((attn_region_kernel<RH, RW, HEADS>), dim3(blocks), dim3(64 * HEADS), lds, st, a);
  return hipGetLastError();
}

// Compiled shapes: regions of 1x1 .. 4x4 tokens with 2, 4 or 8 heads.
bool shape_compiled(int rh, int rw, int heads) {
  auto side = [](int v) { return v == 1 || v == 2 || v == 4; };
  return side(rh) && side(rw) && (heads == 2 || heads == 4 || heads == 8);
}

template <int HEADS>
hipError_t dispatch_shape(const RegionArgs& a, const Shape& s, size_t lds, hipStream_t st) {
  switch (s.rh * 8 + s.rw) {
#define BRA_CASE(RH, RW) \
    case RH * 8 + RW: return launch_shape<RH, RW, HEADS>(a, s.R, lds, st);
    BRA_CASE(1, 1) BRA_CASE(1, 2) BRA_CASE(1, 4) BRA_CASE(2, 1) BRA_CASE(2, 2)
    BRA_CASE(2, 4) BRA_CASE(4, 1) BRA_CASE(4, 2) BRA_CASE(4, 4)
#undef BRA_CASE
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

size_t lce_pack_bytes(int C) { return ((size_t)lce_toep_offset(C) + (size_t)(C / 32) * kLceToepDwords) * 4; }

hipError_t launch_lce_pack(const void* w, int C, uint32_t* wpk, hipStream_t st) {
  launch(lce_pack_kernel, dim3((unsigned)((lce_pack_items(C) + 255) / 256)), dim3(256), 0, st,
                     (const uint16_t*)w, C, wpk);
  return hipGetLastError();
}

bool region_kernel_supports(const Shape& s) {
  if (s.hd != 32 || !shape_compiled(s.rh, s.rw, s.heads)) return false;
  if ((long long)s.H * s.W * s.C >= (1ll << 30)) return false;  // 32-bit byte offsets within an image
  return lds_layout(s.rh, s.rw, s.C).total <= 65536;
}

hipError_t launch_attend_region(const void* q, const void* k, const void* v, const uint32_t* wpk,
                                const void* b, const int32_t* route, const Shape& s, void* out,
                                hipStream_t st) {
  RegionArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.wpk = wpk; a.b = (const uint16_t*)b;
  a.route = route;
  a.out = (uint16_t*)out;
  a.N = s.N; a.H = s.H; a.W = s.W; a.S = s.S; a.topk = s.topk;
  a.qscale = (float)(1.4426950408889634 / __builtin_sqrt((double)s.hd));
  a.inv_s = 1.0f / (float)s.S;
  const size_t lds = lds_layout(s.rh, s.rw, s.C).total;
  switch (s.heads) {
    case 2: return dispatch_shape<2>(a, s, lds, st);
    case 4: return dispatch_shape<4>(a, s, lds, st);
    case 8: return dispatch_shape<8>(a, s, lds, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bra
