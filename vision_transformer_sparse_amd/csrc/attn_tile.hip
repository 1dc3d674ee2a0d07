// Gathered attention + LCE for large regions (T = RH*RW a multiple of 64
// tokens), bf16 tensors -- BiFormer's dense-prediction stages (8x8 regions
// for detection at S=16, 16x16 regions for segmentation at S=8). Eqs. 6-7 of
// the BRA walk-through at TRANSFORMER.niftyadmin.cn/n/347023.html, section
// BRA模块: each query region attends, per head, to the tokens of its topk
// routed regions (topk*T keys, one joint softmax), plus LCE(V).
//
// One workgroup per (image, region, head): 8 waves for regions of 128 or
// more tokens (so that a wave keeps at most two 16-query blocks in registers
// and four waves share a SIMD), else 4. The gathered keys are walked in
// 64-key tiles: 256 threads fetch a tile's K and V rows by route index (16
// bytes each) one tile ahead into registers, then park them in LDS
// row-major. A K operand is one 16-byte LDS read; a V^T operand (eight
// consecutive keys of one channel per lane) is two transposing LDS reads
// (ds_read_b64_tr_b16: the 16 lanes of a group read a 4-key x 16-channel
// block and each gets one channel's 4 keys). Each wave owns T/64 blocks of
// 16 queries and reuses every K / V^T operand read for all of them:
//
//   S^T(16 keys x 16 queries) = K (A: lane = key row) x Q^T (B: lane = query)
//   O^T(16 dims x 16 queries) += V^T (A) x P^T (B),   sum(P) via ones x P^T
//
// Inside each 32-key block the K rows fed to the two score tiles are
// permuted (tile 0 row 4g+e <- key 8g+e, tile 1 row 4g+e <- key 8g+4+e) so
// that a lane's eight scores are eight CONSECUTIVE keys: P^T needs no
// shuffle. Softmax in fp32, base 2, online across tiles; P is rounded to
// bf16 for the products and the row sums are taken over that same bf16 P on
// the matrix cores. The running maximum m is raised only when a score may
// exceed it by more than kTau (then P may reach 2^kTau, which bf16 and the
// fp32 sums hold). Whether one may is first decided from norms: a scaled
// score is at most qscale*|q|*max|k| (Cauchy-Schwarz), with |q| computed
// once and max|k| per tile by the waves that load it; only when that bound
// exceeds m + kTau somewhere in the wave (always on the first tile) is the
// tile's exact maximum taken (a maximum3 tree and two cross-half lane
// swaps) and the accumulators rescaled.
//
// LCE (5x5 depthwise, zero padding 2, bias): the head's 32 channels of the
// V halo (RH+4 x RW+4 pixels) are staged as horizontal pixel pairs and the
// weights as matching pairs, so each lane's output takes 15 packed-bf16 dot
// products per channel. Workgroups of one image are numbered onto one XCD.
#include "bra_internal.h"

namespace bra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kKStr = 40;   // K and V tile row stride (bf16): 32 dims + 8 pad
constexpr float kTau = 64.f;  // slack of the running maximum (log2 units); 2^64 * keys << FLT_MAX

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) { return __builtin_bit_cast(bf16x8, v); }
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
// maximum over the 64 lanes, wave-uniform: quad swaps, half-row and row
// mirrors, then row broadcasts 15 and 31 carry it into lane 63
__device__ __forceinline__ float wave_max(float x) {
  x = dpp_max<0xb1, 0xf>(x);   // quad_perm [1,0,3,2]
  x = dpp_max<0x4e, 0xf>(x);   // quad_perm [2,3,0,1]
  x = dpp_max<0x141, 0xf>(x);  // row_half_mirror
  x = dpp_max<0x140, 0xf>(x);  // row_mirror
  x = dpp_max<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x = dpp_max<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}
// squared norm of eight bf16 (a 16-byte piece)
__device__ __forceinline__ float sq8(uint4 v) {
  float r = 0.f;
  r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.x), __builtin_bit_cast(bf16x2, v.x), r, false);
  r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.y), __builtin_bit_cast(bf16x2, v.y), r, false);
  r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.z), __builtin_bit_cast(bf16x2, v.z), r, false);
  r = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, v.w), __builtin_bit_cast(bf16x2, v.w), r, false);
  return r;
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
// Transposing LDS read: within each group of 16 lanes, lanes 4r..4r+3 give
// the address of row r's 16 consecutive bf16 (4 each); lane i gets element i
// of rows 0..3.
__device__ __forceinline__ bf16x4 ld_tr(const uint16_t* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<uint16_t*>(p)));
  return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}

struct TileArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint32_t* wpk;  // LCE weights as dot2 pairs: [2 parity][15 (row, pair)][C]
  const uint16_t* b;
  const int32_t* route;  // [N][S*S][topk]
  uint16_t* out;
  int N, H, W, C, heads, S, topk;
  float qscale;  // head_dim^-1/2 * log2(e)
};

__host__ __device__ constexpr size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

struct TileLds {
  size_t ks, vs, knorm, halo, wts, total;
};
__host__ __device__ inline TileLds tile_lds(int RH, int RW) {
  TileLds l;
  size_t o = 0;
  l.ks = o; o += align16((size_t)2 * 64 * kKStr * 2);
  l.vs = o; o += align16((size_t)2 * 64 * kKStr * 2);
  l.knorm = o; o += align16((size_t)2 * 4 * 4);
  l.halo = o; o += align16((size_t)(RH + 4) * ((RW + 5) / 2) * 32 * 4);
  l.wts = o; o += align16((size_t)2 * 15 * 32 * 4);
  l.total = o;
  return l;
}

template <int RH, int RW>
constexpr int tile_waves() { return RH * RW >= 128 ? 8 : 4; }

template <int RH, int RW>
__global__ __launch_bounds__((64 * tile_waves<RH, RW>()), 4) void attn_tile_kernel(TileArgs a) {
  constexpr int T = RH * RW;
  constexpr int WAVES = tile_waves<RH, RW>();
  constexpr int QBW = T / (16 * WAVES);  // query blocks of 16 per wave
  constexpr int HP = RH + 4, WP = RW + 4, NPAIR = (WP + 1) / 2;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const TileLds lay = tile_lds(RH, RW);
  uint16_t* ks = reinterpret_cast<uint16_t*>(smem + lay.ks);    // [2][64][kKStr]
  uint16_t* vs = reinterpret_cast<uint16_t*>(smem + lay.vs);    // [2][64][kKStr]
  float* knorm = reinterpret_cast<float*>(smem + lay.knorm);     // [2][4] max |k|^2 per loader wave
  uint32_t* halo = reinterpret_cast<uint32_t*>(smem + lay.halo);  // [HP][NPAIR][32]
  uint32_t* wts = reinterpret_cast<uint32_t*>(smem + lay.wts);    // [2][15][32]

  const int W = a.W, H = a.H, C = a.C, S = a.S, R = S * S, topk = a.topk;
  const int L = topk * T;  // a multiple of 64
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;

  // XCD-aware numbering: consecutive units (n, r, h) share blockIdx % 8.
  const int units = a.N * R * a.heads;
  const int per = (units + 7) / 8;
  const int u = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (u >= units) return;  // the whole workgroup leaves together
  const int h = u % a.heads, nr = u / a.heads;
  const int n = nr / R, r = nr - n * R;
  const int jr = r / S, ir = r - jr * S;
  const int y0 = jr * RH, x0 = ir * RW;
  const size_t img = (size_t)n * H * W * C;
  const uint32_t img_bytes = (uint32_t)H * W * C * 2;
  const Rsrc qb = rsrc(a.q + img, img_bytes), kb = rsrc(a.k + img, img_bytes);
  const Rsrc vb = rsrc(a.v + img, img_bytes);
  const uint32_t rowb = (uint32_t)W * C * 2, pixb = (uint32_t)C * 2;
  const uint32_t hb = (uint32_t)h * 64;  // byte offset of this head's channels
  const int32_t* rrow = a.route + (size_t)nr * topk;

  // ---- tile loader: thread -> (key ld_key of the tile, 8-dim chunk ld_g)
  const int ld_key = tid >> 2, ld_g = tid & 3;
  uint4 kreg, vreg;  // the next tile, in flight during this one
  auto fetch = [&](int tile) {
    const int key = tile * 64 + ld_key;
    const int p = key / T, tt = key - p * T;   // T is compile-time
    const int s = rrow[p];                     // uniform per 4-row group; a cached load
    const int js = s / S, is = s - js * S;
    const uint32_t off = (uint32_t)(js * RH + tt / RW) * rowb + (uint32_t)(is * RW + tt % RW) * pixb +
                         hb + ld_g * 16;
    kreg = ld16(kb, off);
    vreg = ld16(vb, off);
  };
  const bool loader = tid < 256;  // waves 0-3 move the tiles
  auto park = [&](int buf) {
    *reinterpret_cast<uint4*>(ks + (buf * 64 + ld_key) * kKStr + ld_g * 8) = kreg;
    *reinterpret_cast<uint4*>(vs + (buf * 64 + ld_key) * kKStr + ld_g * 8) = vreg;
    // |k|^2 of the key (its four 8-dim pieces sit in one quad of lanes),
    // then the largest of this wave's 16 keys
    float n2 = sq8(kreg);
    n2 += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(n2), 0xb1, 0xf, 0xf, false));
    n2 += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(n2), 0x4e, 0xf, 0xf, false));
    const float wmax = wave_max(n2);
    if (lane == 0) knorm[buf * 4 + wave] = wmax;
  };

  if (loader) fetch(0);

  // ---- halo (the head's 32 channels) and LCE weights -> LDS
  {
    // 4 chunks of 8 channels per pixel pair; 16 pair slots per wave and pass
    constexpr int NSLOT = HP * NPAIR, SLOTS = 16 * WAVES;
    const int ch = tid & 3, slot0 = tid >> 2;
    for (int pp0 = 0; pp0 < NSLOT; pp0 += 2 * SLOTS) {
      uint4 va[2], vb2[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int pp = pp0 + slot0 + SLOTS * i;
        const int pr = pp % NPAIR, py = pp / NPAIR;
        const int y = y0 - 2 + py, x = x0 - 2 + 2 * pr;
        const bool rowok = pp < NSLOT && y >= 0 && y < H;
        const uint32_t base = (uint32_t)y * rowb + hb + ch * 16;
        va[i] = ld16(vb, rowok && x >= 0 && x < W ? base + (uint32_t)x * pixb : kOut);
        vb2[i] = ld16(vb, rowok && x + 1 >= 0 && x + 1 < W && 2 * pr + 1 < WP ? base + (uint32_t)(x + 1) * pixb : kOut);
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int pp = pp0 + slot0 + SLOTS * i;
        if (pp < NSLOT) {
          uint4 lo, hi;
          lo.x = (va[i].x & 0xffffu) | (vb2[i].x << 16); lo.y = (va[i].x >> 16) | (vb2[i].x & 0xffff0000u);
          lo.z = (va[i].y & 0xffffu) | (vb2[i].y << 16); lo.w = (va[i].y >> 16) | (vb2[i].y & 0xffff0000u);
          hi.x = (va[i].z & 0xffffu) | (vb2[i].z << 16); hi.y = (va[i].z >> 16) | (vb2[i].z & 0xffff0000u);
          hi.z = (va[i].w & 0xffffu) | (vb2[i].w << 16); hi.w = (va[i].w >> 16) | (vb2[i].w & 0xffff0000u);
          uint32_t* dst = halo + (size_t)pp * 32 + 8 * ch;
          *reinterpret_cast<uint4*>(dst) = lo;
          *reinterpret_cast<uint4*>(dst + 4) = hi;
        }
      }
    }
    // weights: [2][15][C] -> this head's [2][15][32]; 240 pieces of 16 bytes
    if (tid < 240) {
      const int row = tid >> 3, piece = tid & 7;  // row = parity * 15 + (ay * 3 + j)
      const uint4 w = *reinterpret_cast<const uint4*>(a.wpk + (size_t)row * C + h * 32 + piece * 4);
      *reinterpret_cast<uint4*>(wts + row * 32 + piece * 4) = w;
    }
  }

  // ---- queries: this wave's blocks, B operands
  bf16x8 bq[QBW];
#pragma unroll
  for (int i = 0; i < QBW; ++i) {
    const int t = (wave * QBW + i) * 16 + col;
    bq[i] = as_bf16x8(ld16(qb, (uint32_t)(y0 + t / RW) * rowb + (uint32_t)(x0 + t % RW) * pixb + hb + grp * 16));
  }

  float m[QBW], qn[QBW];  // running maximum; qscale * |q| of the lane's query
  f32x4 o0[QBW], o1[QBW], ls[QBW];
#pragma unroll
  for (int i = 0; i < QBW; ++i) {
    qn[i] = a.qscale * __builtin_sqrtf(group_sum(sq8(__builtin_bit_cast(uint4, bq[i]))));
    m[i] = -INFINITY;
    o0[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    o1[i] = o0[i];
    ls[i] = o0[i];
  }
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;

  // A-operand rows of the two score tiles of a 32-key block (see header)
  const int krow0 = 8 * (col >> 2) + (col & 3), krow1 = krow0 + 4;
  // V^T operand addresses: this lane gives row 8grp + col/4 (+4), channels
  // 4*(col%4) .. +3 of each 16-channel half
  const int vrow = 8 * grp + (col >> 2), vch = 4 * (col & 3);

  const int ntiles = L / 64;
  if (loader) park(0);
  // one 64-key tile, from LDS buffer buf = tile & 1
  auto step = [&](int tile, int buf) {
    __syncthreads();  // tile `buf` parked; the other buffer is free
    if (loader && tile + 1 < ntiles) fetch(tile + 1);
    const uint16_t* kt = ks + buf * 64 * kKStr;
    const uint16_t* vtl = vs + buf * 64 * kKStr;
    const float kmax = __builtin_sqrtf(__builtin_elementwise_maximum(
        __builtin_elementwise_maximum(knorm[buf * 4 + 0], knorm[buf * 4 + 1]),
        __builtin_elementwise_maximum(knorm[buf * 4 + 2], knorm[buf * 4 + 3])));
    bf16x8 ka[4], va0[2], va1[2];
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      ka[2 * b] = as_bf16x8(*reinterpret_cast<const uint4*>(kt + (32 * b + krow0) * kKStr + grp * 8));
      ka[2 * b + 1] = as_bf16x8(*reinterpret_cast<const uint4*>(kt + (32 * b + krow1) * kKStr + grp * 8));
      // keys 32b + 8grp .. +7 of channel col (va0) and 16 + col (va1)
      const uint16_t* vr = vtl + (32 * b + vrow) * kKStr + vch;
      va0[b] = cat(ld_tr(vr), ld_tr(vr + 4 * kKStr));
      va1[b] = cat(ld_tr(vr + 16), ld_tr(vr + 4 * kKStr + 16));
    }
#pragma unroll
    for (int i = 0; i < QBW; ++i) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      f32x4 s[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) s[t] = mfma(ka[t], bq[i], z);
      // Can a score of this tile exceed m + kTau? Not if the norm bound says
      // so for every query of the wave (the common case after the first tile).
      if (__builtin_amdgcn_ballot_w64(qn[i] * kmax > m[i] + kTau) != 0) {
        // this tile's exact maximum for the lane's query (16 scores here, 64 in all)
        const float c0 = max3(s[0][0], s[0][1], s[0][2]), c1 = max3(s[0][3], s[1][0], s[1][1]);
        const float c2 = max3(s[1][2], s[1][3], s[2][0]), c3 = max3(s[2][1], s[2][2], s[2][3]);
        const float c4 = max3(s[3][0], s[3][1], s[3][2]);
        const float cm = group_max(max3(max3(c0, c1, c2), max3(c3, c4, s[3][3]), c4)) * a.qscale;
        // raise the running maximum (and rescale) only where the tile's exceeds
        // it by more than kTau (first tile: everywhere)
        if (cm > m[i] + kTau) {
          const float corr = __builtin_amdgcn_exp2f(m[i] - cm);  // 0 on the first tile
          o0[i] *= corr;
          o1[i] *= corr;
          ls[i] *= corr;
          m[i] = cm;
        }
      }
      bf16x4 pb[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        f32x4 pv;
#pragma unroll
        for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(fmaf(s[t][e], a.qscale, -m[i]));
        pb[t] = to_bf16x4(pv);
      }
#pragma unroll
      for (int b = 0; b < 2; ++b) {
        const bf16x8 pt = cat(pb[2 * b], pb[2 * b + 1]);  // keys 32b + 8g .. 32b + 8g + 7
        o0[i] = mfma(va0[b], pt, o0[i]);
        o1[i] = mfma(va1[b], pt, o1[i]);
        ls[i] = mfma(ones, pt, ls[i]);
      }
    }
    if (loader && tile + 1 < ntiles) park(buf ^ 1);
    };
  for (int tile = 0; tile < ntiles; ++tile) step(tile, tile & 1);
  __syncthreads();  // halo and weights were parked before the first barrier; all reads below

  // ---- LCE + merge + store: lane = (query col, channel group grp); the
  // lane's query rows i = 0..QBW-1 are stacked in one column when RW == 16
  // (one query otherwise), so each halo row is read once for all of them
  const uint32_t* w32 = wts;
  static_assert(QBW == 1 || RW == 16, "stacked queries need 16-token rows");
  const int t0 = wave * QBW * 16 + col;
  const int ty0 = t0 / RW, tx = t0 % RW;
  const int par = tx & 1, p0 = tx >> 1;
  float acc[QBW][8];
  {
    // bias of the lane's channels 4grp.. and 16+4grp.. (no bias: zeros)
    const Rsrc bb = rsrc(a.b, a.b ? (uint32_t)C * 2 : 0u);
    const uint32_t hoff = (uint32_t)(h * 32 + 4 * grp) * 2;
    const uint32_t b01 = __builtin_amdgcn_raw_buffer_load_b32(bb, hoff, 0, 0);
    const uint32_t b23 = __builtin_amdgcn_raw_buffer_load_b32(bb, hoff + 4, 0, 0);
    const uint32_t b45 = __builtin_amdgcn_raw_buffer_load_b32(bb, hoff + 32, 0, 0);
    const uint32_t b67 = __builtin_amdgcn_raw_buffer_load_b32(bb, hoff + 36, 0, 0);
#pragma unroll
    for (int i = 0; i < QBW; ++i) {
      acc[i][0] = bf16_lo(b01); acc[i][1] = bf16_hi(b01);
      acc[i][2] = bf16_lo(b23); acc[i][3] = bf16_hi(b23);
      acc[i][4] = bf16_lo(b45); acc[i][5] = bf16_hi(b45);
      acc[i][6] = bf16_lo(b67); acc[i][7] = bf16_hi(b67);
    }
  }
#pragma unroll
  for (int yy = 0; yy < QBW + 4; ++yy) {  // halo rows ty0 + yy
#pragma unroll
    for (int j = 0; j < 3; ++j) {
      const uint32_t* hp = halo + ((ty0 + yy) * NPAIR + p0 + j) * 32;
      const uint4 h0 = *reinterpret_cast<const uint4*>(hp + 4 * grp);
      const uint4 h1 = *reinterpret_cast<const uint4*>(hp + 16 + 4 * grp);
#pragma unroll
      for (int i = 0; i < QBW; ++i) {
        const int ay = yy - i;  // compile-time after unrolling
        if (ay < 0 || ay >= 5) continue;
        const uint32_t* wp = w32 + (par * 15 + ay * 3 + j) * 32;
        const uint4 w0 = *reinterpret_cast<const uint4*>(wp + 4 * grp);
        const uint4 w1 = *reinterpret_cast<const uint4*>(wp + 16 + 4 * grp);
        acc[i][0] = dot2(h0.x, w0.x, acc[i][0]); acc[i][1] = dot2(h0.y, w0.y, acc[i][1]);
        acc[i][2] = dot2(h0.z, w0.z, acc[i][2]); acc[i][3] = dot2(h0.w, w0.w, acc[i][3]);
        acc[i][4] = dot2(h1.x, w1.x, acc[i][4]); acc[i][5] = dot2(h1.y, w1.y, acc[i][5]);
        acc[i][6] = dot2(h1.z, w1.z, acc[i][6]); acc[i][7] = dot2(h1.w, w1.w, acc[i][7]);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < QBW; ++i) {
    const int ty = ty0 + i;
    const float inv = 1.0f / ls[i][0];
    uint2 lo, hi;
    lo.x = float_to_bf16_bits(fmaf(o0[i][0], inv, acc[i][0])) | (float_to_bf16_bits(fmaf(o0[i][1], inv, acc[i][1])) << 16);
    lo.y = float_to_bf16_bits(fmaf(o0[i][2], inv, acc[i][2])) | (float_to_bf16_bits(fmaf(o0[i][3], inv, acc[i][3])) << 16);
    hi.x = float_to_bf16_bits(fmaf(o1[i][0], inv, acc[i][4])) | (float_to_bf16_bits(fmaf(o1[i][1], inv, acc[i][5])) << 16);
    hi.y = float_to_bf16_bits(fmaf(o1[i][2], inv, acc[i][6])) | (float_to_bf16_bits(fmaf(o1[i][3], inv, acc[i][7])) << 16);
    const Rsrc ob = rsrc(a.out + img, img_bytes);
    const uint32_t oo = (uint32_t)(((y0 + ty) * W + x0 + tx) * C + h * 32) * 2;
    st_nt(ob, oo + 8 * grp, lo);
    st_nt(ob, oo + 32 + 8 * grp, hi);
  }
}

template <int RH, int RW>
hipError_t launch_t(const TileArgs& a, hipStream_t st) {
  const int units = a.N * a.S * a.S * a.heads;
  const unsigned blocks = (unsigned)(((units + 7) / 8) * 8);
  constexpr int threads = 64 * tile_waves<RH, RW>();
  launch((attn_tile_kernel<RH, RW>), dim3(blocks), dim3(threads),
                     tile_lds(RH, RW).total, st, a);
  return hipGetLastError();
}

}  // namespace

bool tile_kernel_supports(const Shape& s) {
  if (s.hd != 32) return false;
  const int code = s.rh * 64 + s.rw;
  const bool compiled = code == 8 * 64 + 8 || code == 16 * 64 + 16 || code == 8 * 64 + 16 ||
                        code == 16 * 64 + 8;
  if (!compiled) return false;
  if ((long long)s.H * s.W * s.C >= (1ll << 30)) return false;  // 32-bit byte offsets in an image
  return tile_lds(s.rh, s.rw).total <= 65536;
}

hipError_t launch_attend_tile(const void* q, const void* k, const void* v, const uint32_t* wpk,
                              const void* b, const int32_t* route, const Shape& s, void* out,
                              hipStream_t st) {
  TileArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.wpk = wpk; a.b = (const uint16_t*)b; a.route = route; a.out = (uint16_t*)out;
  a.N = s.N; a.H = s.H; a.W = s.W; a.C = s.C; a.heads = s.heads; a.S = s.S; a.topk = s.topk;
  a.qscale = (float)(1.4426950408889634 / __builtin_sqrt((double)s.hd));
  switch (s.rh * 64 + s.rw) {
    case 8 * 64 + 8: return launch_t<8, 8>(a, st);
    case 16 * 64 + 16: return launch_t<16, 16>(a, st);
    case 8 * 64 + 16: return launch_t<8, 16>(a, st);
    case 16 * 64 + 8: return launch_t<16, 8>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bra
