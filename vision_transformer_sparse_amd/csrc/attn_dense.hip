// Router-free attention of the last stage: every query attends to all H*W
// tokens of its image, plus the 5x5 depthwise term on V. The walk-through's
// module print (TRANSFORMER.niftyadmin.cn/n/347023.html, section 网络结构)
// builds BiFormer's last stage from AttentionLePE blocks (qkv Linear, a
// depthwise 5x5 lepe Conv2d with padding 2, proj Linear), and
// bernice.tw/posts/biformer, section "Biformer", gives that stage k = S^2,
// i.e. every region routed: the routing step has nothing to choose, so this
// path skips it.
//
// Small maps (at most 256 tokens: 7x7 at 224 input, up to 16x16), bf16,
// head_dim 32. One workgroup owns one (image, head): it stages the head's K
// (one 64-byte row per token) and V (the same rows inside a 2-pixel zero
// border, which is the LePE padding) in LDS once, and its four waves walk the
// image's 16-query blocks:
//
//   S^T = K Q^T   16x16x32 bf16 products; A = 16 keys x 32 dims read from
//                 LDS, B = the block's queries straight from memory; lane
//                 (query j, group g) holds keys 16kt + 4g + i of tile kt
//   softmax       exact: the maximum over the lane's keys, then over the
//                 four groups (permlane swaps); exp2 of the scaled
//                 difference, rounded to bf16; the sum of the rounded values
//   O^T = V^T P^T within a 32-key step the lane's own eight probabilities
//                 (tiles 2s and 2s+1) form its B operand; the A operand is the
//                 same eight keys' values, read transposed from LDS
//                 (ds_read_b64_tr_b16), so both sides agree on the key order
//   LePE          before the attention, in its own pass: a lane owns one
//                 channel (its 25 weights and bias in registers) and a run of
//                 7 pixels of one output row; per window row it reads the 11
//                 values once and applies all five horizontal taps from
//                 registers (about 8 LDS reads an output instead of 25). The
//                 fp32 results wait in LDS for the attention epilogue.
//   store         attention / sum + LePE, one rounding to bf16; two
//                 cross-lane swaps give each lane 8 consecutive channels, so a
//                 token's 64 bytes leave in one instruction (non-temporal)
#include "bra_internal.h"

namespace bra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kDenseThreads = 256;
constexpr int kDenseWaves = kDenseThreads / 64;
constexpr int kDenseMaxTokens = 256;
constexpr int kDenseMaxBordered = 512;  // rows of the bordered V, (H+4)(W+4)
constexpr int kStage = 2;               // 16-byte pieces of K and of V a thread loads at once
constexpr int kSeg = 7;                 // output pixels of one row a lane convolves at once (one run covers a 7-wide map)
// A run of kSeg outputs starting at x0 <= W - 1 reads columns x0 ..
// x0 + kSeg + 3 of a bordered row of W + 4, so the last run of a row reads at
// most kSeg - 1 columns (64 bytes each) past the row's end: into the next row
// or, from the last row, past the bordered V, which this slack keeps inside
// the allocation. Those values feed only outputs past W, which are never read.
constexpr int kLceSlack = (kSeg - 1) * 64;

// LDS: [16 KT][32] bf16 keys | [(H+4)(W+4)][32] bf16 bordered values |
// [H][WP][32] fp32 LePE results (bias included; WP = W rounded up to whole
// runs of kSeg, so every run stores all its outputs) | [16 KT] key -> byte
// offset of its bordered value row
__host__ __device__ inline int lce_pitch(int W) { return (W + kSeg - 1) / kSeg * kSeg; }
struct DenseLds {
  int k, v, lce, rows, total;
};
__host__ __device__ inline DenseLds dense_lds(int H, int W, int KT) {
  DenseLds l;
  l.k = 0;
  l.v = 16 * KT * 64;
  l.lce = l.v + (H + 4) * (W + 4) * 64;
  l.rows = l.lce + H * lce_pitch(W) * 32 * 4;
  l.total = l.rows + 16 * KT * 4 + kLceSlack;
  return l;
}

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

// Up to 64 tokens (the 7x7 and 8x8 maps): eight workgroups a CU, so a
// batch of 128 images x 16 heads runs in one round.
template <int KT>
__global__ __launch_bounds__(kDenseThreads, KT <= 4 ? 8 : 1) void attn_dense_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ lw, const uint16_t* __restrict__ lb, int H, int W, int C, int heads,
    uint16_t* __restrict__ out) {
  extern __shared__ __attribute__((aligned(16))) char lds[];
  const DenseLds L = dense_lds(H, W, KT);
  const int u = xcd_unit(blockIdx.x, gridDim.x);  // an image's heads share an XCD (and its L2 lines)
  const int n = u / heads, h = u - n * heads;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, g = lane >> 4;
  const int HW = H * W, WB = W + 4, VB = (H + 4) * WB;
  const uint32_t rowb = (uint32_t)C * 2, hoff = (uint32_t)h * 64;
  const size_t img = (size_t)n * HW * C;
  const uint32_t img_bytes = (uint32_t)HW * rowb;
  const Rsrc qr = rsrc(q + img, img_bytes), kr = rsrc(k + img, img_bytes), vr = rsrc(v + img, img_bytes);
  const Rsrc orr = rsrc(out + img, img_bytes);
  const int QB = (HW + 15) / 16;

  // the first block's Q^T operand is in flight while K and V are staged
  auto q_operand = [&](int qb) {
    const int t = min(16 * qb + col, HW - 1);
    return ld16(qr, (uint32_t)t * rowb + hoff + 16 * g);
  };
  uint4 qv = q_operand(wave < QB ? wave : 0);
  // LePE weights and bias of this thread's channel (every LePE item of the
  // thread has channel tid % 32)
  const int lc = tid & 31;
  float wreg[25];
#pragma unroll
  for (int tap = 0; tap < 25; ++tap) wreg[tap] = bf16_bits_to_float(lw[(size_t)(h * 32 + lc) * 25 + tap]);
  // (a null bias is a zero-length buffer: its load reads 0, and no branch
  // waits on the loads already in flight)
  const Rsrc br = rsrc(lb, lb ? (uint32_t)C * 2 : 0u);
  const float bias_c = bf16_bits_to_float(__builtin_amdgcn_raw_buffer_load_b16(br, (h * 32 + lc) * 2, 0, 0));
  for (int key = tid; key < 16 * KT; key += kDenseThreads) {  // keys past HW point at a border row (zeros)
    const int y = key / W, x = key - (key / W) * W;
    reinterpret_cast<int*>(lds + L.rows)[key] = key < HW ? ((y + 2) * WB + x + 2) * 64 : 0;
  }
  // K rows (keys past HW stay unwritten: their scores are masked) and the
  // bordered V, in batches of kStage 16-byte pieces of each per thread
  const int kpieces = HW * 4, vpieces = VB * 4;
  for (int e0 = tid; e0 < kpieces || e0 < vpieces; e0 += kStage * kDenseThreads) {
    uint4 kx[kStage], vx[kStage];
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      const int e = e0 + i * kDenseThreads, t = e >> 2;
      kx[i] = ld16(kr, e < kpieces ? (uint32_t)t * rowb + hoff + 16 * (e & 3) : kOut);
      const int p = e >> 2, y = p / WB - 2, x = p - (p / WB) * WB - 2;
      const bool inside = e < vpieces && y >= 0 && y < H && x >= 0 && x < W;
      vx[i] = ld16(vr, inside ? (uint32_t)(y * W + x) * rowb + hoff + 16 * (e & 3) : kOut);  // border: zeros
    }
#pragma unroll
    for (int i = 0; i < kStage; ++i) {
      const int e = e0 + i * kDenseThreads;
      if (e < kpieces) *reinterpret_cast<uint4*>(lds + L.k + e * 16) = kx[i];
      if (e < vpieces) *reinterpret_cast<uint4*>(lds + L.v + e * 16) = vx[i];
    }
  }
  __syncthreads();

  // LePE(V) + bias of every pixel: items (channel, output row, run of kSeg
  // pixels), channel fastest
  float* lce = reinterpret_cast<float*>(lds + L.lce);
  const int segs = (W + kSeg - 1) / kSeg, items = 32 * H * segs, WP = segs * kSeg;
  for (int it = tid; it < items; it += kDenseThreads) {
    const int rs = it >> 5, y = rs / segs, x0 = (rs - y * segs) * kSeg;
    float acc[kSeg];
#pragma unroll
    for (int j = 0; j < kSeg; ++j) acc[j] = bias_c;
#pragma unroll
    for (int a = 0; a < 5; ++a) {
      // bordered row y + a holds image row y + a - 2; column x0 + j + e is
      // tap e of output x0 + j
      const char* rp = lds + L.v + ((y + a) * WB + x0) * 64 + 2 * lc;
      float vrow[kSeg + 4];
#pragma unroll
      for (int j = 0; j < kSeg + 4; ++j) vrow[j] = bf16_bits_to_float(*reinterpret_cast<const uint16_t*>(rp + j * 64));
#pragma unroll
      for (int e = 0; e < 5; ++e)
#pragma unroll
        for (int j = 0; j < kSeg; ++j) acc[j] = fmaf(wreg[5 * a + e], vrow[j + e], acc[j]);
      __builtin_amdgcn_sched_barrier(0);  // one window row's values live at a time
    }
#pragma unroll
    for (int j = 0; j < kSeg; ++j) lce[(y * WP + x0 + j) * 32 + lc] = acc[j];
  }
  __syncthreads();

  const float qscale = 0.17677669529663687f * 1.4426950408889634f;  // head_dim^-1/2, in log2 units
  const int* rows = reinterpret_cast<const int*>(lds + L.rows);
  for (int qb = wave; qb < QB; qb += kDenseWaves) {
    if (qb != wave) qv = q_operand(qb);
    const bf16x8 qb8 = __builtin_bit_cast(bf16x8, qv);
    f32x4 s[KT];
    float m = -__builtin_inff();
#pragma unroll
    for (int kt = 0; kt < KT; ++kt) {
      const bf16x8 ka = *reinterpret_cast<const bf16x8*>(lds + L.k + (16 * kt + col) * 64 + 16 * g);
      s[kt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka, qb8, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (16 * kt + 16 > HW && 16 * kt + 4 * g + i >= HW) s[kt][i] = -__builtin_inff();
        m = __builtin_elementwise_maximum(m, s[kt][i]);
      }
    }
    const float mq = group_max(m) * qscale;
    bf16x4 p[KT];
    float l = 0.f;
#pragma unroll
    for (int kt = 0; kt < KT; ++kt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        p[kt][i] = (__bf16)__builtin_amdgcn_exp2f(fmaf(s[kt][i], qscale, -mq));
        l += (float)p[kt][i];
      }
    l = group_sum(l);
    f32x4 o[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
    const int r = col >> 2, c = col & 3;  // this lane's row and piece of the transposing reads
#pragma unroll
    for (int j = 0; j < KT / 2; ++j) {
      const bf16x8 pb = cat(p[2 * j], p[2 * j + 1]);
      const char* v0 = lds + L.v + rows[32 * j + 4 * g + r] + 8 * c;
      const char* v1 = lds + L.v + rows[32 * j + 16 + 4 * g + r] + 8 * c;
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(cat(ld_tr(v0 + 32 * dt), ld_tr(v1 + 32 * dt)), pb, o[dt],
                                                        0, 0, 0);
    }
    // lane (query col, group g) holds channels 16 dt + 4g + i of its query
    const int t = 16 * qb + col, tc = min(t, HW - 1);
    const int y = tc / W, x = tc - y * W;
    const float inv = 1.f / l;
    uint32_t pk[2][2];  // [dt][pair]: channels 16 dt + 4g + (0, 1) and (2, 3), bf16
#pragma unroll
    for (int dt = 0; dt < 2; ++dt) {
      const f32x4 le = *reinterpret_cast<const f32x4*>(lce + (y * WP + x) * 32 + 16 * dt + 4 * g);
      float r[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) r[i] = fmaf(o[dt][i], inv, le[i]);
      pk[dt][0] = pack_bf16x2(r[0], r[1]);
      pk[dt][1] = pack_bf16x2(r[2], r[3]);
    }
    // Regroup so that lane group g holds channels 8g .. 8g+7 of its query (one
    // 16-byte store; the four groups write the token's 64 bytes in one
    // instruction): with A = the dt 0 quartets and B = the dt 1 quartets of
    // groups 0..3, the 32-lane swap gives X = (A0, A1, B0, B1), Y = (A2, A3,
    // B2, B3), and the 16-lane swap X = (A0, A2, B0, B2), Y = (A1, A3, B1, B3).
    uint32_t xs[2], ys[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const auto h32 = __builtin_amdgcn_permlane32_swap(pk[0][j], pk[1][j], false, false);
      const auto h16 = __builtin_amdgcn_permlane16_swap(h32[0], h32[1], false, false);
      xs[j] = h16[0];
      ys[j] = h16[1];
    }
    if (t < HW) {
      typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
      const u32x4 w4 = {xs[0], xs[1], ys[0], ys[1]};
      __builtin_amdgcn_raw_buffer_store_b128(w4, orr, (uint32_t)t * rowb + hoff + 16 * g, 0, kNt);
    }
  }
}

int dense_key_tiles(const Shape& s) { return 2 * ((s.H * s.W + 31) / 32); }

}  // namespace

bool dense_kernel_supports(const Shape& s) {
  const int HW = s.H * s.W;
  if (s.hd != 32 || HW > kDenseMaxTokens) return false;
  if ((s.H + 4) * (s.W + 4) > kDenseMaxBordered) return false;
  return dense_lds(s.H, s.W, dense_key_tiles(s)).total <= 64 * 1024;
}

hipError_t launch_attend_dense(const void* q, const void* k, const void* v, const void* w, const void* b,
                               const Shape& s, void* out, hipStream_t st) {
  const int KT = dense_key_tiles(s);
  const size_t lds = (size_t)dense_lds(s.H, s.W, KT).total;
  const dim3 grid((unsigned)(s.N * s.heads)), block(kDenseThreads);
#define BRA_DENSE(KTV)                                                                                   \
  launch(attn_dense_kernel<KTV>, grid, block, lds, st, (const uint16_t*)q, (const uint16_t*)k,       \
         (const uint16_t*)v, (const uint16_t*)w, (const uint16_t*)b, s.H, s.W, s.C, s.heads, (uint16_t*)out)
  switch (KT) {
    case 2: BRA_DENSE(2); break;
    case 4: BRA_DENSE(4); break;
    case 6: BRA_DENSE(6); break;
    case 8: BRA_DENSE(8); break;
    case 10: BRA_DENSE(10); break;
    case 12: BRA_DENSE(12); break;
    case 14: BRA_DENSE(14); break;
    case 16: BRA_DENSE(16); break;
    default: return hipErrorInvalidValue;
  }
#undef BRA_DENSE
  return hipGetLastError();
}

}  // namespace bra
