// Region-to-region routing: A = (Q^r * C^-1/2) K^r^T, an S^2 x S^2 affinity
// (Eq. 4), and per row the indices of the topk largest entries (Eq. 5) --
// TopkRouting.forward in the BRA walk-through at
// TRANSFORMER.niftyadmin.cn/n/347023.html, section BRA模块. The routing
// embedding is the identity; the softmax of the selected logits (routing
// weights) is not consumed by the gather and is not computed.
//
// Each shape is served by one kernel, in a fixed accumulation order, so its
// logits (and routes) are reproducible bit for bit:
//  * R <= 64 (route_kernel): affinities on the bf16 matrix cores with split
//    operands (x = hi + lo, products hi.lo + lo.hi + hi.hi accumulated in
//    fp32; see route_common.h). One workgroup per 16 query rows of one
//    image, one wave per 16-column tile. Lane (i, g) of a tile takes
//    channels k0+8g..+7 of row i of its A (Q^r) and B (K^r) operands -- the
//    same channels on both sides -- straight from memory with buffer loads
//    (pieces past C read as zero), 32 channels per step with the next step
//    in flight. The scaled logits go to LDS. The attention kernel for 4x4
//    regions routes its own images with the same tile code.
//  * R > 64 (route_wide_kernel): one workgroup per 4 query rows, one wave per
//    64 candidates; each lane streams its own candidate's K^r row from L2
//    into registers (double-buffered 32-channel batches) and reads the 4 Q^r
//    rows as LDS broadcasts; each logit is one fp32 fma chain in ascending
//    channel order. The 4 rows of logits go to LDS. (This spreads a few
//    large images over many more CUs than 16-row tiles would.)
// The workgroups of one image are numbered onto one XCD, so K^r comes from
// memory once per image and then from that XCD's L2.
//
// Top-k with an exact tie rule: every (A, s) becomes a 64-bit key whose
// unsigned order is "larger A first, then lower s first". With at most 64
// candidates each lane ranks its own key against all others (LDS broadcast
// reads, four rows interleaved per wave) and the lanes of rank < topk write
// their index at that rank. With more, topk rounds of a wave-wide maximum
// (DPP row reductions, then the last lane's value) emit the winners in
// descending order.
#include "bra_internal.h"
#include "route_common.h"

namespace bra {
namespace {

using namespace route;

// max of x and the DPP-moved copy of x (lanes the pattern leaves out keep x)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_step(uint64_t x) {
  const uint32_t lo = (uint32_t)x, hi = (uint32_t)(x >> 32);
  const uint32_t ylo = (uint32_t)__builtin_amdgcn_update_dpp((int)lo, (int)lo, CTRL, ROW_MASK, 0xf, false);
  const uint32_t yhi = (uint32_t)__builtin_amdgcn_update_dpp((int)hi, (int)hi, CTRL, ROW_MASK, 0xf, false);
  const uint64_t y = ((uint64_t)yhi << 32) | ylo;
  return y > x ? y : x;
}

// Maximum over the 64 lanes, returned wave-uniform: quad swaps, half-row and
// row mirrors (each row of 16 then holds its maximum), then row broadcasts
// 15 and 31 carry it into lane 63, which is read out.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t x) {
  x = dpp_max_step<0xb1, 0xf>(x);   // quad_perm [1,0,3,2]
  x = dpp_max_step<0x4e, 0xf>(x);   // quad_perm [2,3,0,1]
  x = dpp_max_step<0x141, 0xf>(x);  // row_half_mirror
  x = dpp_max_step<0x140, 0xf>(x);  // row_mirror
  x = dpp_max_step<0x142, 0xa>(x);  // row_bcast:15 into rows 1 and 3
  x = dpp_max_step<0x143, 0xc>(x);  // row_bcast:31 into rows 2 and 3
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)x, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(x >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// ---------------------------------------------------------------- R <= 64
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ qr,
                                                    const float* __restrict__ kr, int R, int C,
                                                    int topk, float scale,
                                                    int32_t* __restrict__ route) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int CT = col_tiles(R);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int u = xcd_unit(blockIdx.x, gridDim.x);
  const int n = u / CT;
  const int r0 = (u - n * CT) * 16;
  route_block(qr + (size_t)n * R * C, kr + (size_t)n * R * C, R, C, topk, scale, route + (size_t)n * R * topk,
              r0, smem, wave, blockDim.x >> 6, lane);
}

hipError_t launch_small(const float* qr, const float* kr, int N, int R, int C, int topk,
                        int32_t* route, hipStream_t st) {
  const float scale = (float)(1.0 / __builtin_sqrt((double)C));
  const unsigned blocks = (unsigned)(N * col_tiles(R));
  launch(route_kernel, dim3(blocks), dim3(64 * col_tiles(R)), route_block_lds(R, C, col_tiles(R)), st, qr, kr, R, C,
         topk, scale, route);
  return hipGetLastError();
}

// ---------------------------------------------------------------- R > 64
constexpr int kWideRows = 4;   // query rows per workgroup
constexpr int kWideBatch = 8;  // 16-byte loads per lane per batch (32 channels)

template <int MPL>
__global__ __launch_bounds__(64 * MPL) void route_wide_kernel(
    const float* __restrict__ qr, const float* __restrict__ kr, int R, int C, int topk,
    float scale, int32_t* __restrict__ route) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  float* qs = reinterpret_cast<float*>(smem);  // [4][C]
  float* logit = qs + kWideRows * C;           // [4][64 * MPL]
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int blocks_per_img = (R + kWideRows - 1) / kWideRows;
  const int u = xcd_unit(blockIdx.x, gridDim.x);
  const int n = u / blocks_per_img;
  const int r0 = (u - n * blocks_per_img) * kWideRows;
  const float* krn = kr + (size_t)n * R * C;
  const float* qrn = qr + (size_t)n * R * C;

  // candidate s's first batch, then the Q^r rows r0..r0+3 (clamped) into LDS
  const int s = 64 * wave + lane;
  const float* krow = krn + (size_t)min(s, R - 1) * C;
  float4 cur[kWideBatch], nxt[kWideBatch];
#pragma unroll
  for (int b = 0; b < kWideBatch; ++b) cur[b] = *reinterpret_cast<const float4*>(krow + 4 * b);
  for (int e = tid; e < kWideRows * C / 4; e += 64 * MPL) {
    const int rr = e / (C / 4), j = e - rr * (C / 4);
    *reinterpret_cast<float4*>(qs + rr * C + 4 * j) =
        *reinterpret_cast<const float4*>(qrn + (size_t)min(r0 + rr, R - 1) * C + 4 * j);
  }
  __syncthreads();

  float acc[kWideRows];
#pragma unroll
  for (int i = 0; i < kWideRows; ++i) acc[i] = 0.f;
  for (int c0 = 0; c0 < C; c0 += 4 * kWideBatch) {
    const int cn = min(c0 + 4 * kWideBatch, C - 4 * kWideBatch);  // the last batch reloads itself
#pragma unroll
    for (int b = 0; b < kWideBatch; ++b) nxt[b] = *reinterpret_cast<const float4*>(krow + cn + 4 * b);
#pragma unroll
    for (int b = 0; b < kWideBatch; ++b) {
#pragma unroll
      for (int i = 0; i < kWideRows; ++i) {
        const float4 qv = *reinterpret_cast<const float4*>(qs + i * C + c0 + 4 * b);
        acc[i] = fmaf(qv.x, cur[b].x, acc[i]);
        acc[i] = fmaf(qv.y, cur[b].y, acc[i]);
        acc[i] = fmaf(qv.z, cur[b].z, acc[i]);
        acc[i] = fmaf(qv.w, cur[b].w, acc[i]);
      }
    }
#pragma unroll
    for (int b = 0; b < kWideBatch; ++b) cur[b] = nxt[b];
  }
#pragma unroll
  for (int i = 0; i < kWideRows; ++i) logit[i * 64 * MPL + s] = acc[i] * scale;
  __syncthreads();

  // rows wave, wave + MPL, ... (no barrier follows)
  for (int i = wave; i < kWideRows && r0 + i < R; i += MPL) {
    const float* lrow = logit + i * 64 * MPL;
    uint64_t key[MPL];
#pragma unroll
    for (int m = 0; m < MPL; ++m) {
      const int sm = lane + 64 * m;
      key[m] = sm < R ? route_key(lrow[sm], sm) : 0ull;
    }
    int32_t* out = route + ((size_t)n * R + r0 + i) * topk;
    for (int p = 0; p < topk; ++p) {
      uint64_t best = 0ull;
#pragma unroll
      for (int m = 0; m < MPL; ++m) best = key[m] > best ? key[m] : best;
      best = wave_max_u64(best);
      const int win = (int)(0xffffffffu - (uint32_t)(best & 0xffffffffu));
#pragma unroll
      for (int m = 0; m < MPL; ++m)
        if (lane + 64 * m == win) key[m] = 0ull;
      if (lane == 0) out[p] = win;
    }
  }
}

template <int MPL>
hipError_t launch_wide(const float* qr, const float* kr, int N, int R, int C, int topk,
                       int32_t* route, hipStream_t st) {
  const float scale = (float)(1.0 / __builtin_sqrt((double)C));
  const unsigned blocks = (unsigned)(N * ((R + kWideRows - 1) / kWideRows));
  const size_t lds = ((size_t)kWideRows * C + (size_t)kWideRows * 64 * MPL) * sizeof(float);
  launch((route_wide_kernel<MPL>), dim3(blocks), dim3(64 * MPL), lds, st, qr, kr, R,
                     C, topk, scale, route);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* qr, const float* kr, int N, int R, int C, int topk,
                        int32_t* route, hipStream_t st) {
  if (R <= 64) return launch_small(qr, kr, N, R, C, topk, route, st);
  if (R <= 128) return launch_wide<2>(qr, kr, N, R, C, topk, route, st);
  if (R <= 256) return launch_wide<4>(qr, kr, N, R, C, topk, route, st);
  if (R <= 512) return launch_wide<8>(qr, kr, N, R, C, topk, route, st);
  return launch_wide<16>(qr, kr, N, R, C, topk, route, st);
}

}  // namespace bra
