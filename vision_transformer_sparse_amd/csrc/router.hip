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
//    fp32; see route_common.h). One workgroup of 16 waves per 16 query rows
//    of one image: all waves split the rows' and the image's K^r rows into
//    LDS (128 channels a phase, the next phase's loads in flight), one wave
//    per 16-column tile runs the products (lane (i, g) takes channels
//    k0+8g..+7 of row i of its A (Q^r) and B (K^r) operands, 32 channels a
//    step), the scaled logits go to LDS, and each wave ranks one row. The
//    attention kernels that route their own images use the same split and
//    the same product order.
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
// reads, one row per wave) and the lanes of rank < topk write
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
// One workgroup of kRouteWaves waves per 16 query rows of an image. The
// workgroup's 16 query rows (rows clamped to R-1) and the image's R
// candidate rows are split into hi/lo bf16 (as route::split_bf16) and written
// to LDS by all waves, kRoutePhase channels at a time, the next two phases'
// fp32 pieces already loaded into registers; wave ct < col_tiles(R) then runs
// candidate tile ct's split-bf16 chain over the phase's 32-channel steps in
// ascending order (route::logit_step_x3, the accumulator carried across the
// phases: the products and their order are route_region's, so the logits
// equal it bit for bit), and writes its scaled tile to LDS; wave i ranks
// query row i.
constexpr int kRouteWaves = 16;
constexpr int kRoutePhase = 128;                            // channels per phase
constexpr int kRoutePitch = 2 * kRoutePhase * 2 + 16;       // bytes of a split row: hi, lo, pad
constexpr int kRoutePieces = (16 + 64) * kRoutePhase / 4;   // 16-byte fp32 pieces of a phase, at most
constexpr int kRoutePer = (kRoutePieces + 64 * kRouteWaves - 1) / (64 * kRouteWaves);  // per thread

__host__ __device__ inline size_t route_lds(int R) {
  return (size_t)(16 + R) * kRoutePitch                       // split rows: query 0..15, candidates
         + (size_t)16 * 16 * col_tiles(R) * sizeof(float)     // logits [16][16 col_tiles]
         + (size_t)kRouteWaves * 64 * sizeof(uint64_t);       // a 64-key buffer per wave
}

__global__ __launch_bounds__(64 * kRouteWaves) void route_kernel(const float* __restrict__ qr,
                                                                 const float* __restrict__ kr, int R, int C,
                                                                 int topk, float scale,
                                                                 int32_t* __restrict__ route) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const int CT = col_tiles(R), RP = 16 * CT;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int u = xcd_unit(blockIdx.x, gridDim.x);
  const int n = u / CT;
  const int r0 = (u - n * CT) * 16;
  char* split = smem;                                                          // [16 + R][kRoutePitch]
  float* logit = reinterpret_cast<float*>(smem + (size_t)(16 + R) * kRoutePitch);  // [16][RP]
  uint64_t* kw = reinterpret_cast<uint64_t*>(logit + 16 * RP) + wave * 64;         // this wave's keys
  const uint32_t img_bytes = (uint32_t)R * C * 4;
  const Rsrc qb = rsrc(qr + (size_t)n * R * C, img_bytes), kb = rsrc(kr + (size_t)n * R * C, img_bytes);
  const int NR = 16 + R, QP = kRoutePhase / 4;  // rows, pieces of a row in a phase

  // piece e of phase p: row e / QP (query rows first), channels 4 (e % QP)..
  // The query rows are pieces 0 .. 16 QP - 1, whole waves of the first
  // batch, so each load reads one buffer across its wave.
  static_assert(16 * (kRoutePhase / 4) % 64 == 0 && 16 * (kRoutePhase / 4) <= 64 * kRouteWaves,
                "the query pieces are whole waves of the first batch");
  auto fetch = [&](int p, uint4* v) {
#pragma unroll
    for (int j = 0; j < kRoutePer; ++j) {
      const int e = tid + j * 64 * kRouteWaves, row = e / QP, c = p * kRoutePhase + 4 * (e - row * QP);
      const bool isq = j == 0 && wave < 16 * QP / 64;  // wave-uniform
      uint32_t off = kOut;
      if (c < C && row < NR)
        off = (uint32_t)((isq ? min(r0 + row, R - 1) : row - 16) * C + c) * 4;
      v[j] = ld16(isq ? qb : kb, off);
    }
  };
  auto put = [&](const uint4* v) {  // the fetched pieces as hi and lo bf16 (pieces past C are zeros)
#pragma unroll
    for (int j = 0; j < kRoutePer; ++j) {
      const int e = tid + j * 64 * kRouteWaves, row = e / QP, c4 = e - row * QP;
      if (row < NR) {
        const float x[4] = {__uint_as_float(v[j].x), __uint_as_float(v[j].y), __uint_as_float(v[j].z),
                            __uint_as_float(v[j].w)};
        __bf16 hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          hi[i] = (__bf16)x[i];
          lo[i] = (__bf16)(x[i] - (float)hi[i]);
        }
        char* d = split + (size_t)row * kRoutePitch + c4 * 8;
        *reinterpret_cast<uint2*>(d) = __builtin_bit_cast(uint2, hi);
        *reinterpret_cast<uint2*>(d + 2 * kRoutePhase) = __builtin_bit_cast(uint2, lo);
      }
    }
  };

  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const char* arow = split + (size_t)col * kRoutePitch + 16 * grp;
  const char* brow = split + (size_t)(16 + min(16 * wave + col, R - 1)) * kRoutePitch + 16 * grp;
  // phase p's pieces: put into LDS, the loads of phase p + 2 issued into the
  // same registers, then the phase's products (two phases' loads are in
  // flight from the start, so C <= 256 waits for memory once)
  auto phase = [&](int p, uint4* v) {
    __syncthreads();  // the previous phase's operands are read
    put(v);
    if ((p + 2) * kRoutePhase < C) fetch(p + 2, v);
    __syncthreads();
    if (wave < CT) {
      const int steps = min(kRoutePhase, C - p * kRoutePhase) / 32;
      for (int k = 0; k < steps; ++k) {
        const rbf16x8 ah = __builtin_bit_cast(rbf16x8, *reinterpret_cast<const uint4*>(arow + 64 * k));
        const rbf16x8 al = __builtin_bit_cast(rbf16x8, *reinterpret_cast<const uint4*>(arow + 64 * k + 2 * kRoutePhase));
        const rbf16x8 bh = __builtin_bit_cast(rbf16x8, *reinterpret_cast<const uint4*>(brow + 64 * k));
        const rbf16x8 bl = __builtin_bit_cast(rbf16x8, *reinterpret_cast<const uint4*>(brow + 64 * k + 2 * kRoutePhase));
        acc = logit_step_x3(acc, ah, al, bh, bl);
      }
    }
  };
  uint4 va[kRoutePer], vb[kRoutePer];
  fetch(0, va);
  if (kRoutePhase < C) fetch(1, vb);
  for (int p = 0; p * kRoutePhase < C; p += 2) {
    phase(p, va);
    if ((p + 1) * kRoutePhase < C) phase(p + 1, vb);
  }
  // lane (col, grp) of tile ct holds rows 4grp..4grp+3 at column col
  if (wave < CT) {
#pragma unroll
    for (int e = 0; e < 4; ++e) logit[(4 * grp + e) * RP + 16 * wave + col] = acc[e] * scale;
  }
  __syncthreads();
  // ---- wave i ranks query row r0 + i: lane s < R holds candidate s's key
  // and counts the keys above it (every real key is nonzero, the padded
  // ones are 0, so the pairs may run over the padding)
  const int i = wave;
  if (i < 16 && r0 + i < R) {
    const uint64_t key = lane < R ? route_key(logit[i * RP + lane], lane) : 0ull;
    kw[lane] = key;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    const int R2 = (R + 1) & ~1;
    int rank = 0;
#pragma unroll 4
    for (int s2 = 0; s2 < R2; s2 += 2) {
      const uint4 two = *reinterpret_cast<const uint4*>(kw + s2);
      rank += ((((uint64_t)two.y << 32) | two.x) > key) + ((((uint64_t)two.w << 32) | two.z) > key);
    }
    if (lane < R && rank < topk) route[((size_t)n * R + r0 + i) * topk + rank] = lane;
  }
}

hipError_t launch_small(const float* qr, const float* kr, int N, int R, int C, int topk,
                        int32_t* route, hipStream_t st) {
  const float scale = (float)(1.0 / __builtin_sqrt((double)C));
  const unsigned blocks = (unsigned)(N * col_tiles(R));
  launch(route_kernel, dim3(blocks), dim3(64 * kRouteWaves), route_lds(R), st, qr, kr, R, C, topk, scale, route);
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
