// Routing pieces shared by the route kernels and the attention kernels that
// route their own images: the 64-bit top-k key, the split-bf16 logit step
// and one region's routes. One definition, so every caller computes the
// same logits in the same order and picks the same routes, bit for bit.
#pragma once
#include "bra_internal.h"

namespace bra {
namespace route {

typedef float f32x4 __attribute__((ext_vector_type(4)));


// order-preserving map of a logit to unsigned (-0 and +0 are the same logit;
// every value maps above 0)
__device__ __forceinline__ uint32_t key_u32(float a) {
  if (a == 0.0f) a = 0.0f;
  const uint32_t u = __float_as_uint(a);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ uint64_t route_key(float a, int s) {
  return ((uint64_t)key_u32(a) << 32) | (uint32_t)(0xffffffffu - (uint32_t)s);
}
// A (key, index) pair as one double, exactly: key * 64 + (63 - index)
// (< 2^38, so every code is an integer a double holds exactly). Codes order
// as route_key orders the pairs -- larger key first, equal keys in index
// order -- for indices below 64, and every key above 0 codes above any
// index-only (key 0) code.
__device__ __forceinline__ double rank_code(uint32_t key, int idx) {
  return __builtin_fma((double)key, 64.0, (double)(63 - idx));
}
__device__ __forceinline__ int rank_code_index(double c) {
  return 63 - (int)__builtin_fma(-64.0, __builtin_floor(c * (1.0 / 64.0)), c);
}
// Sorting networks on codes (max and min only, no compare-and-select
// chains); codes of one row are distinct, so the order is exact.
__device__ __forceinline__ void code_ce(double& hi, double& lo) {  // larger to hi
  const double a = hi, b = lo;
  hi = __builtin_fmax(a, b);
  lo = __builtin_fmin(a, b);
}
__device__ __forceinline__ void sort4_code(double* c) {  // largest first
  code_ce(c[0], c[1]);
  code_ce(c[2], c[3]);
  code_ce(c[0], c[2]);
  code_ce(c[1], c[3]);
  code_ce(c[1], c[2]);
}
// the 4 largest of two lists sorted largest first, into a: the larger of
// a[i] and b[3 - i] holds them (in a V-shaped order), which a 4-element
// bitonic sorter puts in order
__device__ __forceinline__ void merge4_code(double* a, const double* b) {
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = __builtin_fmax(a[i], b[3 - i]);
  code_ce(a[0], a[2]);
  code_ce(a[1], a[3]);
  code_ce(a[0], a[1]);
  code_ce(a[2], a[3]);
}

// ---- split-bf16 logit tiles (R <= 64) --------------------------------------
// A logit Q^r_i . K^r_s in fp32 from bf16 matrix products: each fp32 operand
// is split as x = hi + lo (hi = bf16(x), lo = bf16(x - hi), both rounded to
// nearest even; the remainder is below 2^-16 |x|), and per 32-channel step
// the tile accumulates hi.lo + lo.hi + hi.hi (each bf16 product exact in the
// fp32 accumulator). The dropped lo.lo and remainder terms are ~2^-16 of the
// products, far inside the 1e-5 near-tie margin of the routing; the order is
// fixed, so every caller gets the same logits bit for bit.
typedef __bf16 rbf16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void split_bf16(const float* x, rbf16x8& hi, rbf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi[e] = (__bf16)x[e];
    lo[e] = (__bf16)(x[e] - (float)hi[e]);
  }
}
__device__ __forceinline__ f32x4 logit_step_x3(f32x4 acc, rbf16x8 ah, rbf16x8 al, rbf16x8 bh, rbf16x8 bl) {
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bl, acc, 0, 0, 0);
  acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(al, bh, acc, 0, 0, 0);
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(ah, bh, acc, 0, 0, 0);
}
// 16-wide candidate tiles of R regions (also the 16-row blocks of R <= 64)
__host__ __device__ inline int col_tiles(int R) { return (R + 15) / 16; }

// ---- one query region's routes inside an attention kernel (R <= 64) ------
// Region r's logits against every region of its image with route_kernel's
// split-bf16 steps in their order (an MFMA output element depends only on
// its row and column, so the logits equal route_kernel's bit for bit): wave
// w < col_tiles(R) computes candidates 16w .. 16w+15 (its tile's row 0 is
// region r) over channels cbase .. cbase + CR - 1 of the fp32 means [R][C]
// (CR % 32 == 0; the whole C, or one head's slice for per-head routing);
// then wave 0 ranks the R keys (larger logit first, ties to the lower
// index), and the region's top-k go to sel[rank] (LDS) and, when emit is
// true, to route_row[rank]. lrow (64 floats) and kw (64 keys, 16-byte
// aligned) are LDS scratch. Every wave of the workgroup calls it; it ends
// with a workgroup barrier (sel is then visible to all).
__device__ __forceinline__ void route_region(const float* qr_img, const float* kr_img, int R, int C, int cbase,
                                             int CR, float scale, int r, int topk, int wave, int lane,
                                             float* lrow, uint64_t* kw, int32_t* sel, bool emit,
                                             int32_t* route_row) {
  const int col = lane & 15, grp = lane >> 4;
  if (wave < col_tiles(R)) {
    const uint32_t mbytes = (uint32_t)R * C * 4;
    const Rsrc qm = rsrc(qr_img, mbytes), km = rsrc(kr_img, mbytes);
    const uint32_t qrow = (uint32_t)(r * C + cbase) * 4;
    const uint32_t krow = (uint32_t)(min(16 * wave + col, R - 1) * C + cbase) * 4;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    auto step = [&](const uint4& a0, const uint4& a1, const uint4& b0, const uint4& b1) {
      const float fa[8] = {__uint_as_float(a0.x), __uint_as_float(a0.y), __uint_as_float(a0.z), __uint_as_float(a0.w),
                           __uint_as_float(a1.x), __uint_as_float(a1.y), __uint_as_float(a1.z), __uint_as_float(a1.w)};
      const float fb[8] = {__uint_as_float(b0.x), __uint_as_float(b0.y), __uint_as_float(b0.z), __uint_as_float(b0.w),
                           __uint_as_float(b1.x), __uint_as_float(b1.y), __uint_as_float(b1.z), __uint_as_float(b1.w)};
      rbf16x8 ah, al, bh, bl;
      split_bf16(fa, ah, al);
      split_bf16(fb, bh, bl);
      acc = logit_step_x3(acc, ah, al, bh, bl);
    };
    // two steps' operands in flight at once
    for (int k0 = 0; k0 < CR; k0 += 64) {
      const uint32_t c = (uint32_t)(k0 + 8 * grp) * 4;
      const bool two = k0 + 32 < CR;
      const uint4 a0 = ld16(qm, qrow + c), a1 = ld16(qm, qrow + c + 16);
      const uint4 b0 = ld16(km, krow + c), b1 = ld16(km, krow + c + 16);
      const uint4 a2 = ld16(qm, two ? qrow + c + 128 : kOut), a3 = ld16(qm, two ? qrow + c + 144 : kOut);
      const uint4 b2 = ld16(km, two ? krow + c + 128 : kOut), b3 = ld16(km, two ? krow + c + 144 : kOut);
      step(a0, a1, b0, b1);
      if (two) step(a2, a3, b2, b3);
    }
    if (grp == 0) lrow[16 * wave + col] = acc[0] * scale;
  }
  __syncthreads();
  if (wave == 0) {
    const uint64_t key = lane < R ? route_key(lrow[lane], lane) : 0ull;
    kw[lane] = key;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    int rank = 0;  // keys are distinct; the 64 - R past R are 0
#pragma unroll
    for (int s2 = 0; s2 < 64; s2 += 2) {
      const uint4 two = *reinterpret_cast<const uint4*>(kw + s2);
      rank += (((uint64_t)two.y << 32 | two.x) > key) + (((uint64_t)two.w << 32 | two.z) > key);
    }
    if (lane < R && rank < topk) {
      sel[rank] = lane;
      if (emit) route_row[rank] = lane;
    }
  }
  __syncthreads();
}

}  // namespace route
}  // namespace bra
