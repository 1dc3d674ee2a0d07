// Routing pieces shared by the route kernels and the attention kernel that
// routes its own images: the 64-bit top-k key, the fp32 matrix-core logit
// tile and the rank selection. One definition, so every caller computes the
// same logits in the same order and picks the same routes, bit for bit.
#pragma once
#include "bra_internal.h"

namespace bra {
namespace route {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kChunk = 64;  // channels per load batch: 4 pieces of A and 4 of B per lane

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

// One 16 x 16 logit tile: rows r0.., columns 16ct.. of (Q^r K^r^T) * scale,
// lane (col, grp) returning rows 4grp..4grp+3 at column col. get(row, c)
// returns the 16-byte piece of channels c..c+3 of a Q^r (a) / K^r (b) row
// (rows clamped to R-1, pieces past C zero). The fp32 MFMA sequence is the
// same wherever the operands come from, so the logits are too.
// one 64-channel batch of the tile: lane (col, grp) holds channels
// 16j + 4grp .. +3 of its A and B rows in a[j], b[j]
__device__ __forceinline__ f32x4 logit_batch(f32x4 acc, const uint4* a, const uint4* b) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[j].x), __uint_as_float(b[j].x), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[j].y), __uint_as_float(b[j].y), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[j].z), __uint_as_float(b[j].z), acc, 0, 0, 0);
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[j].w), __uint_as_float(b[j].w), acc, 0, 0, 0);
  }
  return acc;
}

template <typename GetA, typename GetB>
__device__ __forceinline__ f32x4 logit_tile(int col, int grp, int C, GetA geta, GetB getb) {
  uint4 a[4], b[4], an[4], bn[4];
  auto fetch = [&](int c0, uint4* aa, uint4* bb) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = c0 + 16 * j + 4 * grp;
      aa[j] = geta(c);
      bb[j] = getb(c);
    }
  };
  // the next batch is always in flight while one is multiplied (the last
  // batch is peeled off, so no branch guards the loads)
  fetch(0, a, b);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  int c0 = 0;
  for (; c0 + kChunk < C; c0 += kChunk) {
    fetch(c0 + kChunk, an, bn);
    acc = logit_batch(acc, a, b);
#pragma unroll
    for (int j = 0; j < 4; ++j) { a[j] = an[j]; b[j] = bn[j]; }
  }
  return logit_batch(acc, a, b);
}

// The same tile in two steps, for a caller that must issue the operand loads
// early: all NB = ceil(C / 64) batches into registers, then the batches in
// logit_tile's order (so the logits are the same bit for bit).
template <int NB>
struct LogitOps {
  uint4 a[NB][4], b[NB][4];
};
template <int NB, typename GetA, typename GetB>
__device__ __forceinline__ void logit_load(LogitOps<NB>& o, int grp, GetA geta, GetB getb) {
#pragma unroll
  for (int k = 0; k < NB; ++k)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int c = kChunk * k + 16 * j + 4 * grp;
      o.a[k][j] = geta(c);
      o.b[k][j] = getb(c);
    }
}
template <int NB>
__device__ __forceinline__ f32x4 logit_mma(const LogitOps<NB>& o) {
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < NB; ++k) acc = logit_batch(acc, o.a[k], o.b[k]);
  return acc;
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
// One 16 x 16 tile with the operands in memory as fp32: lane (col, grp) of
// the tile holds row col of A and of B, channels k0 + 8 grp .. + 7 of each
// 32-channel step; get(c) returns the fp32 piece of channels c..c+3 of its A
// (geta) / B (getb) row (zero past C). Returns rows 4grp..4grp+3 at column
// col, as logit_tile.
template <typename GetA, typename GetB>
__device__ __forceinline__ f32x4 logit_tile_x3(int grp, int C, GetA geta, GetB getb) {
  // the operands of the next kAhead steps are in flight while a step's
  // products run (loads past C read nothing and are never used)
  constexpr int kAhead = 3;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  uint4 ra[kAhead][2], rb[kAhead][2];
#pragma unroll
  for (int d = 0; d < kAhead; ++d) {
    ra[d][0] = geta(32 * d + 8 * grp);
    ra[d][1] = geta(32 * d + 8 * grp + 4);
    rb[d][0] = getb(32 * d + 8 * grp);
    rb[d][1] = getb(32 * d + 8 * grp + 4);
  }
  for (int k0 = 0; k0 < C; k0 += 32 * kAhead) {
#pragma unroll
    for (int d = 0; d < kAhead; ++d) {
      const int k = k0 + 32 * d;
      const uint4 ca0 = ra[d][0], ca1 = ra[d][1], cb0 = rb[d][0], cb1 = rb[d][1];
      const int kn = k + 32 * kAhead;  // this slot's next step
      ra[d][0] = geta(kn + 8 * grp);
      ra[d][1] = geta(kn + 8 * grp + 4);
      rb[d][0] = getb(kn + 8 * grp);
      rb[d][1] = getb(kn + 8 * grp + 4);
      if (k < C) {
        const float fa[8] = {__uint_as_float(ca0.x), __uint_as_float(ca0.y), __uint_as_float(ca0.z), __uint_as_float(ca0.w),
                             __uint_as_float(ca1.x), __uint_as_float(ca1.y), __uint_as_float(ca1.z), __uint_as_float(ca1.w)};
        const float fb[8] = {__uint_as_float(cb0.x), __uint_as_float(cb0.y), __uint_as_float(cb0.z), __uint_as_float(cb0.w),
                             __uint_as_float(cb1.x), __uint_as_float(cb1.y), __uint_as_float(cb1.z), __uint_as_float(cb1.w)};
        rbf16x8 ah, al, bh, bl;
        split_bf16(fa, ah, al);
        split_bf16(fb, bh, bl);
        acc = logit_step_x3(acc, ah, al, bh, bl);
      }
    }
  }
  return acc;
}

// Top-k of rows i0, i0 + step, ... (four at a time) of the logit block
// logit[row][RP] (rows past nrows skipped): each lane ranks its candidate's
// key against all R others through kw (this wave's [4][64] key buffer) and
// the lanes of rank < topk hand their index to emit(row, rank, index).
template <typename Emit>
__device__ __forceinline__ void rank_rows(const float* logit, int RP, int R, int nrows, int i0,
                                          int step, int topk, uint64_t* kw, int lane, Emit emit) {
  const int s_rd = min(lane, R - 1);
  const int R2 = (R + 1) & ~1;
  for (; i0 < nrows; i0 += 4 * step) {
    uint64_t key[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + q * step;
      const bool ok = lane < R && i < nrows;
      key[q] = ok ? route_key(logit[min(i, nrows - 1) * RP + s_rd], lane) : 0ull;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();  // the previous group's reads of kw are done
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q = 0; q < 4; ++q) kw[q * 64 + lane] = key[q];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // every real key is nonzero and the keys past R are 0, so the pairs
    // may run over the padded row
    int rank[4] = {0, 0, 0, 0};
#pragma unroll 4
    for (int s2 = 0; s2 < R2; s2 += 2) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 two = *reinterpret_cast<const uint4*>(kw + q * 64 + s2);  // keys s2, s2+1
        const uint64_t k0 = ((uint64_t)two.y << 32) | two.x;
        const uint64_t k1 = ((uint64_t)two.w << 32) | two.z;
        rank[q] += (k0 > key[q]) + (k1 > key[q]);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int i = i0 + q * step;
      if (key[q] != 0ull && rank[q] < topk) emit(i, rank[q], lane);
    }
  }
}

// ---- one 16-row block of an image's routes (R <= 64) ----------------------
__host__ __device__ inline int col_tiles(int R) { return (R + 15) / 16; }
// The block's 16 query rows are staged in LDS once (row pitch C + 4 floats,
// so the 16 rows a tile column reads fall on different banks) where they fit:
// otherwise every wave would fetch all of them again from L2 for its column
// tile. The operand values, and so the logits, are the same either way.
constexpr int kRouteStageC = 512;
// LDS of route_block: the logit block [16][16 col_tiles], a [4][64] key
// buffer per wave, then (C <= kRouteStageC) the query rows [16][C + 4]
__host__ __device__ inline size_t route_block_lds(int R, int C, int waves) {
  return (size_t)16 * 16 * col_tiles(R) * sizeof(float) + (size_t)waves * 4 * 64 * sizeof(uint64_t) +
         (C <= kRouteStageC ? (size_t)16 * (C + 4) * sizeof(float) : 0);
}
// Routes of query rows r0 .. r0+15 (those below R) of image n, from the
// image's fp32 region means qr_img, kr_img ([R][C]), written to
// route_img[row][topk]. Wave w of `waves` computes column tiles w, w +
// waves, ... (split-bf16 matrix-core logits), the logits go to LDS, and the
// waves rank rows w, w + waves, ... Starts and ends with a workgroup
// barrier (the caller may reuse smem before and after).
__device__ __forceinline__ void route_block(const float* qr_img, const float* kr_img, int R, int C, int topk,
                                            float scale, int32_t* route_img, int r0, char* smem, int wave,
                                            int waves, int lane) {
  const int CT = col_tiles(R), RP = 16 * CT;  // padded logit row
  float* logit = reinterpret_cast<float*>(smem);                   // [16][RP]
  uint64_t* keys = reinterpret_cast<uint64_t*>(logit + 16 * RP);   // [waves][4][64]
  float* qrows = reinterpret_cast<float*>(keys + (size_t)waves * 4 * 64);  // [16][C + 4]
  const bool staged = C <= kRouteStageC;
  const int col = lane & 15, grp = lane >> 4;
  const uint32_t img_bytes = (uint32_t)R * C * 4;
  const Rsrc qb = rsrc(qr_img, img_bytes), kb = rsrc(kr_img, img_bytes);
  const uint32_t qrow = (uint32_t)min(r0 + col, R - 1) * C * 4;
  __syncthreads();
  if (staged) {
    const int cp = C / 4, pieces = 16 * cp;  // 16-byte pieces of the rows
    const int tid = wave * 64 + lane, nt = waves * 64;
    for (int e0 = tid; e0 < pieces; e0 += 4 * nt) {
      uint4 v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = e0 + i * nt, row = e / cp, c4 = e - row * cp;
        v[i] = ld16(qb, e < pieces ? (uint32_t)min(r0 + row, R - 1) * C * 4 + (uint32_t)c4 * 16 : kOut);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int e = e0 + i * nt, row = e / cp, c4 = e - row * cp;
        if (e < pieces) *reinterpret_cast<uint4*>(qrows + (size_t)row * (C + 4) + 4 * c4) = v[i];
      }
    }
    __syncthreads();
  }
  const float* qlds = qrows + (size_t)col * (C + 4);
  for (int ct = wave; ct < CT; ct += waves) {
    const uint32_t krow = (uint32_t)min(16 * ct + col, R - 1) * C * 4;
    const f32x4 acc = logit_tile_x3(
        grp, C,
        [&](int c) {
          if (staged) return c < C ? *reinterpret_cast<const uint4*>(qlds + c) : uint4{0u, 0u, 0u, 0u};
          return ld16(qb, c < C ? qrow + 4 * c : kOut);
        },
        [&](int c) { return ld16(kb, c < C ? krow + 4 * c : kOut); });
    // lane (col, grp) holds rows 4grp..4grp+3 of the tile at column col
#pragma unroll
    for (int e = 0; e < 4; ++e) logit[(4 * grp + e) * RP + 16 * ct + col] = acc[e] * scale;
  }
  __syncthreads();
  rank_rows(logit, RP, R, min(16, R - r0), wave, waves, topk, keys + (size_t)wave * 4 * 64, lane,
            [&](int i, int k, int s) { route_img[(size_t)(r0 + i) * topk + k] = s; });
  __syncthreads();
}

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
