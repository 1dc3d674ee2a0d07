// Internal declarations shared by the host library and the kernel files.
// Not part of the public ABI (include/bra.h is).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bra {

// Timing of the next kernel launched on this host thread: when the library
// profiles a kernel kind it leaves a pair of events here; launch() hands them
// to hipExtLaunchKernelGGL, which stamps them with that dispatch's own start
// and end, and clears them.
struct ProfEvents {
  hipEvent_t start = nullptr, stop = nullptr;
};
ProfEvents& prof_events();  // per host thread

// Compute units of the current device (cached per device).
int device_cu_count();

// Every kernel of the library is launched through here. Errors are left for
// the caller's hipGetLastError().
template <typename... Args, typename F = void (*)(Args...)>
void launch(F kernel, dim3 grid, dim3 block, size_t lds, hipStream_t st, Args... args) {
  ProfEvents& pe = prof_events();
  if (pe.start) {
    const hipEvent_t a = pe.start, b = pe.stop;
    pe.start = pe.stop = nullptr;
    hipExtLaunchKernelGGL(kernel, grid, block, (uint32_t)lds, st, a, b, 0u, args...);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, lds, st, args...);
  }
}

// Problem sizes, derived once on the host after validation.
struct Shape {
  int N, H, W, C, heads, S, topk;
  int R;       // S*S regions
  int rh, rw;  // region height / width in tokens
  int T;       // tokens per region
  int hd;      // head dim (C / heads)
  int L;       // gathered keys per query region (topk * T)
};

constexpr int kHeadDim = 32;     // compiled head dimension

// Division by a fixed d in [1, 2^16) of any n in [0, 2^16) with one
// multiply-high: with m = ceil(2^32 / d) = (2^32 + e) / d, e < d,
// n * m / 2^32 = n / d + n e / (d 2^32), and the second term is below 1/d,
// which the fractional part of n / d never comes within, so the floor is
// exact. m is made on the host (d = 1 keeps m = 0 and divides by identity).
struct FastDiv {
  uint32_t d, m;
};
inline FastDiv make_fastdiv(uint32_t d) {
  return FastDiv{d, d <= 1 ? 0u : (uint32_t)((0x100000000ull + d - 1) / d)};
}
#if defined(__HIPCC__)
__device__ __forceinline__ uint32_t fdiv(const FastDiv& f, uint32_t n) {
  return f.m ? __umulhi(n, f.m) : n;
}
#endif
constexpr int kMaxRegions = 1024;

// Region means; for bf16 (wpk non-null) also repacks the LCE weights for the
// attention kernels, and (kn non-null) writes the largest squared key norm
// per (image, region, head) to kn [N][S*S][C/32].
hipError_t launch_region_pool(const void* q, const void* k, const Shape& s,
                              int dtype, float* qr, float* kr, const void* lce_w,
                              uint32_t* wpk, float* kn, hipStream_t st);
hipError_t launch_route(const float* qr, const float* kr, int N, int R, int C,
                        int topk, int32_t* route, hipStream_t st);
hipError_t launch_attend(const void* q, const void* k, const void* v,
                         const void* w, const void* b, const int32_t* route,
                         const Shape& s, int dtype, void* out, hipStream_t st);
hipError_t launch_lce(const void* v, const void* w, const void* b,
                      const Shape& s, int dtype, float* out, hipStream_t st);
hipError_t launch_copy(const void* src, void* dst, size_t bytes, hipStream_t st);

// Device helpers ------------------------------------------------------------
#if defined(__HIPCC__)
__device__ __forceinline__ float bf16_bits_to_float(uint32_t bits16) {
  return __uint_as_float(bits16 << 16);
}
// Low / high bf16 of a 32-bit word, as float.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Raw buffer access: a uniform base in SGPRs, a 32-bit byte offset per lane;
// offsets at or past `bytes` read as zero.
typedef __amdgpu_buffer_rsrc_t Rsrc;
constexpr uint32_t kOut = 0x80000000u;  // an offset past every buffer this library builds
__device__ __forceinline__ Rsrc rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ uint4 ld16(Rsrc r, uint32_t off) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}
// the same with a uniform (scalar) offset added to the lane's
__device__ __forceinline__ uint4 ld16s(Rsrc r, uint32_t off, uint32_t soff) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, soff, 0);
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Streaming (non-temporal) stores for outputs that nothing in the kernel
// reads back: they leave without staying dirty in L2, which the end of the
// kernel would otherwise have to write back. (Buffer stores carry the
// cache policy as an operand; a plain store's hint can be lost when the
// compiler merges stores.)
constexpr int kNt = 2;  // cache-policy bit: non-temporal
__device__ __forceinline__ void st_nt(Rsrc r, uint32_t off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, off, 0, kNt);
}
__device__ __forceinline__ void st_nt(Rsrc r, uint32_t off, uint2 v) {
  typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
  u32x2 x;
  x[0] = v.x;
  x[1] = v.y;
  __builtin_amdgcn_raw_buffer_store_b64(x, r, off, 0, kNt);
}

// Workgroup b -> logical unit u such that consecutive units share b % 8,
// the XCD that dispatch sends workgroup b to. Bijective on [0, blocks).
__device__ __forceinline__ int xcd_unit(int b, int blocks) {
  const int per = blocks / 8, rem = blocks % 8, x = b % 8;
  return x * per + min(x, rem) + b / 8;
}

// float -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}
// Two floats rounded to nearest even into one packed bf16 pair (lo in bits
// 0..15) by the hardware conversion (one v_cvt_pk_bf16_f32); for finite
// values the same bits as float_to_bf16_bits, a NaN stays a NaN.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float max3(float a, float b, float c) {
  return __builtin_elementwise_maximum(__builtin_elementwise_maximum(a, b), c);
}
// maximum over the lanes l, l^16, l^32, l^48 (the four key groups of a query)
__device__ __forceinline__ float group_max(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);  // {x[l & ~16], x[l | 16]}
  x = __builtin_elementwise_maximum(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const uint32_t w = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);  // {x[l & 31], x[l | 32]}
  return __builtin_elementwise_maximum(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// sum over the lanes l, l^16, l^32, l^48
__device__ __forceinline__ float group_sum(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto a = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const uint32_t w = __float_as_uint(x);
  const auto b = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
// max of x and its DPP-moved copy (lanes the pattern leaves out keep x)
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_max(float x) {
  const int y = __builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, ROW_MASK, 0xf, false);
  return __builtin_elementwise_maximum(x, __int_as_float(y));
}
// x of another lane by a DPP pattern (every lane of the pattern is valid)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// sum over the four lanes of a quad (quad_perm swaps [1,0,3,2], [2,3,0,1])
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0xb1, 0xf, 0xf, false));
  return x + __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x4e, 0xf, 0xf, false));
}
// maximum / sum over the lanes of a 16-lane row that share l % P (P a power
// of two dividing 16): DPP row rotations by P, 2P, .. 8
template <int P>
__device__ __forceinline__ float row_class_max(float x) {
  if constexpr (P < 16) {
    x = dpp_max<0x120 + P, 0xf>(x);  // row_ror:P
    return row_class_max<2 * P>(x);
  }
  return x;
}
template <int P>
__device__ __forceinline__ float row_class_sum(float x) {
  if constexpr (P < 16) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), 0x120 + P, 0xf, 0xf, false));
    return row_class_sum<2 * P>(x);
  }
  return x;
}

// The LCE weights repacked for packed-bf16 dot products, two layouts in one
// buffer of lce_pack_items(C) entries:
//  * [parity][row][pair][C] dwords (30*C): pixel-pair weights. For an even
//    output column the pixel pairs start at tap 0 ((w0,w1),(w2,w3),(w4,0));
//    for an odd one a pixel earlier ((0,w0),(w1,w2),(w3,w4)). Entry e < 15*C
//    (row*3+pair major, C minor) writes one dword of each parity.
//  * then [tap][C/2] dwords (25*C/2): the weights of channels 2p and 2p+1
//    for tap t (= 5*row + column) in one dword (low half: channel 2p).
//  * then, per head of 32 channels, the 5x5 weights as Toeplitz blocks of a
//    4x4x4 product (2560 dwords a head, 80*C in all): bf16 entry
//    [h][dy][ch][b][j][k] (h, ch < 2; dy < 5; b < 16; j, k < 4) is
//    w_c[dy][4 ch + k - j] for channel c = 2b + h of the head, zero where that
//    tap index leaves 0..4. Block b, chunk ch multiplies four bordered pixels
//    4ch..4ch+3 of a window row into output columns j = 0..3.
constexpr int kLceToepDwords = 2560;  // per head (32 channels)
__host__ __device__ inline int lce_toep_offset(int C) { return 30 * C + 25 * (C / 2); }
__host__ __device__ inline int lce_pack_items(int C) { return 15 * C + 25 * (C / 2) + C / 32 * kLceToepDwords; }
__device__ __forceinline__ uint32_t lce_toep_entry(const uint16_t* __restrict__ lw, int c, int dy, int tap) {
  return tap >= 0 && tap < 5 ? (uint32_t)lw[(size_t)c * 25 + dy * 5 + tap] : 0u;
}
// dword e (< kLceToepDwords) of one head's Toeplitz blocks, from that head's
// 32 channels of 5x5 weights (global memory or LDS)
__device__ __forceinline__ uint32_t lce_toep_dword(const uint16_t* __restrict__ lw_head, int e) {
  const int f = 2 * e;  // bf16 index, even
  const int k = f & 3, j = (f >> 2) & 3, b = (f >> 4) & 15, ch = (f >> 8) & 1;
  const int dy = (f >> 9) % 5, h = (f >> 9) / 5;
  const int c = 2 * b + h, tap = 4 * ch + k - j;
  return lce_toep_entry(lw_head, c, dy, tap) | (lce_toep_entry(lw_head, c, dy, tap + 1) << 16);
}
__device__ __forceinline__ void pack_lce_item(const uint16_t* __restrict__ lw, int C, int e,
                                              uint32_t* __restrict__ wpk) {
  if (e < 15 * C) {
    const int c = e % C, rest = e / C;
    const int ay = rest / 3, d0 = 2 * (rest % 3);
    const uint16_t* wr = lw + (size_t)c * 25 + ay * 5;
    const uint32_t t0 = wr[d0];
    const uint32_t t1 = d0 + 1 < 5 ? (uint32_t)wr[d0 + 1] : 0u;
    const uint32_t tm = d0 > 0 ? (uint32_t)wr[d0 - 1] : 0u;
    wpk[rest * C + c] = t0 | (t1 << 16);
    wpk[(15 + rest) * C + c] = tm | (t0 << 16);
  } else if (e < 15 * C + 25 * (C / 2)) {
    const int e2 = e - 15 * C;
    const int t = e2 / (C / 2), p = e2 - t * (C / 2);
    wpk[30 * C + e2] = (uint32_t)lw[(size_t)(2 * p) * 25 + t] | ((uint32_t)lw[(size_t)(2 * p + 1) * 25 + t] << 16);
  } else {
    const int e3 = e - 15 * C - 25 * (C / 2);  // dword of the Toeplitz section
    const int head = e3 / kLceToepDwords;
    wpk[lce_toep_offset(C) + e3] = lce_toep_dword(lw + (size_t)head * 32 * 25, e3 - head * kLceToepDwords);
  }
}

template <typename T> struct Elem;
template <> struct Elem<float> {
  __device__ static float load(const float* p, size_t i) { return p[i]; }
  __device__ static void store(float* p, size_t i, float x) { p[i] = x; }
};
template <> struct Elem<uint16_t> {  // bf16 storage
  __device__ static float load(const uint16_t* p, size_t i) { return bf16_bits_to_float(p[i]); }
  __device__ static void store(uint16_t* p, size_t i, float x) { p[i] = (uint16_t)float_to_bf16_bits(x); }
};
#endif

}  // namespace bra
