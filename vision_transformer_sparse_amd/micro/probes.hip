// Throughput probes of the gfx950 units the attention kernels lean on:
// v_exp_f32 (the softmax's exponential), plain fp32 fma, the bf16 matrix
// cores (v_mfma_f32_16x16x32_bf16), the three mixed with one another (do
// they run side by side on one SIMD?), and HBM read / write / copy
// bandwidth. Built with the library's flags into libbra_micro.so; no part of
// the BRA forward pass uses it.
//
// Every probe kernel writes one value per lane to `out` (so nothing is
// optimised away) and, from lane 0 of each workgroup, a start and end stamp
// of the shader clock (s_memtime) and of the constant-rate wall clock
// (s_memrealtime), from which the host derives the clock the probe ran at.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void stamp(uint64_t* st, int which) {
  if (threadIdx.x == 0) {
    st[(size_t)blockIdx.x * 4 + 2 * which] = __builtin_readcyclecounter();
    st[(size_t)blockIdx.x * 4 + 2 * which + 1] = __builtin_amdgcn_s_memrealtime();
  }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// kind bits: 1 = exp chains, 2 = fma chains, 4 = mfma chains, 8 = the
// mfma chains use v_mfma_f32_32x32x16_bf16 (twice the flops of one
// 16x16x32 instruction)
template <int KIND, int NEXP, int NFMA, int NMFMA>
__global__ __launch_bounds__(256) void unit_kernel(float* out, int iters, uint64_t* st) {
  const int gid = blockIdx.x * blockDim.x + threadIdx.x;
  const float base = 0.25f + (threadIdx.x & 63) * 1e-3f;
  float e[NEXP > 0 ? NEXP : 1], f[NFMA > 0 ? NFMA : 1];
#pragma unroll
  for (int i = 0; i < NEXP; ++i) e[i] = base + 0.01f * i;
#pragma unroll
  for (int i = 0; i < NFMA; ++i) f[i] = base - 0.01f * i;
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(base * 0.001f * (i + 1));
    b[i] = (__bf16)(base * 0.002f * (i + 1));
  }
  f32x4 acc[NMFMA > 0 ? NMFMA : 1];
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x16 acc32[NMFMA > 0 ? NMFMA : 1];
#pragma unroll
  for (int i = 0; i < NMFMA; ++i)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc32[i][e] = 0.f;
  __syncthreads();
  stamp(st, 0);
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      if constexpr ((KIND & 12) == 4) {
#pragma unroll
        for (int i = 0; i < NMFMA; ++i) acc[i] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[i], 0, 0, 0);
      }
      if constexpr ((KIND & 12) == 12) {
#pragma unroll
        for (int i = 0; i < NMFMA; ++i) acc32[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc32[i], 0, 0, 0);
      }
      if constexpr ((KIND & 1) != 0) {
        // x <- 2^-x converges to about 0.64: the inputs stay ordinary numbers
#pragma unroll
        for (int i = 0; i < NEXP; ++i) e[i] = __builtin_amdgcn_exp2f(-e[i]);
      }
      if constexpr ((KIND & 2) != 0) {
#pragma unroll
        for (int i = 0; i < NFMA; ++i) f[i] = __builtin_fmaf(f[i], 0.999f, 0.0005f);
      }
    }
  }
  stamp(st, 1);
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < NEXP; ++i) s += e[i];
#pragma unroll
  for (int i = 0; i < NFMA; ++i) s += f[i];
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) s += acc[i][0] + acc[i][1] + acc[i][2] + acc[i][3];
#pragma unroll
  for (int i = 0; i < NMFMA; ++i) s += acc32[i][0] + acc32[i][15];
  out[gid] = s;
}

// HBM: read (sum of 16-byte pieces), write (fill), copy; grid-stride loops
__global__ __launch_bounds__(256) void read_kernel(const u32x4* __restrict__ src, size_t n16, float* out) {
  uint32_t acc = 0;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    const u32x4 v = __builtin_nontemporal_load(src + i);
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == 0x9e3779b9u) out[0] = 1.f;  // keeps the loads; practically never taken
}
__global__ __launch_bounds__(256) void write_kernel(u32x4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  const u32x4 v = {threadIdx.x, 1u, 2u, 3u};
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(v, dst + i);
}
__global__ __launch_bounds__(256) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    __builtin_nontemporal_store(__builtin_nontemporal_load(src + i), dst + i);
}

// LDS read patterns of the attention kernels' operand loads, 64 lanes per
// instruction, eight independent reads per step:
//  0  ds_read_b128, lanes read 1 KiB contiguously (the reference)
//  1  ds_read_b128, 16 rows x one 16-byte chunk per 16 lanes, rows of 64
//     bytes with the chunk XOR-swizzled by the row (the K-operand read)
//  2  the same rows without the swizzle
//  3  the same rows at an 80-byte pitch (padding instead of a swizzle)
//  4  ds_read_b64_tr_b16, 4 rows x 16 channels per 16 lanes, swizzled rows
//     (the V^T-operand read)
//  5  the same without the swizzle
//  6  the same at an 80-byte pitch
//  7  ds_read_b64_tr_b16, the 16 lanes of a group read one contiguous 128
//     bytes (4 rows x 32 bytes) and the four groups contiguous blocks
template <int PAT>
__global__ __launch_bounds__(256) void lds_kernel(float* out, int iters, uint64_t* st) {
  __shared__ __attribute__((aligned(16))) unsigned char buf[16384];
  for (int i = threadIdx.x; i < 16384 / 4; i += blockDim.x) reinterpret_cast<unsigned*>(buf)[i] = i * 2654435761u;
  __syncthreads();
  const int lane = threadIdx.x & 63, col = lane & 15, grp = lane >> 4;
  auto swz = [](int r) { const int g = (r >> 3) & 3; return ((g & 1) << 1) | (g >> 1); };
  int off;
  if (PAT == 0) {
    off = lane * 16;
  } else if (PAT <= 3) {
    const int row = 8 * (col >> 2) + (col & 3);
    off = PAT == 1 ? row * 64 + ((grp ^ swz(row)) << 4) : PAT == 2 ? row * 64 + grp * 16 : row * 80 + grp * 16;
  } else {
    const int row = 8 * grp + (col >> 2), chn = 4 * (col & 3);
    off = PAT == 4 ? row * 64 + (((chn >> 3) ^ swz(row)) << 4) + (chn & 7) * 2
        : PAT == 5 ? row * 64 + chn * 2 : PAT == 6 ? row * 80 + chn * 2
        : grp * 128 + (col >> 2) * 32 + (col & 3) * 8;
  }
  u32x4 acc = {0u, 0u, 0u, 0u};
  __syncthreads();
  stamp(st, 0);
  for (int it = 0; it < iters; ++it) {
    // the LDS may have changed for all the compiler knows: every read is
    // issued again in every iteration
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      // eight distinct places 1280 bytes (5 x 256) apart, shifted by 32
      // bytes every other step: the same banks for every read
      const int o = off + j * 1280 + (it & 1) * 32;
      if constexpr (PAT <= 3) {
        acc += *reinterpret_cast<const u32x4*>(buf + o);
      } else {
        typedef short s16x4 __attribute__((ext_vector_type(4)));
        const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (__attribute__((address_space(3))) s16x4*)(buf + o));
        acc[j & 3] += (unsigned)v[0] + ((unsigned)v[3] << 16);
      }
    }
  }
  stamp(st, 1);
  out[blockIdx.x * blockDim.x + threadIdx.x] = (float)(acc[0] + acc[1] + acc[2] + acc[3]);
}

thread_local char g_err[256];

int fail(const char* what, hipError_t e) {
  snprintf(g_err, sizeof g_err, "%s: %s", what, hipGetErrorString(e));
  return -1;
}

#define CK(x)                          \
  do {                                 \
    hipError_t e_ = (x);               \
    if (e_ != hipSuccess) return fail(#x, e_); \
  } while (0)

typedef void (*UnitFn)(float*, int, uint64_t*);

UnitFn unit_fn(int probe) {
  switch (probe) {
    case 0: return unit_kernel<1, 8, 0, 0>;    // exp, 8 chains
    case 1: return unit_kernel<2, 0, 8, 0>;    // fma, 8 chains
    case 2: return unit_kernel<4, 0, 0, 4>;    // mfma, 4 chains
    case 3: return unit_kernel<3, 8, 8, 0>;    // exp + fma (8 + 8 per step)
    case 4: return unit_kernel<5, 4, 0, 4>;    // mfma + exp (4 + 4 per step)
    case 5: return unit_kernel<5, 8, 0, 4>;    // mfma + exp (4 + 8)
    case 6: return unit_kernel<7, 8, 8, 4>;    // mfma + exp + fma (4 + 8 + 8)
    case 7: return unit_kernel<6, 0, 8, 4>;    // mfma + fma (4 + 8)
    case 8: return unit_kernel<12, 0, 0, 2>;   // mfma 32x32x16, 2 chains
    case 9: return unit_kernel<13, 8, 0, 2>;   // mfma 32x32x16 + exp (2 + 8)
    case 18: return unit_kernel<15, 8, 8, 2>;  // mfma 32x32x16 + exp + fma (2 + 8 + 8)
    case 19: return unit_kernel<13, 16, 0, 4>; // mfma 32x32x16 + exp (4 + 16)
    case 10: return lds_kernel<0>;
    case 11: return lds_kernel<1>;
    case 12: return lds_kernel<2>;
    case 13: return lds_kernel<3>;
    case 14: return lds_kernel<4>;
    case 15: return lds_kernel<5>;
    case 16: return lds_kernel<6>;
    case 17: return lds_kernel<7>;
    default: return nullptr;
  }
}

}  // namespace

extern "C" {

const char* micro_error(void) { return g_err; }

// Runs unit probe `probe` (see unit_fn) on `blocks` workgroups of 256
// threads, `iters` outer iterations (4 inner steps each), best of `reps`.
// Writes: ms = kernel time (events), clk_mhz = shader clock from the stamps
// (mean over workgroups), span = mean fraction of the kernel time a
// workgroup spent between its stamps.
int micro_unit(int probe, int blocks, int iters, int reps, double* ms, double* clk_mhz, double* span) {
  UnitFn fn = unit_fn(probe);
  if (!fn || blocks <= 0 || iters <= 0 || reps <= 0 || !ms || !clk_mhz || !span) {
    snprintf(g_err, sizeof g_err, "bad arguments");
    return -2;
  }
  int dev = 0, wall_khz = 0;
  CK(hipGetDevice(&dev));
  CK(hipDeviceGetAttribute(&wall_khz, hipDeviceAttributeWallClockRate, dev));
  float* out = nullptr;
  uint64_t* st = nullptr;
  CK(hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)));
  CK(hipMalloc(&st, (size_t)blocks * 4 * sizeof(uint64_t)));
  hipEvent_t a, b;
  CK(hipEventCreate(&a));
  CK(hipEventCreate(&b));
  double best = 1e30, best_clk = 0, best_span = 0;
  uint64_t* hst = (uint64_t*)malloc((size_t)blocks * 4 * sizeof(uint64_t));
  for (int r = 0; r < reps; ++r) {
    CK(hipEventRecord(a, 0));
    hipLaunchKernelGGL(fn, dim3(blocks), dim3(256), 0, 0, out, iters, st);
    CK(hipGetLastError());
    CK(hipEventRecord(b, 0));
    CK(hipEventSynchronize(b));
    float t = 0.f;
    CK(hipEventElapsedTime(&t, a, b));
    CK(hipMemcpy(hst, st, (size_t)blocks * 4 * sizeof(uint64_t), hipMemcpyDeviceToHost));
    double clk = 0, sp = 0;
    for (int i = 0; i < blocks; ++i) {
      const double dc = (double)(hst[4 * i + 2] - hst[4 * i]);
      const double dw = (double)(hst[4 * i + 3] - hst[4 * i + 1]);
      const double wall_s = dw / (wall_khz * 1e3);
      clk += dc / wall_s / 1e6;
      sp += wall_s * 1e3 / t;
    }
    if (t < best) {
      best = t;
      best_clk = clk / blocks;
      best_span = sp / blocks;
    }
  }
  free(hst);
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  (void)hipFree(out);
  (void)hipFree(st);
  *ms = best;
  *clk_mhz = best_clk;
  *span = best_span;
  return 0;
}

// HBM probe: kind 0 = read, 1 = write, 2 = copy, over `bytes` (a multiple
// of 16; copy moves bytes from one buffer to another). Best of `reps`.
int micro_hbm(int kind, size_t bytes, int blocks, int reps, double* ms) {
  if (kind < 0 || kind > 2 || bytes == 0 || bytes % 16 || blocks <= 0 || reps <= 0 || !ms) {
    snprintf(g_err, sizeof g_err, "bad arguments");
    return -2;
  }
  u32x4 *src = nullptr, *dst = nullptr;
  float* out = nullptr;
  CK(hipMalloc(&src, bytes));
  if (kind == 2) CK(hipMalloc(&dst, bytes));
  CK(hipMalloc(&out, 16));
  CK(hipMemset(src, 1, bytes));
  hipEvent_t a, b;
  CK(hipEventCreate(&a));
  CK(hipEventCreate(&b));
  const size_t n16 = bytes / 16;
  double best = 1e30;
  for (int r = 0; r < reps; ++r) {
    CK(hipEventRecord(a, 0));
    if (kind == 0) hipLaunchKernelGGL(read_kernel, dim3(blocks), dim3(256), 0, 0, src, n16, out);
    else if (kind == 1) hipLaunchKernelGGL(write_kernel, dim3(blocks), dim3(256), 0, 0, src, n16);
    else hipLaunchKernelGGL(copy_kernel, dim3(blocks), dim3(256), 0, 0, src, dst, n16);
    CK(hipGetLastError());
    CK(hipEventRecord(b, 0));
    CK(hipEventSynchronize(b));
    float t = 0.f;
    CK(hipEventElapsedTime(&t, a, b));
    if (t < best) best = t;
  }
  (void)hipEventDestroy(a);
  (void)hipEventDestroy(b);
  (void)hipFree(src);
  if (dst) (void)hipFree(dst);
  (void)hipFree(out);
  *ms = best;
  return 0;
}

int micro_cu_count(void) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
  return cus;
}

}  // extern "C"
