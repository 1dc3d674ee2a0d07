// Host side of the C ABI declared in include/bra.h: argument checks, the
// library-owned workspace, stream selection, kernel dispatch, error text and
// event-based per-kernel timing. No kernel lives here.
#include "../../include/bra.h"

#include <math.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "bra_internal.h"

namespace bra {
hipError_t launch_attend_valu(const void* q, const void* k, const void* v,
                              const void* w, const void* b, const int32_t* route,
                              const Shape& s, int dtype, void* out, hipStream_t st);
hipError_t launch_attend_mfma(const void* q, const void* k, const void* v,
                              const void* w, const void* b, const int32_t* route,
                              const Shape& s, void* out, hipStream_t st);
bool mfma_supports(const Shape& s);
bool region_kernel_supports(const Shape& s);
hipError_t launch_attend_region(const void* q, const void* k, const void* v, const uint32_t* wpk,
                                const void* b, const int32_t* route, const Shape& s, void* out,
                                hipStream_t st);
bool image_kernel_supports(const Shape& s);
bool image_kernel_routes(const Shape& s);
hipError_t launch_attend_image(const void* q, const void* k, const void* v, const uint32_t* wpk,
                               const void* b, const int32_t* route, const Shape& s, void* out,
                               hipStream_t st);
// The whole forward in one kernel (4x4 regions, image_kernel_routes): region
// means, routes (reported to route_out), attention and LCE from the weights
// as given; no workspace
hipError_t launch_forward_image(const void* q, const void* k, const void* v, const void* lce_w,
                                const void* b, const Shape& s, void* out, int32_t* route_out,
                                hipStream_t st);
// y = x w^T + b, output features split over y0..y2 in blocks of split
// (linear.hip)
hipError_t launch_linear(const void* x, const void* w, const void* b, int M, int K, int Nout,
                         int split, int dtype, void* y0, void* y1, void* y2, hipStream_t st);
bool tile_kernel_supports(const Shape& s);
bool f32_kernel_supports(const Shape& s);
hipError_t launch_attend_f32(const void* q, const void* k, const void* v, const void* w,
                             const void* b, const int32_t* route, const Shape& s, void* out,
                             hipStream_t st);
hipError_t launch_attend_tile(const void* q, const void* k, const void* v, const uint32_t* wpk,
                              const void* b, const int32_t* route, const Shape& s, void* out,
                              hipStream_t st);
size_t lce_pack_bytes(int C);
hipError_t launch_lce_pack(const void* w, int C, uint32_t* wpk, hipStream_t st);

ProfEvents& prof_events() {
  thread_local ProfEvents pe;
  return pe;
}

int device_cu_count() {
  static std::atomic<int> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < 64) {
    const int c = cached[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
  }
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 0;
  if (dev < 64 && cus > 0) cached[dev].store(cus, std::memory_order_relaxed);
  return cus;
}
}  // namespace bra

namespace {

thread_local hipStream_t g_stream = nullptr;
thread_local hipError_t g_last_hip = hipSuccess;
thread_local char g_msg[256];

struct Workspace {
  void* ptr = nullptr;
  size_t bytes = 0;
};
std::mutex g_ws_mutex;
std::vector<Workspace> g_ws;  // indexed by device ordinal

// ---- event timing ---------------------------------------------------------
constexpr int kMaxEvents = 4096;
struct KindRecord {
  std::vector<hipEvent_t> start, stop;
  int used = 0;
};
std::mutex g_prof_mutex;
int g_prof_mask = 0;  // bit k: record events around kernels of kind k
KindRecord g_prof[BRA_K_COUNT];

// Arms the event pair of one record slot for the next kernel this thread
// launches (bra::launch stamps them with that dispatch's start and end). If
// no kernel took them, both are recorded on the stream when the scope ends.
struct ProfScope {
  int kind;
  hipStream_t st;
  int slot = -1;
  ProfScope(int kind_, hipStream_t st_) : kind(kind_), st(st_) {
    if (!(g_prof_mask & (1 << kind))) return;
    std::lock_guard<std::mutex> lk(g_prof_mutex);
    KindRecord& rec = g_prof[kind];
    if (rec.used >= kMaxEvents) return;
    if ((int)rec.start.size() <= rec.used) {
      hipEvent_t a, b;
      // device-scope release: no L2 write-back to memory is timed with the kernel
      if (hipEventCreateWithFlags(&a, hipEventReleaseToDevice) != hipSuccess) return;
      if (hipEventCreateWithFlags(&b, hipEventReleaseToDevice) != hipSuccess) {
        hipEventDestroy(a);
        return;
      }
      rec.start.push_back(a);
      rec.stop.push_back(b);
    }
    slot = rec.used++;
    bra::ProfEvents& pe = bra::prof_events();
    pe.start = rec.start[slot];
    pe.stop = rec.stop[slot];
  }
  ~ProfScope() {
    if (slot < 0) return;
    bra::ProfEvents& pe = bra::prof_events();
    if (pe.start) {
      hipEventRecord(pe.start, st);
      hipEventRecord(pe.stop, st);
      pe.start = pe.stop = nullptr;
    }
  }
};

int hip_fail(hipError_t e) {
  g_last_hip = e;
  return BRA_ERR_HIP;
}

int check_dims(int N, int H, int W, int C, int heads, int S, int topk, int dtype,
               bool use_heads, bool use_topk, bra::Shape* out) {
  if (dtype != BRA_F32 && dtype != BRA_BF16) return BRA_ERR_DTYPE;
  if (N <= 0 || H <= 0 || W <= 0 || C <= 0 || S <= 0) return BRA_ERR_SHAPE;
  if (use_heads && heads <= 0) return BRA_ERR_SHAPE;
  if (H % S != 0 || W % S != 0) return BRA_ERR_SHAPE;
  if (use_heads && C % heads != 0) return BRA_ERR_SHAPE;
  const long long R = (long long)S * S;
  if (use_topk && (topk < 1 || topk > R)) return BRA_ERR_TOPK;
  // compiled envelope
  if (R > bra::kMaxRegions) return BRA_ERR_UNSUPPORTED;
  if (C % bra::kHeadDim != 0 || C > 1024) return BRA_ERR_UNSUPPORTED;
  if (use_heads && C / heads != bra::kHeadDim) return BRA_ERR_UNSUPPORTED;
  const long long T = (long long)(H / S) * (W / S);
  if (use_topk && T * topk > 65536) return BRA_ERR_UNSUPPORTED;
  if ((long long)N * H * W * C >= (1ll << 40)) return BRA_ERR_UNSUPPORTED;
  bra::Shape& s = *out;
  s.N = N; s.H = H; s.W = W; s.C = C; s.heads = use_heads ? heads : 1;
  s.S = S; s.topk = use_topk ? topk : 1;
  s.R = (int)R; s.rh = H / S; s.rw = W / S; s.T = (int)T;
  s.hd = use_heads ? C / heads : bra::kHeadDim;
  s.L = s.topk * s.T;
  return BRA_OK;
}

// Rejects host or unknown pointers (a kernel dereferencing one would fault).
int check_device_ptr(const void* p) {
  if (p == nullptr) return BRA_OK;
  hipPointerAttribute_t attr;
  hipError_t e = hipPointerGetAttributes(&attr, p);
  if (e != hipSuccess) {
    (void)hipGetLastError();
    return BRA_ERR_POINTER;
  }
  if (attr.type != hipMemoryTypeDevice && attr.type != hipMemoryTypeManaged)
    return BRA_ERR_POINTER;
  return BRA_OK;
}

int check_ptrs(std::initializer_list<const void*> ps) {
  for (const void* p : ps) {
    int rc = check_device_ptr(p);
    if (rc) return rc;
  }
  return BRA_OK;
}

// Kernels read tensors with 16-byte vector loads (the bias and route
// indices with 4-byte loads).
int check_align(std::initializer_list<const void*> p16, std::initializer_list<const void*> p4) {
  for (const void* p : p16)
    if (p && ((uintptr_t)p & 15u)) return BRA_ERR_ALIGN;
  for (const void* p : p4)
    if (p && ((uintptr_t)p & 3u)) return BRA_ERR_ALIGN;
  return BRA_OK;
}

int workspace(size_t bytes, void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0) return hip_fail(hipErrorInvalidDevice);
  if ((int)g_ws.size() <= dev) g_ws.resize(dev + 1);
  Workspace& ws = g_ws[dev];
  if (ws.bytes < bytes) {
    if (ws.ptr) {
      e = hipDeviceSynchronize();  // earlier calls may still read the old buffer
      if (e != hipSuccess) return hip_fail(e);
      (void)hipFree(ws.ptr);
      ws.ptr = nullptr;
      ws.bytes = 0;
    }
    e = hipMalloc(&ws.ptr, bytes);
    if (e != hipSuccess) {
      ws.ptr = nullptr;
      return hip_fail(e);
    }
    ws.bytes = bytes;
  }
  *ptr = ws.ptr;
  return BRA_OK;
}

// Workspace layout: fp32 region means of q and k ([N][S*S][C] each), then the
// LCE weights packed for the small-region kernel (30*C dwords).
struct WsLayout {
  size_t means, wpk, total;
};
WsLayout ws_layout(int N, int C, int S) {
  WsLayout l;
  l.means = (size_t)2 * N * S * S * C * sizeof(float);
  l.wpk = (l.means + 255) & ~(size_t)255;
  l.total = l.wpk + bra::lce_pack_bytes(C);
  return l;
}

// Attention + LCE over given routes (wpk: packed LCE weights, required by the
// small-region kernel).
int attend(const void* q, const void* k, const void* v, const void* w, const void* b,
           const int32_t* route, const bra::Shape& s, int dtype, void* out, const uint32_t* wpk,
           hipStream_t st) {
  hipError_t e;
  {
    ProfScope ps(BRA_K_ATTN, st);
    if (dtype == BRA_BF16 && wpk && bra::image_kernel_supports(s))
      e = bra::launch_attend_image(q, k, v, wpk, b, route, s, out, st);
    else if (dtype == BRA_BF16 && wpk && bra::region_kernel_supports(s))
      e = bra::launch_attend_region(q, k, v, wpk, b, route, s, out, st);
    else if (dtype == BRA_BF16 && wpk && bra::tile_kernel_supports(s))
      e = bra::launch_attend_tile(q, k, v, wpk, b, route, s, out, st);
    else if (dtype == BRA_BF16 && bra::mfma_supports(s))
      e = bra::launch_attend_mfma(q, k, v, w, b, route, s, out, st);
    else if (dtype == BRA_F32 && bra::f32_kernel_supports(s))
      e = bra::launch_attend_f32(q, k, v, w, b, route, s, out, st);
    else
      e = bra::launch_attend_valu(q, k, v, w, b, route, s, dtype, out, st);
  }
  return e == hipSuccess ? BRA_OK : hip_fail(e);
}

}  // namespace

extern "C" {

int bra_forward(const void* q, const void* k, const void* v, const void* lce_w,
                const void* lce_b, int N, int H, int W, int C, int heads, int S,
                int topk, int dtype, void* out, int32_t* route_idx) {
  if (!q || !k || !v || !lce_w || !out || !route_idx) return BRA_ERR_NULL;
  bra::Shape s;
  int rc = check_dims(N, H, W, C, heads, S, topk, dtype, true, true, &s);
  if (rc) return rc;
  rc = check_align({q, k, v, lce_w, out}, {lce_b, route_idx});
  if (rc) return rc;
  rc = check_ptrs({q, k, v, lce_w, lce_b, out, route_idx});
  if (rc) return rc;
  hipStream_t st = g_stream;
  hipError_t e;
  if (dtype == BRA_BF16 && bra::image_kernel_routes(s)) {
    // one kernel: it pools and routes its own images (the route kernel's
    // logit and selection code) and reports the routes to route_idx
    {
      ProfScope ps(BRA_K_ATTN, st);
      e = bra::launch_forward_image(q, k, v, lce_w, lce_b, s, out, route_idx, st);
    }
    return e == hipSuccess ? BRA_OK : hip_fail(e);
  }
  std::lock_guard<std::mutex> lk(g_ws_mutex);
  const WsLayout wl = ws_layout(N, C, S);
  void* ws = nullptr;
  rc = workspace(wl.total, &ws);
  if (rc) return rc;
  float* qr = static_cast<float*>(ws);
  float* kr = qr + (size_t)N * s.R * C;
  uint32_t* wpk = dtype == BRA_BF16 ? reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + wl.wpk) : nullptr;
  {
    ProfScope ps(BRA_K_POOL, st);
    e = bra::launch_region_pool(q, k, s, dtype, qr, kr, lce_w, wpk, st);
  }
  if (e != hipSuccess) return hip_fail(e);
  {
    ProfScope ps(BRA_K_ROUTE, st);
    e = bra::launch_route(qr, kr, N, s.R, C, topk, route_idx, st);
  }
  if (e != hipSuccess) return hip_fail(e);
  return attend(q, k, v, lce_w, lce_b, route_idx, s, dtype, out, wpk, st);
}

int bra_region_means(const void* q, const void* k, int N, int H, int W, int C, int S,
                     int dtype, float* qr, float* kr) {
  if (!q || !k || !qr || !kr) return BRA_ERR_NULL;
  bra::Shape s;
  int rc = check_dims(N, H, W, C, 1, S, 1, dtype, false, false, &s);
  if (rc) return rc;
  rc = check_align({q, k, qr, kr}, {});
  if (rc) return rc;
  rc = check_ptrs({q, k, qr, kr});
  if (rc) return rc;
  hipStream_t st = g_stream;
  hipError_t e;
  {
    ProfScope ps(BRA_K_POOL, st);
    e = bra::launch_region_pool(q, k, s, dtype, qr, kr, nullptr, nullptr, st);
  }
  return e == hipSuccess ? BRA_OK : hip_fail(e);
}

int bra_route(const float* qr, const float* kr, int N, int R, int C, int topk,
              int32_t* route_idx) {
  if (!qr || !kr || !route_idx) return BRA_ERR_NULL;
  if (N <= 0 || R <= 0 || C <= 0) return BRA_ERR_SHAPE;
  if (topk < 1 || topk > R) return BRA_ERR_TOPK;
  if (R > bra::kMaxRegions || C % bra::kHeadDim != 0 || C > 1024) return BRA_ERR_UNSUPPORTED;
  int rc = check_align({qr, kr}, {route_idx});
  if (rc) return rc;
  rc = check_ptrs({qr, kr, route_idx});
  if (rc) return rc;
  hipStream_t st = g_stream;
  hipError_t e;
  {
    ProfScope ps(BRA_K_ROUTE, st);
    e = bra::launch_route(qr, kr, N, R, C, topk, route_idx, st);
  }
  return e == hipSuccess ? BRA_OK : hip_fail(e);
}

int bra_attend(const void* q, const void* k, const void* v, const void* lce_w,
               const void* lce_b, const int32_t* route_idx, int N, int H, int W, int C,
               int heads, int S, int topk, int dtype, void* out) {
  if (!q || !k || !v || !lce_w || !route_idx || !out) return BRA_ERR_NULL;
  bra::Shape s;
  int rc = check_dims(N, H, W, C, heads, S, topk, dtype, true, true, &s);
  if (rc) return rc;
  rc = check_align({q, k, v, lce_w, out}, {lce_b, route_idx});
  if (rc) return rc;
  rc = check_ptrs({q, k, v, lce_w, lce_b, route_idx, out});
  if (rc) return rc;
  hipStream_t st = g_stream;
  if (dtype == BRA_BF16 && (bra::image_kernel_supports(s) || bra::region_kernel_supports(s) ||
                            bra::tile_kernel_supports(s))) {
    std::lock_guard<std::mutex> lk(g_ws_mutex);
    void* ws = nullptr;
    rc = workspace(bra::lce_pack_bytes(C), &ws);
    if (rc) return rc;
    uint32_t* wpk = static_cast<uint32_t*>(ws);
    hipError_t e = bra::launch_lce_pack(lce_w, C, wpk, st);
    if (e != hipSuccess) return hip_fail(e);
    return attend(q, k, v, lce_w, lce_b, route_idx, s, dtype, out, wpk, st);
  }
  return attend(q, k, v, lce_w, lce_b, route_idx, s, dtype, out, nullptr, st);
}

int bra_lce(const void* v, const void* lce_w, const void* lce_b, int N, int H, int W,
            int C, int dtype, float* out) {
  if (!v || !lce_w || !out) return BRA_ERR_NULL;
  bra::Shape s;
  int rc = check_dims(N, H, W, C, 1, 1, 1, dtype, false, false, &s);
  if (rc) return rc;
  rc = check_align({v, out}, {lce_b});
  if (rc) return rc;
  rc = check_ptrs({v, lce_w, lce_b, out});
  if (rc) return rc;
  hipStream_t st = g_stream;
  hipError_t e;
  {
    ProfScope ps(BRA_K_LCE, st);
    e = bra::launch_lce(v, lce_w, lce_b, s, dtype, out, st);
  }
  return e == hipSuccess ? BRA_OK : hip_fail(e);
}

int bra_linear(const void* x, const void* w, const void* b, int M, int K, int Nout, int split,
               int dtype, void* y0, void* y1, void* y2) {
  if (!x || !w || !y0) return BRA_ERR_NULL;
  if (dtype != BRA_F32 && dtype != BRA_BF16) return BRA_ERR_DTYPE;
  if (M <= 0 || K <= 0 || Nout <= 0 || split <= 0) return BRA_ERR_SHAPE;
  const int parts = Nout / split;
  if (Nout % split != 0 || parts > 3) return BRA_ERR_SHAPE;
  if ((parts > 1 && !y1) || (parts > 2 && !y2)) return BRA_ERR_NULL;
  const long long esz = dtype == BRA_BF16 ? 2 : 4;
  if (K % 32 != 0 || split % 8 != 0) return BRA_ERR_UNSUPPORTED;
  if (dtype == BRA_BF16 && K > 256) return BRA_ERR_UNSUPPORTED;
  if ((long long)M * K * esz >= (1ll << 31) || (long long)Nout * K * esz >= (1ll << 31) ||
      (long long)M * split * esz >= (1ll << 40))
    return BRA_ERR_UNSUPPORTED;
  const void* y1c = parts > 1 ? y1 : nullptr;
  const void* y2c = parts > 2 ? y2 : nullptr;
  int rc = check_align({x, w}, {b, y0, y1c, y2c});
  if (rc) return rc;
  if (((uintptr_t)y0 | (uintptr_t)y1c | (uintptr_t)y2c) & 15u) return BRA_ERR_ALIGN;
  rc = check_ptrs({x, w, b, y0, y1c, y2c});
  if (rc) return rc;
  hipStream_t st = g_stream;
  hipError_t e;
  {
    ProfScope ps(BRA_K_LINEAR, st);
    e = bra::launch_linear(x, w, b, M, K, Nout, split, dtype, y0, const_cast<void*>(y1c),
                           const_cast<void*>(y2c), st);
  }
  return e == hipSuccess ? BRA_OK : hip_fail(e);
}

int bra_set_stream(void* stream) {
  g_stream = static_cast<hipStream_t>(stream);
  return BRA_OK;
}

void* bra_get_stream(void) { return g_stream; }

size_t bra_workspace_bytes(int N, int C, int S) {
  if (N <= 0 || C <= 0 || S <= 0) return 0;
  return ws_layout(N, C, S).total;
}

void bra_release(void) {
  std::lock_guard<std::mutex> lk(g_ws_mutex);
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) cur = -1;
  for (size_t d = 0; d < g_ws.size(); ++d) {
    if (!g_ws[d].ptr) continue;
    if (hipSetDevice((int)d) == hipSuccess) {
      (void)hipDeviceSynchronize();
      (void)hipFree(g_ws[d].ptr);
    }
    g_ws[d].ptr = nullptr;
    g_ws[d].bytes = 0;
  }
  if (cur >= 0) (void)hipSetDevice(cur);
}

const char* bra_error_string(int code) {
  switch (code) {
    case BRA_OK: return "ok";
    case BRA_ERR_NULL: return "a required pointer is NULL";
    case BRA_ERR_SHAPE: return "invalid sizes: a size <= 0, H or W not divisible by S, or C not divisible by heads";
    case BRA_ERR_TOPK: return "topk outside [1, S*S]";
    case BRA_ERR_DTYPE: return "unknown dtype (0 = f32, 1 = bf16)";
    case BRA_ERR_UNSUPPORTED: return "outside the compiled envelope (head_dim 32, C <= 1024, S*S <= 1024, topk*T <= 65536)";
    case BRA_ERR_POINTER: return "a tensor pointer is not device memory";
    case BRA_ERR_ALIGN: return "a tensor pointer is misaligned (16 bytes for q, k, v, out, lce_w and region means; 4 for lce_b and route_idx)";
    case BRA_ERR_HIP:
      snprintf(g_msg, sizeof g_msg, "HIP failure: %s", hipGetErrorString(g_last_hip));
      return g_msg;
    default: return "unknown status code";
  }
}

int bra_version(void) { return 100; }

int bra_profile_begin(int mask) {
  std::lock_guard<std::mutex> lk(g_prof_mutex);
  g_prof_mask = mask & ((1 << BRA_K_COUNT) - 1);
  for (auto& r : g_prof) r.used = 0;
  return BRA_OK;
}

int bra_profile_set_mask(int mask) {
  std::lock_guard<std::mutex> lk(g_prof_mutex);
  g_prof_mask = mask & ((1 << BRA_K_COUNT) - 1);
  return BRA_OK;
}

int bra_profile_read(double* ms, int* counts, int n) {
  if (!ms || !counts) return BRA_ERR_NULL;
  std::lock_guard<std::mutex> lk(g_prof_mutex);
  for (int kd = 0; kd < n; ++kd) {
    ms[kd] = 0.0;
    counts[kd] = 0;
    if (kd >= BRA_K_COUNT) continue;
    KindRecord& rec = g_prof[kd];
    for (int i = 0; i < rec.used; ++i) {
      hipError_t e = hipEventSynchronize(rec.stop[i]);
      if (e != hipSuccess) return hip_fail(e);
      float t = 0.f;
      e = hipEventElapsedTime(&t, rec.start[i], rec.stop[i]);
      if (e != hipSuccess) return hip_fail(e);
      ms[kd] += t;
      counts[kd] += 1;
    }
    rec.used = 0;
  }
  return BRA_OK;
}

int bra_calib_copy(const void* src, void* dst, size_t bytes) {
  if (!src || !dst) return BRA_ERR_NULL;
  if (bytes % 16 != 0 || ((uintptr_t)src % 16) || ((uintptr_t)dst % 16)) return BRA_ERR_SHAPE;
  int rc = check_ptrs({src, dst});
  if (rc) return rc;
  hipError_t e = bra::launch_copy(src, dst, bytes, g_stream);
  return e == hipSuccess ? BRA_OK : hip_fail(e);
}

}  // extern "C"
