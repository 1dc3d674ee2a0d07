// Gathered attention + LCE for large regions (T = RH*RW a multiple of 64
// tokens), bf16 tensors -- BiFormer's dense-prediction stages (8x8 regions
// for detection at S=16, 16x16 regions for segmentation at S=8). Eqs. 6-7 of
// the BRA walk-through at TRANSFORMER.niftyadmin.cn/n/347023.html, section
// BRA模块: each query region attends, per head, to the tokens of its topk
// routed regions (topk*T keys, one joint softmax), plus LCE(V).
//
// One workgroup of four waves per (image, region, head, query slab): a wave
// owns one 16-query block, or two when region rows are 16 tokens long (then
// its two blocks are two rows of one column band), so a workgroup covers 64
// or 128 queries and a larger region is cut into slabs of whole rows. Small
// workgroups keep four independent ones on each CU, in different phases of
// their tile loops, so one's matrix-core work overlaps another's softmax.
// The gathered keys are walked in 64-key tiles, loaded straight into LDS
// (buffer loads with the LDS as destination: no registers hold them) one
// tile ahead of the one being computed, in two tile buffers, one workgroup
// barrier a tile. (The compiler makes every LDS read wait for all loads into
// LDS issued before it, so a step reads its operands first and then starts
// the next tile's loads.)
// The K tile is stored in the matrix cores' operand order: the 16-byte
// slot (x, c, col) at x*1024 + c*256 + col*16 holds chunk c (dims 8c..8c+7)
// of the key that row col of score tile x takes, so an A-operand read is
// one contiguous KiB per wave -- the pattern gfx950's LDS serves at its full
// 256 bytes per clock (16 rows x one chunk per 16 lanes runs at half that).
// The V tile is row-major, one key's 64 bytes a row with its four 16-byte
// chunks XOR-swizzled by the row (chunk c of row r at c ^ swz(r)), for the
// transposing V^T reads (ds_read_b64_tr_b16: 4 rows x 16 channels per 16
// lanes; these run at 128 bytes per clock whatever the layout). The loads
// into LDS place every chunk where it belongs. Each wave reuses every K /
// V^T operand read for its query blocks:
//
//   S^T(16 keys x 16 queries) = K (A: lane = key row) x Q^T (B: lane = query)
//   O^T(16 dims x 16 queries) += V^T (A) x P^T (B),   sum(P) via ones x P^T
//
// Inside each 32-key block the K rows fed to the two score tiles are
// permuted (tile 0 row 4g+e <- key 8g+e, tile 1 row 4g+e <- key 8g+4+e) so
// that a lane's eight scores are eight CONSECUTIVE keys: P^T needs no
// shuffle.
//
// Softmax with a fixed maximum per query. The query operand is scaled
// first, q' = bf16(qscale * q), and every score q'.k is at most |q'| *
// max |k| over the routed keys (Cauchy-Schwarz); the pool kernel reports
// max |k|^2 per (image, region, head), so a query's bound m is known before
// its first key. The score products start from -m, and P = 2^(s - m) <= 1
// needs no running maximum, no rescaling and no per-tile check: per score
// one v_exp_f32 and half a packed bf16 conversion. P is rounded to bf16 for
// the products and the row sums are taken over that same bf16 P on the
// matrix cores. The bound can sit far above the true maximum (a query
// nearly orthogonal to long keys); then the P of that query underflow.
// Whenever some query's row sum ends below 2^-64 -- i.e. its largest score
// lies more than 64 (base 2) under the bound -- the workgroup runs the exact
// way instead: one pass over the keys for each query's maximum score, then
// the softmax pass again with m = that maximum. Without reported norms (the
// stage entry point that takes given routes) it starts that way.
//
// LCE (5x5 depthwise, zero padding 2, bias): the head's 32 channels of the
// slab's V halo (its rows +- 2, RW+4 pixels wide) are loaded into LDS in the
// first tile step, behind the keys; after the last tile they are repacked
// into the freed tile buffers as horizontal pixel pairs, and with the
// weights as matching pairs each lane's output takes 15 packed-bf16 dot
// products per channel. Workgroups of one image are numbered onto one XCD.
//
// With HG > 1 (the block's path: HG = heads) one workgroup covers every head
// of its (image, region, slab): four waves per head, each head with its own
// tile buffers and halo (the LCE weights are loaded after the key loop into
// the head's freed halo staging, so two heads fit 64 KiB of LDS), and the
// output projection of the walk-through's BRA block (wo = Linear(C, C),
// section BRA模块) runs in the epilogue: the attention + LCE output is
// rounded to bf16 (the block's hand-off precision) in the channel order
// {4g..4g+3, 16+4g..16+4g+3} of lane group g, which is a B operand of the
// 16x16x32 products as it stands; the waves of the same queries exchange
// theirs through LDS and wave (head h) computes output channels 32h..32h+31
// of its queries as y^T = Wo . o^T (the weight rows read in the same channel
// order), adds the bias and stores them.
#include "bra_internal.h"
#include "route_common.h"

namespace bra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kTileBytes = 64 * 64;  // one 64-key tile of K (or V): 64 rows of 64 bytes
constexpr float kUnderflow = 5.421010862427522e-20f;  // 2^-64
// s_waitcnt immediates (vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt
// 11:8): no vector memory and no LDS operation outstanding
constexpr int kVmcnt0 = 0x0070;

// The workgroup barrier of the tile loop: the caller's s_waitcnt has already
// drained this wave's loads into LDS and its LDS reads, and the empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void tile_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

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
__device__ __forceinline__ bf16x4 ld_tr(const char* p) {
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(const_cast<char*>(p)));
  return __builtin_bit_cast(bf16x4, v);
}
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a),
                                         __builtin_bit_cast(bf16x2, b), c, false);
}
// Chunk swizzle of tile row r: rows 8g..8g+7 take XOR mask 0, 2, 1, 3 for
// g % 4 = 0, 1, 2, 3. Bytes of (row r, chunk c): r * 64 + ((c ^ swz(r)) << 4).
__device__ __forceinline__ int swz(int r) {
  const int g = (r >> 3) & 3;
  return ((g & 1) << 1) | (g >> 1);
}
__device__ __forceinline__ int tile_off(int r, int c) { return r * 64 + ((c ^ swz(r)) << 4); }
// The key (0..63 within a tile) that row `row` of score tile x (0..3) takes:
// tile 2b+o, row 4g+e <- key 32b + 8g + 4o + e (see the permutation above)
__device__ __forceinline__ int score_key(int x, int row) {
  return 32 * (x >> 1) + 8 * (row >> 2) + 4 * (x & 1) + (row & 3);
}

struct TileArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint32_t* wpk;  // LCE weights as dot2 pairs: [2 parity][15 (row, pair)][C]
  const uint16_t* b;
  const int32_t* route;  // [N][S*S][topk]
  const float* kn;       // [N][S*S][heads] max |k|^2 of each region's head slice, or null
  const uint16_t* wo;    // HG > 1: the output projection's weight [C][C] (out, in) and bias [C] or null
  const uint16_t* bo;
  // routing in the kernel (S*S <= 64): the region means [N][S*S][C] (fp32),
  // or null when the routes are given; the chosen routes are written to
  // route_out ([N][S*S][topk])
  const float* qr;
  const float* kr;
  int32_t* route_out;
  float rscale;    // the affinity's scale: C^-1/2, or head_dim^-1/2 with head_routes
  int head_routes;  // each head routes on its own channels: logits over the
                    // head's 32-channel slice of the means, route_out
                    // [N][heads][S*S][topk]
  uint16_t* out;
  int N, H, W, C, heads, S, topk;
  float qscale;  // head_dim^-1/2 * log2(e)
};

__host__ __device__ constexpr size_t align16(size_t x) { return (x + 15) & ~(size_t)15; }

// which pass over the keys: each query's maximum score, or the softmax
struct MaxTag { static constexpr bool value = true; };
struct SoftTag { static constexpr bool value = false; };

constexpr int kTileWaves = 4;
constexpr int kBufs = 2;                     // tile buffers: one computed, one landing
constexpr int kBufBytes = 2 * kTileBytes;    // K rows, then V rows of one 64-key tile
// query blocks of 16 per wave, and query slabs per region
template <int RH, int RW>
constexpr int tile_qbw() { return RW == 16 ? 2 : 1; }
template <int RH, int RW>
constexpr int tile_slabs() { return RH * RW / (16 * kTileWaves * tile_qbw<RH, RW>()); }
// LCE halo of a slab of SR query rows, (SR + 4) x (RW + 4) pixels of the
// head's 32 channels: as loaded (64 bytes a pixel) and as pixel pairs
__host__ __device__ constexpr size_t halo_raw_bytes(int SR, int RW) { return (size_t)(SR + 4) * (RW + 4) * 64; }
__host__ __device__ constexpr size_t halo_bytes(int SR, int RW) {
  return (size_t)(SR + 4) * ((RW + 5) / 2) * 32 * 4;
}

constexpr size_t kWtsBytes = align16((size_t)2 * 15 * 32 * 4);  // a head's LCE weight pairs
// the output exchange of one head's waves (HG > 1): [waves][QBW][64 lanes] x 16 bytes
__host__ __device__ constexpr size_t xch_bytes(int qbw) { return (size_t)kTileWaves * qbw * 64 * 16; }

struct TileLds {
  size_t tiles, halo, raw, wts, xch, head, flag, rbase, total;
};
// The halo is loaded into `raw` at the start and repacked into pixel pairs
// in the tile buffers after the last tile. The route table (topk entries)
// goes last, so the other offsets stay constant. With HG > 1 heads a
// workgroup, each head has its own [tiles | raw] block (stride `head`), and
// its LCE weights and output exchange go into its raw area after the repack.
__host__ __device__ inline TileLds tile_lds(int SR, int RW, int topk, int HG, int qbw) {
  TileLds l;
  size_t o = 0;
  l.tiles = o; l.halo = o; o += (size_t)kBufs * kBufBytes;
  l.raw = o; o += halo_raw_bytes(SR, RW);
  if (HG == 1) {
    l.head = 0;
    l.xch = 0;
    l.wts = o; o += kWtsBytes;
  } else {
    l.head = o;
    l.wts = l.raw;
    l.xch = l.raw + kWtsBytes;
    o *= (size_t)HG;
  }
  l.flag = o; o += 16;
  l.rbase = o; o += (size_t)4 * topk;
  l.total = o;
  return l;
}

template <int RH, int RW, int HG, bool WO>
__global__ __launch_bounds__(64 * kTileWaves * HG, 4) void attn_tile_kernel(TileArgs a) {
  static_assert(!WO || HG > 1, "the output projection needs every head of the region in the workgroup");
  constexpr int T = RH * RW;
  constexpr int WAVES = kTileWaves;  // waves of one head
  constexpr int NT = 64 * WAVES;     // threads of one head
  constexpr int QBW = tile_qbw<RH, RW>();
  constexpr int SLABS = tile_slabs<RH, RW>();
  constexpr int SR = RH / SLABS;  // region rows per slab
  constexpr int HP = SR + 4, WP = RW + 4, NPAIR = (WP + 1) / 2;
  static_assert(SLABS * SR == RH && SR * RW == 16 * WAVES * QBW, "slabs of whole rows");
  static_assert(halo_bytes(SR, RW) <= (size_t)kBufs * kBufBytes, "the halo fits the tile buffers");
  static_assert(halo_raw_bytes(SR, RW) % 1024 == 0 && WP % 2 == 0, "whole 1 KiB loads, whole pixel pairs");
  static_assert(64 % RW == 0, "a tile starts on a region row");
  static_assert(HG == 1 || kWtsBytes + xch_bytes(QBW) <= halo_raw_bytes(SR, RW),
                "weights and output exchange fit a head's halo staging");
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const TileLds lay = tile_lds(SR, RW, a.topk, HG, QBW);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = lane & 15, grp = lane >> 4;
  // the wave's head within the workgroup, its wave and thread index there
  const int hw = wave / WAVES, wv = wave % WAVES, htid = tid % NT;
  char* hsm = smem + hw * lay.head;  // this head's block (HG > 1)
  char* tiles = hsm + lay.tiles;  // [kBufs][K: 64 rows x 64 bytes | V: the same], swizzled chunks
  uint32_t* halo = reinterpret_cast<uint32_t*>(hsm + lay.halo);  // [HP][NPAIR][32] after the loop
  char* raw = hsm + lay.raw;                                      // [HP][WP][64 bytes]
  uint32_t* wts = reinterpret_cast<uint32_t*>(hsm + lay.wts);    // [2][15][32]
  int* flag = reinterpret_cast<int*>(smem + lay.flag);
  uint32_t* rbase = reinterpret_cast<uint32_t*>(smem + lay.rbase);  // [topk] byte offset of each routed region

  const int W = a.W, H = a.H, C = a.C, S = a.S, R = S * S, topk = a.topk;
  const int L = topk * T;  // a multiple of 64
  const int ntiles = L / 64;

  // XCD-aware numbering: consecutive units (n, r, h, slab) share blockIdx %
  // 8, so the slabs and heads of a region -- the same K/V cache lines -- are
  // read through one XCD's L2. (HG > 1: units (n, r, group of HG heads,
  // slab), the head within the group from the wave.)
  const int groups = a.heads / HG;
  const int units = a.N * R * groups * SLABS;
  const int per = (units + 7) / 8;
  const int u = (int)(blockIdx.x % 8) * per + (int)(blockIdx.x / 8);
  if (u >= units) return;  // the whole workgroup leaves together
  const int slab = u % SLABS, hu = u / SLABS;
  const int h = (hu % groups) * HG + hw, nr = hu / groups;
  const int n = nr / R, r = nr - n * R;
  const int jr = r / S, ir = r - jr * S;
  const int y0 = jr * RH + slab * SR, x0 = ir * RW;  // the slab's first query row and column
  const size_t img = (size_t)n * H * W * C;
  const uint32_t img_bytes = (uint32_t)H * W * C * 2;
  const Rsrc qb = rsrc(a.q + img, img_bytes), kb = rsrc(a.k + img, img_bytes);
  const Rsrc vb = rsrc(a.v + img, img_bytes);
  const uint32_t rowb = (uint32_t)W * C * 2, pixb = (uint32_t)C * 2;
  const uint32_t hb = (uint32_t)h * 64;  // byte offset of this head's channels
  const int32_t* rrow = a.route + (size_t)nr * topk;

  // ---- tile loader. A 64-key tile lies inside one routed region (T is a
  // multiple of 64) and starts on a region row: region p = tile * 64 / T,
  // first token tt0 = (tile * 64) % T. Wave w fills the w-th KiB of the K
  // tile and of the V tile with one direct-to-LDS 16-byte load each: lane i
  // lands at byte 16i of the wave's KiB. K: that is slot (x = w, c = i/16,
  // col = i%16), the chunk c of key krow(w, col). V: row 16w + i/4, chunk
  // position i%4, i.e. logical chunk (i%4) ^ swz(row) of that key. The
  // lane's offsets within the region are constant; the region's offset (LDS
  // route table) and the tile's first row are a uniform add.
  uint32_t ld_off_k, ld_off_v;
  {
    const int kk = score_key(wv, lane & 15), kc = lane >> 4;
    ld_off_k = (uint32_t)(kk / RW) * rowb + (uint32_t)(kk % RW) * pixb + hb + (uint32_t)kc * 16;
    const int kr = 16 * wv + (lane >> 2), c = (lane & 3) ^ swz(kr);
    ld_off_v = (uint32_t)(kr / RW) * rowb + (uint32_t)(kr % RW) * pixb + hb + (uint32_t)c * 16;
  }
  auto issue = [&](int tile, int buf) {
    const int p = tile * 64 / T, tt0 = tile * 64 - p * T;
    const uint32_t soff = __builtin_amdgcn_readfirstlane(rbase[p]) + (uint32_t)(tt0 / RW) * rowb;
    char* dst = tiles + buf * kBufBytes + wv * 1024;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(kb, (__attribute__((address_space(3))) void*)dst, 16, ld_off_k,
                                             soff, 0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(vb, (__attribute__((address_space(3))) void*)(dst + kTileBytes),
                                             16, ld_off_v, soff, 0, 0);
  };

  // ---- the slab's V halo (rows y0-2 .. y0+SR+1, columns x0-2 .. x0+RW+1,
  // the head's 32 channels) straight into LDS, 64 bytes a pixel: piece
  // j*64 + i (instruction j, lane i) is chunk i%4 of pixel (j*64 + i)/4;
  // pixels outside the image read as zero (the LCE padding). It is issued
  // in the first tile step, behind that step's key loads (a wait for an
  // earlier-issued load would wait for it too), and lands while the keys
  // are walked.
  auto issue_halo = [&]() {
    constexpr int NLOAD = (int)(halo_raw_bytes(SR, RW) / 1024);
    for (int j = wv; j < NLOAD; j += WAVES) {
      const int piece = j * 64 + lane, pix = piece >> 2, ch = piece & 3;
      const int y = y0 - 2 + pix / WP, x = x0 - 2 + pix % WP;
      const uint32_t off = y >= 0 && y < H && x >= 0 && x < W
                               ? (uint32_t)y * rowb + (uint32_t)x * pixb + hb + (uint32_t)ch * 16 : kOut;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vb, (__attribute__((address_space(3))) void*)(raw + j * 1024), 16,
                                               off, 0, 0, 0);
    }
  };
  bool halo_issued = false;

  // ---- queries: this wave's blocks (B operands) -- issued first, they are
  // on the path to the first product
  bf16x8 bq[QBW];
#pragma unroll
  for (int i = 0; i < QBW; ++i) {
    const int t = (wv * QBW + i) * 16 + col;
    bq[i] = as_bf16x8(ld16(qb, (uint32_t)(y0 + t / RW) * rowb + (uint32_t)(x0 + t % RW) * pixb + hb + grp * 16));
  }
  // ---- the key norms of the image's regions for this head (R <= 64:
  // region lane in lane lane), loaded before the routes are known: the bound
  // over the routed regions is then a lane shuffle, not a load that waits
  // for the routes (larger images load the routed regions' norms after
  // the route row: measured faster there)
  const bool bounded = a.kn != nullptr;
  const bool kn_pre = bounded && R <= 64;
  const float knv = kn_pre && lane < R ? a.kn[((size_t)n * R + lane) * a.heads + h] : 0.f;
  // ---- routes chosen here (region means given, S*S <= 64): region r's
  // logits against every region of its image with the router's split-bf16
  // matrix-core tile (route_common.h: the operands, products and scale of
  // route_kernel, so the same logits bit for bit; wave w takes regions
  // 16w .. 16w+15, its tile's row 0 is region r), then wave 0 ranks the R
  // keys (larger logit first, ties to the lower index) and region r's top-k
  // go to LDS and, from one workgroup of the region, to route_out. With
  // head_routes the logits run over the head's own 32 channels (the same
  // steps as the route kernel over a one-head, 32-channel input) and every
  // head reports its routes. The scratch is the halo staging, unused until
  // the first tile step.
  int32_t* sel = reinterpret_cast<int32_t*>(smem + lay.raw + 256);  // [topk] chosen regions
  if (a.qr) {
    const size_t row = a.head_routes ? ((size_t)n * a.heads + h) * R + r : (size_t)nr;
    route::route_region(a.qr + (size_t)n * R * C, a.kr + (size_t)n * R * C, R, C,
                        a.head_routes ? h * 32 : 0, a.head_routes ? 32 : C, a.rscale, r, topk, wave, lane,
                        reinterpret_cast<float*>(smem + lay.raw), reinterpret_cast<uint64_t*>(smem + lay.raw + 512),
                        sel, slab == 0 && (a.head_routes || h == 0), a.route_out + row * topk);
  }
  // ---- route table -> LDS, and the largest squared key norm over the
  // routed regions: each wave reads the route row and the norms with one
  // load per lane (two dependent loads in all, not two per route)
  float k2 = 0.f;
  for (int p0 = 0; p0 < topk; p0 += 64) {
    const int p = p0 + lane;
    const int s = p < topk ? (a.qr ? sel[p] : rrow[p]) : 0;
    if (p < topk && wave == 0) {
      const int js = s / S, is = s - js * S;
      rbase[p] = (uint32_t)(js * RH) * rowb + (uint32_t)(is * RW) * pixb;
    }
    if (kn_pre) {  // every lane takes part in the shuffle
      const float v = __shfl(knv, s);
      if (p < topk) k2 = fmaxf(k2, v);
    } else if (bounded && p < topk) {
      k2 = fmaxf(k2, a.kn[((size_t)n * R + s) * a.heads + h]);
    }
  }
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) k2 = fmaxf(k2, __shfl_xor(k2, d));
  // weights: [2][15][C] -> this head's [2][15][32]; 240 pieces of 16 bytes
  // (HG > 1: after the key loop, into the freed halo staging)
  if (HG == 1 && tid < 240) {
    const int row = tid >> 3, piece = tid & 7;  // row = parity * 15 + (ay * 3 + j)
    const uint4 w = *reinterpret_cast<const uint4*>(a.wpk + (size_t)row * C + h * 32 + piece * 4);
    *reinterpret_cast<uint4*>(wts + row * 32 + piece * 4) = w;
  }
  // The query enters the products already scaled, q' = bf16(qscale * q),
  // as the walk-through's BRA code scales it before the product: a score is
  // then q'.k in base-2 units. The softmax's fixed maximum of the lane's
  // query is |q'| * max |k| (replaced by the exact maximum on the exact
  // way), and it is the score accumulators' starting value (-m), so the
  // products give s - m and P = 2^(s - m) takes no arithmetic before the
  // exponential.
#pragma unroll
  for (int i = 0; i < QBW; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) bq[i][e] = (__bf16)((float)bq[i][e] * a.qscale);
  float m[QBW];
  {
    const float kmax = __builtin_sqrtf(k2);
#pragma unroll
    for (int i = 0; i < QBW; ++i)
      m[i] = bounded ? __builtin_sqrtf(group_sum(sq8(__builtin_bit_cast(uint4, bq[i])))) * kmax : 0.f;
  }

  f32x4 o0[QBW], o1[QBW], ls[QBW];
  bf16x8 ones;
#pragma unroll
  for (int e = 0; e < 8; ++e) ones[e] = (__bf16)1.0f;

  // K operand of score tile x: slot (x, grp, col), i.e. byte x*1024 + 16*lane
  // V^T operands: this lane gives row 8grp + col/4 (+4) of each 32-key block,
  // channels 4*(col%4) .. +3 of each 16-channel half
  int voff[2][2][2];  // [block b][row +0 / +4][channel half]
#pragma unroll
  for (int b = 0; b < 2; ++b)
#pragma unroll
    for (int rr = 0; rr < 2; ++rr)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const int row = 32 * b + 8 * grp + (col >> 2) + 4 * rr;
        const int chn = 16 * hh + 4 * (col & 3);  // first of the 4 channels
        voff[b][rr][hh] = tile_off(row, chn >> 3) + (chn & 7) * 2;
      }

  // One pass over all tiles. MAXPASS: each lane's largest raw score into
  // smax (no exponentials); otherwise the softmax pass with maximum m.
  float smax[QBW];
  auto pass = [&](auto maxpass_tag) {
    constexpr bool MAXPASS = decltype(maxpass_tag)::value;
#pragma unroll
    for (int i = 0; i < QBW; ++i) {
      o0[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      o1[i] = o0[i];
      ls[i] = o0[i];
      smax[i] = -INFINITY;
    }
    __syncthreads();  // nobody reads the tile buffers any more
    issue(0, 0);
    for (int t = 0; t < ntiles; ++t) {
      // this wave's share of tile t has landed and every LDS read of this
      // wave has returned (so tile t - 1's buffer may be refilled once all
      // waves pass the barrier)
      __builtin_amdgcn_s_waitcnt(kVmcnt0);
      tile_barrier();
      const char* kt = tiles + (t & 1) * kBufBytes;
      const char* vt = kt + kTileBytes;
      bf16x8 ka[4], va0[2], va1[2];
#pragma unroll
      for (int x = 0; x < 4; ++x) ka[x] = as_bf16x8(*reinterpret_cast<const uint4*>(kt + x * 1024 + lane * 16));
      if constexpr (!MAXPASS) {
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          // keys 32b + 8grp .. +7 of channel col (va0) and 16 + col (va1)
          va0[b] = cat(ld_tr(vt + voff[b][0][0]), ld_tr(vt + voff[b][1][0]));
          va1[b] = cat(ld_tr(vt + voff[b][0][1]), ld_tr(vt + voff[b][1][1]));
        }
      }
      // the next tile goes into the other buffer (tile t - 1's) only after
      // this tile's operands are read: the compiler makes an LDS read wait
      // for every load into LDS issued before it
      if (t + 1 < ntiles) issue(t + 1, (t + 1) & 1);
      if (!halo_issued) {
        issue_halo();
        halo_issued = true;
      }
      if constexpr (MAXPASS) {
#pragma unroll
        for (int i = 0; i < QBW; ++i) {
          const f32x4 z = {0.f, 0.f, 0.f, 0.f};
          f32x4 s[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) s[x] = mfma(ka[x], bq[i], z);
          const float c0 = max3(s[0][0], s[0][1], s[0][2]), c1 = max3(s[0][3], s[1][0], s[1][1]);
          const float c2 = max3(s[1][2], s[1][3], s[2][0]), c3 = max3(s[2][1], s[2][2], s[2][3]);
          const float c4 = max3(s[3][0], s[3][1], s[3][2]);
          smax[i] = max3(smax[i], max3(c0, c1, c2), max3(c3, c4, s[3][3]));
        }
      } else {
#pragma unroll
        for (int i = 0; i < QBW; ++i) {
          const f32x4 mi = {-m[i], -m[i], -m[i], -m[i]};  // the lane's four scores are of one query
          f32x4 s[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) s[x] = mfma(ka[x], bq[i], mi);
          bf16x4 pb[4];
#pragma unroll
          for (int x = 0; x < 4; ++x) {
            f32x4 pv;
#pragma unroll
            for (int e = 0; e < 4; ++e) pv[e] = __builtin_amdgcn_exp2f(s[x][e]);
            pb[x] = to_bf16x4(pv);
          }
#pragma unroll
          for (int b = 0; b < 2; ++b) {
            const bf16x8 pt = cat(pb[2 * b], pb[2 * b + 1]);  // keys 32b + 8g .. 32b + 8g + 7
            o0[i] = mfma(va0[b], pt, o0[i]);
            o1[i] = mfma(va1[b], pt, o1[i]);
            ls[i] = mfma(ones, pt, ls[i]);
          }
        }
      }
    }
  };

  bool exact = !bounded;
  if (bounded) {
    pass(SoftTag{});
    // did some query's largest P underflow (its maximum far under the bound)?
    bool low = false;
#pragma unroll
    for (int i = 0; i < QBW; ++i) low |= !(ls[i][0] >= kUnderflow);
    if (tid == 0) *flag = 0;
    __syncthreads();
    if (__builtin_amdgcn_ballot_w64(low) != 0 && lane == 0) *flag = 1;
    __syncthreads();
    exact = *flag != 0;
  }
  if (exact) {
    pass(MaxTag{});
#pragma unroll
    for (int i = 0; i < QBW; ++i) m[i] = group_max(smax[i]);
    pass(SoftTag{});
  }
  __syncthreads();  // every wave is done with the tile buffers: the halo goes there
  uint4 wreg = {0u, 0u, 0u, 0u};
  if (HG > 1 && htid < 240)
    wreg = *reinterpret_cast<const uint4*>(a.wpk + (size_t)(htid >> 3) * C + h * 32 + (htid & 7) * 4);

  // ---- the halo as horizontal pixel pairs of the head's 32 channels (the
  // raw halo landed before the second tile's barrier, or before the
  // barrier above when there is one tile)
  __builtin_amdgcn_s_waitcnt(kVmcnt0);
  __syncthreads();
  {
    constexpr int NSLOT = HP * NPAIR;
    for (int e = htid; e < NSLOT * 4; e += NT) {
      const int pp = e >> 2, ch = e & 3;
      const int pr = pp % NPAIR, py = pp / NPAIR;
      const char* src = raw + (py * WP + 2 * pr) * 64 + ch * 16;
      const uint4 va = *reinterpret_cast<const uint4*>(src);
      const uint4 vb2 = *reinterpret_cast<const uint4*>(src + 64);
      uint4 lo, hi;
      lo.x = (va.x & 0xffffu) | (vb2.x << 16); lo.y = (va.x >> 16) | (vb2.x & 0xffff0000u);
      lo.z = (va.y & 0xffffu) | (vb2.y << 16); lo.w = (va.y >> 16) | (vb2.y & 0xffff0000u);
      hi.x = (va.z & 0xffffu) | (vb2.z << 16); hi.y = (va.z >> 16) | (vb2.z & 0xffff0000u);
      hi.z = (va.w & 0xffffu) | (vb2.w << 16); hi.w = (va.w >> 16) | (vb2.w & 0xffff0000u);
      uint32_t* dst = halo + (size_t)pp * 32 + 8 * ch;
      *reinterpret_cast<uint4*>(dst) = lo;
      *reinterpret_cast<uint4*>(dst + 4) = hi;
    }
  }
  __syncthreads();
  if constexpr (HG > 1) {  // the weights into the head's freed halo staging
    if (htid < 240) *reinterpret_cast<uint4*>(wts + (htid >> 3) * 32 + (htid & 7) * 4) = wreg;
    __syncthreads();
  }
  // WO: the output projection's A operands, loaded now so that they land
  // during the LCE: rows 32h + 16 ot + col of wo, input channels of head g in
  // the B operand's order (4 grp .. +3, then 16 + 4 grp .. +3)
  uint2 wa[WO ? 2 : 1][HG][2];
  if constexpr (WO) {
#pragma unroll
    for (int ot = 0; ot < 2; ++ot)
#pragma unroll
      for (int g = 0; g < HG; ++g) {
        const uint16_t* wrow = a.wo + (size_t)(32 * h + 16 * ot + col) * C + 32 * g + 4 * grp;
        wa[ot][g][0] = *reinterpret_cast<const uint2*>(wrow);
        wa[ot][g][1] = *reinterpret_cast<const uint2*>(wrow + 16);
      }
  }

  // ---- LCE + merge + store: lane = (query col, channel group grp); the
  // lane's query rows i = 0..QBW-1 are stacked in one column when RW == 16
  // (one query otherwise), so each halo row is read once for all of them
  const uint32_t* w32 = wts;
  static_assert(QBW == 1 || RW == 16, "stacked queries need 16-token rows");
  const int t0 = wv * QBW * 16 + col;
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
  // regroup (lo: channels 4grp..+3, hi: 16+4grp..+3 of the head slice) so
  // lane group g holds channels 8g .. 8g+7 (the 32-lane swap of (lo, hi)
  // gives (lo0, lo1, hi0, hi1) / (lo2, lo3, hi2, hi3) by group, the 16-lane
  // swap (lo0, lo2, hi0, hi2) / (lo1, lo3, hi1, hi3)), so the token's 64
  // bytes of the slice leave in one 16-byte-per-lane store
  const Rsrc ob = rsrc(a.out + img, img_bytes);
  auto store_slice = [&](uint2 lo, uint2 hi, int ty) {
    const uint32_t la[2] = {lo.x, lo.y}, hb[2] = {hi.x, hi.y};
    uint32_t xs[2], ys[2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const auto h32 = __builtin_amdgcn_permlane32_swap(la[j], hb[j], false, false);
      const auto h16 = __builtin_amdgcn_permlane16_swap(h32[0], h32[1], false, false);
      xs[j] = h16[0];
      ys[j] = h16[1];
    }
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w4 = {xs[0], xs[1], ys[0], ys[1]};
    const uint32_t oo = (uint32_t)(((y0 + ty) * W + x0 + tx) * C + h * 32) * 2;
    __builtin_amdgcn_raw_buffer_store_b128(w4, ob, oo + 16 * grp, 0, kNt);
  };
  uint4 oq[QBW];  // WO: the rounded output, a B operand of the projection
#pragma unroll
  for (int i = 0; i < QBW; ++i) {
    const float inv = 1.0f / ls[i][0];
    uint2 lo, hi;
    lo.x = pack_bf16x2(fmaf(o0[i][0], inv, acc[i][0]), fmaf(o0[i][1], inv, acc[i][1]));
    lo.y = pack_bf16x2(fmaf(o0[i][2], inv, acc[i][2]), fmaf(o0[i][3], inv, acc[i][3]));
    hi.x = pack_bf16x2(fmaf(o1[i][0], inv, acc[i][4]), fmaf(o1[i][1], inv, acc[i][5]));
    hi.y = pack_bf16x2(fmaf(o1[i][2], inv, acc[i][6]), fmaf(o1[i][3], inv, acc[i][7]));
    if constexpr (!WO)
      store_slice(lo, hi, ty0 + i);
    else
      oq[i] = make_uint4(lo.x, lo.y, hi.x, hi.y);
  }
  if constexpr (WO) {
    // ---- output projection: y^T (32 output channels of head h's slice x
    // 16 queries) = sum over heads g of Wo[:, head g] . o_g^T, the o_g of
    // the same queries from the exchange (wave wv of every head holds the
    // same queries)
    auto xch = [&](int g, int i) {
      return reinterpret_cast<uint4*>(smem + g * lay.head + lay.xch) + (wv * QBW + i) * 64 + lane;
    };
#pragma unroll
    for (int i = 0; i < QBW; ++i) *xch(hw, i) = oq[i];
    __syncthreads();
    f32x4 ya[2][QBW];
#pragma unroll
    for (int ot = 0; ot < 2; ++ot)
#pragma unroll
      for (int i = 0; i < QBW; ++i) ya[ot][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int g = 0; g < HG; ++g) {
      bf16x8 ob8[QBW];
#pragma unroll
      for (int i = 0; i < QBW; ++i) ob8[i] = as_bf16x8(*xch(g, i));
#pragma unroll
      for (int ot = 0; ot < 2; ++ot) {
        const bf16x8 av = as_bf16x8(make_uint4(wa[ot][g][0].x, wa[ot][g][0].y, wa[ot][g][1].x, wa[ot][g][1].y));
#pragma unroll
        for (int i = 0; i < QBW; ++i) ya[ot][i] = mfma(av, ob8[i], ya[ot][i]);
      }
    }
    // bias of the lane's output channels (no bias: zeros), round, store
    const Rsrc bb = rsrc(a.bo, a.bo ? (uint32_t)C * 2 : 0u);
    const uint32_t boff = (uint32_t)(h * 32 + 4 * grp) * 2;
    const uint32_t bw[4] = {__builtin_amdgcn_raw_buffer_load_b32(bb, boff, 0, 0),
                            __builtin_amdgcn_raw_buffer_load_b32(bb, boff + 4, 0, 0),
                            __builtin_amdgcn_raw_buffer_load_b32(bb, boff + 32, 0, 0),
                            __builtin_amdgcn_raw_buffer_load_b32(bb, boff + 36, 0, 0)};
    const float bias[8] = {bf16_lo(bw[0]), bf16_hi(bw[0]), bf16_lo(bw[1]), bf16_hi(bw[1]),
                           bf16_lo(bw[2]), bf16_hi(bw[2]), bf16_lo(bw[3]), bf16_hi(bw[3])};
#pragma unroll
    for (int i = 0; i < QBW; ++i) {
      uint2 lo, hi;
      lo.x = pack_bf16x2(ya[0][i][0] + bias[0], ya[0][i][1] + bias[1]);
      lo.y = pack_bf16x2(ya[0][i][2] + bias[2], ya[0][i][3] + bias[3]);
      hi.x = pack_bf16x2(ya[1][i][0] + bias[4], ya[1][i][1] + bias[5]);
      hi.y = pack_bf16x2(ya[1][i][2] + bias[6], ya[1][i][3] + bias[7]);
      store_slice(lo, hi, ty0 + i);
    }
  }
}

template <int RH, int RW, int HG, bool WO>
hipError_t launch_t(const TileArgs& a, hipStream_t st) {
  const int units = a.N * a.S * a.S * (a.heads / HG) * tile_slabs<RH, RW>();
  const unsigned blocks = (unsigned)(((units + 7) / 8) * 8);
  constexpr int threads = 64 * kTileWaves * HG;
  launch((attn_tile_kernel<RH, RW, HG, WO>), dim3(blocks), dim3(threads),
         tile_lds(RH / tile_slabs<RH, RW>(), RW, a.topk, HG, tile_qbw<RH, RW>()).total, st, a);
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
  const int qbw = s.rw == 16 ? 2 : 1, slabs = s.rh * s.rw / (16 * kTileWaves * qbw);
  return tile_lds(s.rh / slabs, s.rw, s.topk, 1, qbw).total <= 65536;
}

// Can the kernel choose the routes itself (from the region means)?
bool tile_kernel_routes(const Shape& s) { return s.R <= 64; }

namespace {
// 16x16 regions routed in the kernel (one set of routes for all heads): the
// two heads of a pair in one workgroup, which routes the region once for
// both (measured faster than a workgroup per head)
bool tile_head_pairs(const Shape& s, bool routed_here, bool head_routes) {
  return s.rh == 16 && s.rw == 16 && routed_here && !head_routes && s.heads % 2 == 0 &&
         tile_lds(8, 16, s.topk, 2, 2).total <= 65536;
}
}  // namespace


// The block's attention + output projection: every head of a region in one
// workgroup (two heads of 32 channels; 8x8 or 16x16 regions), routes chosen
// in the kernel (S*S <= 64).
bool tile_block_supports(const Shape& s) {
  if (s.hd != 32 || s.heads != 2 || !tile_kernel_routes(s)) return false;
  const int code = s.rh * 64 + s.rw;
  if (code != 8 * 64 + 8 && code != 16 * 64 + 16) return false;
  if ((long long)s.H * s.W * s.C >= (1ll << 30)) return false;
  const int qbw = s.rw == 16 ? 2 : 1, slabs = s.rh * s.rw / (16 * kTileWaves * qbw);
  return tile_lds(s.rh / slabs, s.rw, s.topk, 2, qbw).total <= 65536;
}

hipError_t launch_attend_tile_block(const void* q, const void* k, const void* v, const uint32_t* wpk,
                                    const void* b, const float* qr, const float* kr, int32_t* route_out,
                                    const float* kn, const void* wo, const void* bo, const Shape& s, void* y,
                                    hipStream_t st) {
  TileArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.wpk = wpk; a.b = (const uint16_t*)b; a.route = route_out; a.kn = kn; a.out = (uint16_t*)y;
  a.wo = (const uint16_t*)wo; a.bo = (const uint16_t*)bo;
  a.qr = qr; a.kr = kr; a.route_out = route_out;
  a.head_routes = 0;
  a.rscale = (float)(1.0 / __builtin_sqrt((double)s.C));
  a.N = s.N; a.H = s.H; a.W = s.W; a.C = s.C; a.heads = s.heads; a.S = s.S; a.topk = s.topk;
  a.qscale = (float)(1.4426950408889634 / __builtin_sqrt((double)s.hd));
  switch (s.rh * 64 + s.rw) {
    case 8 * 64 + 8: return launch_t<8, 8, 2, true>(a, st);
    case 16 * 64 + 16: return launch_t<16, 16, 2, true>(a, st);
    default: return hipErrorInvalidValue;
  }
}

// Routes: given (route), or, with qr and kr (the region means; S*S <= 64),
// chosen in the kernel and written to route_out -- per head with
// head_routes (route_out [N][heads][S*S][topk]).
hipError_t launch_attend_tile(const void* q, const void* k, const void* v, const uint32_t* wpk,
                              const void* b, const int32_t* route, const float* kn, const Shape& s,
                              void* out, hipStream_t st, const float* qr, const float* kr,
                              int32_t* route_out, bool head_routes) {
  TileArgs a;
  a.q = (const uint16_t*)q; a.k = (const uint16_t*)k; a.v = (const uint16_t*)v;
  a.wpk = wpk; a.b = (const uint16_t*)b; a.route = route; a.kn = kn; a.out = (uint16_t*)out;
  a.wo = nullptr; a.bo = nullptr;
  a.qr = qr; a.kr = kr; a.route_out = route_out;
  a.head_routes = head_routes ? 1 : 0;
  a.rscale = (float)(1.0 / __builtin_sqrt((double)(head_routes ? s.hd : s.C)));
  a.N = s.N; a.H = s.H; a.W = s.W; a.C = s.C; a.heads = s.heads; a.S = s.S; a.topk = s.topk;
  a.qscale = (float)(1.4426950408889634 / __builtin_sqrt((double)s.hd));
  if (tile_head_pairs(s, qr != nullptr, head_routes)) return launch_t<16, 16, 2, false>(a, st);
  switch (s.rh * 64 + s.rw) {
    case 8 * 64 + 8: return launch_t<8, 8, 1, false>(a, st);
    case 16 * 64 + 16: return launch_t<16, 16, 1, false>(a, st);
    case 8 * 64 + 16: return launch_t<8, 16, 1, false>(a, st);
    case 16 * 64 + 8: return launch_t<16, 8, 1, false>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace bra
