/*
 * bra.h -- C ABI of the MI355X (gfx950) Bi-Level Routing Attention forward pass.
 *
 * The operation is the BRA operator of BiFormer as walked through at
 * TRANSFORMER.niftyadmin.cn/n/347023.html, section "BRA模块" (Algorithm 1 and
 * Eqs. 3-7 of the paper, whose code survives on that page), and summarised on
 * bernice.tw/posts/biformer, section "Bi-Level Routing Attention":
 *
 *   1. partition the (H, W) map into S x S regions of T = (H/S)(W/S) tokens;
 *      region r = j*S + i (j along H), tokens row-major inside a region;
 *   2. Q^r, K^r = per-region means of q and k over the region's tokens;
 *   3. A = (Q^r * C^-1/2) K^r^T, an S^2 x S^2 region affinity (Eq. 4);
 *   4. route_idx = per-row indices of the topk largest A, descending, exact
 *      ties to the lower region index (Eq. 5);
 *   5. each query region gathers the tokens of its routed regions (Eq. 6);
 *   6. per head (channels [h*hd, (h+1)*hd), hd = C/heads), softmax attention
 *      of the region's queries over all topk*T gathered keys, scale hd^-1/2
 *      (Eq. 7, first term);
 *   7. LCE(V): 5x5 depthwise cross-correlation of v over the whole image,
 *      zero padding 2, plus bias (Eq. 7, second term; the Conv2d(C, C, 5,
 *      padding=2, groups=C) of the module print);
 *   8. out = attention + LCE, rounded once to the storage dtype.
 *
 * The query/key/value projections and the output projection that surround
 * the operator in BiFormer are not part of this call: q, k, v are inputs.
 *
 * Conventions for every entry point
 *   - Tensor pointers are caller-owned DEVICE pointers (hipMalloc'd or a
 *     framework tensor's data pointer) of contiguous arrays. Host pointers are
 *     rejected with BRA_ERR_POINTER. q, k, v, out, lce_w and the fp32 region
 *     means must be 16-byte aligned, lce_b and route_idx 4-byte aligned
 *     (BRA_ERR_ALIGN otherwise).
 *   - q, k, v, out are NHWC: [N][H][W][C] of `dtype`.
 *   - lce_w is [C][5][5] of `dtype` (a depthwise Conv2d weight (C,1,5,5)
 *     flattened); lce_b is [C] of `dtype`, or NULL for a zero bias.
 *   - route_idx is int32 [N][S*S][topk], each row in descending-affinity order.
 *   - Outputs must not alias inputs.
 *   - Work is enqueued asynchronously on the stream set by bra_set_stream
 *     (per host thread; the null stream by default). No entry point
 *     synchronises the device; kernel faults surface at the caller's next
 *     synchronisation.
 *   - Every argument check runs before any launch. On a non-zero return no
 *     work was enqueued (except BRA_ERR_HIP, which reports a failed launch or
 *     allocation) and the outputs are untouched.
 *
 * Compiled envelope: head_dim = C/heads = 32 (every BiFormer stage), C <=
 * 1024, S*S <= 1024, topk * T <= 65536. Outside it the calls return
 * BRA_ERR_UNSUPPORTED.
 */
#ifndef BRA_H_
#define BRA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum bra_dtype {
  BRA_F32 = 0,  /* IEEE binary32 */
  BRA_BF16 = 1  /* bfloat16 (attention products on bf16 matrix cores) */
};

enum bra_status {
  BRA_OK = 0,
  BRA_ERR_NULL = -1,        /* a required pointer is NULL */
  BRA_ERR_SHAPE = -2,       /* a size <= 0, H % S, W % S or C % heads != 0 */
  BRA_ERR_TOPK = -3,        /* topk outside [1, S*S] */
  BRA_ERR_DTYPE = -4,       /* unknown dtype */
  BRA_ERR_UNSUPPORTED = -5, /* outside the compiled envelope (see above) */
  BRA_ERR_HIP = -6,         /* a HIP launch or allocation failed */
  BRA_ERR_POINTER = -7,     /* a tensor pointer is not device memory */
  BRA_ERR_ALIGN = -8,       /* a tensor pointer is misaligned (see above) */
  BRA_ERR_SCRATCH = -9      /* bra_forward_noalloc: workspace beyond its static array */
};

/* The whole forward pass, steps 1-8 above.
 * Uses a library-owned fp32 workspace of bra_workspace_bytes(N, C, S) bytes
 * per device (grow-only, allocated on first need, freed by bra_release).
 * Calls on one device that use the library workspace must not overlap: the
 * library serialises them on the host, but two streams would race on the
 * device. */
int bra_forward(const void* q, const void* k, const void* v,
                const void* lce_w, const void* lce_b,
                int N, int H, int W, int C, int heads, int S, int topk,
                int dtype, void* out, int32_t* route_idx);

/* bra_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, hosts that forbid allocation):
 * same arguments, checks, results and routes as bra_forward, but the
 * workspace is a static device array of BRA_NOALLOC_SCRATCH_BYTES (16 MiB)
 * that each device the library runs on holds until the process ends. The
 * call never allocates or frees memory (no hipMalloc, hipFree or allocating
 * library routine) and records no profiling events. Shapes whose workspace
 * (bra_workspace_bytes) exceeds the array return BRA_ERR_SCRATCH before any
 * launch; shapes that run as one kernel need no workspace at all. All calls
 * on one device share that device's array and nothing serialises them on
 * the device: calls that overlap on one GPU (two streams, or two host
 * threads) race on it and give undefined results. Every kernel writes the
 * scratch it later reads, so nothing needs clearing between calls. */
#define BRA_NOALLOC_SCRATCH_BYTES (16u << 20)
int bra_forward_noalloc(const void* q, const void* k, const void* v,
                        const void* lce_w, const void* lce_b,
                        int N, int H, int W, int C, int heads, int S, int topk,
                        int dtype, void* out, int32_t* route_idx);

/* Backward of the operator for given routes (training): gradients of
 * sum(out * dout) with respect to q, k, v (same layout and dtype as the
 * inputs), the LCE weights (dlce_w, fp32 [C][25]) and the LCE bias (dlce_b,
 * fp32 [C], or NULL to skip). The walk-through (section BRA模块) detaches the
 * router, so route_idx -- the forward's routes, int32 [N][S*S][topk], every
 * entry in [0, S*S) (not checked on the device) -- is an input and gets no
 * gradient. For query region r with gathered keys/values K, V and rows G of
 * dout: dS = P * (G V^T - rowsum(G * O)), dQ = hd^-1/2 dS K, and each routed
 * region collects hd^-1/2 dS^T Q into dk and P^T G into dv; LCE adds dout
 * correlated with the flipped 5x5 kernel to dv, dlce_w[c][a*5+e] = sum over
 * pixels of dout * v shifted by (a-2, e-2), dlce_b[c] = sum of dout.
 * Every gradient is a fixed-order sum (bit-reproducible). bf16 only, with
 * regions of a multiple of 16 tokens and topk <= 16 (else
 * BRA_ERR_UNSUPPORTED). Uses the library workspace; alignment as for
 * bra_forward (dout, dq, dk, dv 16 bytes; dlce_w, dlce_b 4 bytes). */
int bra_backward(const void* q, const void* k, const void* v, const void* lce_w,
                 const int32_t* route_idx, const void* dout,
                 int N, int H, int W, int C, int heads, int S, int topk, int dtype,
                 void* dq, void* dk, void* dv, float* dlce_w, float* dlce_b);

/* The per-head routing variant (the qqiyuan.cn blog's BRA class routes
 * every head on its own channels, section on region-level routing): for
 * head h, steps 2-4 run on channels [h*32, h*32+32) alone -- region means of
 * that slice, A_h = (Q^r_h * 32^-1/2) K^r_h^T (the class scales by
 * head_dim^-1/2), top-k with the same order and tie rule -- and head h
 * gathers its own routed regions; the joint softmax, LCE and merge are as in
 * bra_forward. route_idx is int32 [N][heads][S*S][topk]. Same tensor
 * conventions and checks as bra_forward. Runs the operator once per head on
 * head-major copies of q, k, v (library workspace: 4 copies of the tensor,
 * the per-head routes and one head's bra_forward workspace). */
int bra_forward_head_routed(const void* q, const void* k, const void* v,
                            const void* lce_w, const void* lce_b,
                            int N, int H, int W, int C, int heads, int S, int topk,
                            int dtype, void* out, int32_t* route_idx);

/* The router-free attention of BiFormer's last stage (AttentionLePE; the
 * walk-through's module print, section 网络结构, and bernice.tw/posts/biformer,
 * section "Biformer", which gives that stage k = S^2): per image and head,
 * softmax attention of every query over all H*W tokens of its image, scale
 * hd^-1/2, plus LCE(V) as in step 7, rounded once. Equal to bra_forward with
 * every region routed (topk = S*S) for any S, without the routing. Same
 * tensor conventions and checks as bra_forward (no S, topk or route_idx).
 * bf16 maps of at most 256 tokens (7x7 .. 16x16) run one kernel; other
 * shapes run the routed path with a single region (S = 1), in the library
 * workspace. */
int bra_attention_dense(const void* q, const void* k, const void* v,
                        const void* lce_w, const void* lce_b,
                        int N, int H, int W, int C, int heads, int dtype, void* out);

/* Step 2 alone: qr, kr = region means of q and k, fp32 [N][S*S][C] each
 * (caller-owned device buffers). Same checks as bra_forward (heads and topk
 * are not involved). The means are bit-identical to the ones bra_forward
 * routes on (the same kernel), so bra_route(bra_region_means(...)) reproduces
 * its routes. */
int bra_region_means(const void* q, const void* k, int N, int H, int W, int C,
                     int S, int dtype, float* qr, float* kr);

/* Steps 3-4 alone: route_idx [N][R][topk] from fp32 region means qr, kr
 * [N][R][C] (R = S*S, R <= 1024). */
int bra_route(const float* qr, const float* kr, int N, int R, int C, int topk,
              int32_t* route_idx);

/* Steps 5-8 with given routes: out = attention over the regions listed in
 * route_idx [N][S*S][topk] (device, int32, every entry in [0, S*S); entries
 * are not checked on the device and an index outside that range is undefined
 * behaviour) plus LCE. */
int bra_attend(const void* q, const void* k, const void* v,
               const void* lce_w, const void* lce_b, const int32_t* route_idx,
               int N, int H, int W, int C, int heads, int S, int topk,
               int dtype, void* out);

/* Step 7 alone: LCE(v) into a caller-owned fp32 buffer [N][H][W][C]. */
int bra_lce(const void* v, const void* lce_w, const void* lce_b,
            int N, int H, int W, int C, int dtype, float* out);

/* The Linear layers around the operator: y = x w^T + b over the channels of
 * every token (the walk-through TRANSFORMER.niftyadmin.cn/n/347023.html,
 * section BRA模块: one Linear(C, 3C) gives q, k and v, split in that order,
 * and the output Linear(C, C), wo, follows attention + LCE; section 网络结构
 * prints them as Linear(64, 192) and Linear(64, 64)).
 * x: [M][K] row-major (M tokens of K channels), w: [Nout][K] row-major (the
 * Linear weight as stored), b: [Nout] or NULL (no bias); all device memory
 * of dtype, owned by the caller. Output feature f goes to part p = f / split
 * at column f - p*split: y0, y1, y2 are row-major [M][split] each, and
 * Nout = split * parts with 1 <= parts <= 3 (y1 / y2 are ignored, and may be
 * NULL, when unused). bf16 runs on the matrix cores with fp32 accumulation
 * and rounds y to nearest even; f32 accumulates with fma in k order.
 * The outputs must not alias x, w or b (they are written while x is still
 * being read by other workgroups).
 * Requires K % 32 == 0, split % 8 == 0 and, for bf16, K <= 256 (else
 * BRA_ERR_UNSUPPORTED), and
 * x and w each under 2 GiB. x, w and the outputs must be 16-byte aligned and
 * b 4-byte aligned (BRA_ERR_ALIGN). Errors: BRA_ERR_NULL
 * for a missing x, w or used output, BRA_ERR_SHAPE for sizes <= 0 or Nout not
 * 1-3 times split, BRA_ERR_DTYPE, BRA_ERR_POINTER, BRA_ERR_HIP. */
int bra_linear(const void* x, const void* w, const void* b, int M, int K, int Nout, int split,
               int dtype, void* y0, void* y1, void* y2);

/* The BRA block around the operator (the walk-through at
 * TRANSFORMER.niftyadmin.cn/n/347023.html, section BRA模块: one Linear(C, 3C)
 * whose output splits into q, k, v in that order along the channels, the
 * operator, then wo = Linear(C, C); its module print in section 网络结构
 * shows both layers):
 *   q, k, v = split(x . w_qkv^T + b_qkv),  o = bra_forward(q, k, v, ...),
 *   y = o . w_o^T + b_o.
 * x, y: [N][H][W][C] in dtype; w_qkv: [3C][C] and w_o: [C][C] as a Linear
 * layer stores them (output feature, input feature); b_qkv [3C], b_o [C],
 * each may be NULL (no bias); lce_w, lce_b, heads, S, topk as bra_forward;
 * route_idx [N][S*S][topk] int32 receives the routes. q, k, v and o are held
 * in dtype between the steps (bf16: rounded to nearest even), as separate
 * bra_linear / bra_forward calls would store them, so the result equals that
 * chain's up to the order of fp32 sums.
 * bf16 shapes that bra_forward runs on its large-region kernel with two heads
 * and regions of 8x8 or 16x16 tokens run fused (bra_block_fused): the qkv
 * projection also writes the region means and key norms that routing needs
 * (no pass re-reads q and k), and the attention kernel, with both heads of a
 * region in one workgroup, applies w_o and b_o before it stores. Other shapes
 * run the three steps as bra_linear and bra_forward do.
 * Workspace: the library's own (allocated or grown on first need, kept until
 * bra_release), 4 * N*H*W*C * sizeof(dtype) bytes (256-byte aligned parts)
 * plus bra_workspace_bytes(N, C, S); y and route_idx must not alias it, x,
 * the weights or each other. Requires C <= 256 for bf16 and x under 2 GiB
 * (else BRA_ERR_UNSUPPORTED), plus bra_forward's envelope. Alignment: x, the
 * weights, lce_w and y 16 bytes, biases and route_idx 4 bytes (BRA_ERR_ALIGN).
 * Errors: those of bra_forward and bra_linear. */
int bra_block_forward(const void* x, const void* w_qkv, const void* b_qkv, const void* lce_w,
                      const void* lce_b, const void* w_o, const void* b_o, int N, int H, int W,
                      int C, int heads, int S, int topk, int dtype, void* y, int32_t* route_idx);

/* 1 if bra_block_forward runs these sizes on its fused path, else 0 (also
 * for invalid sizes). */
int bra_block_fused(int N, int H, int W, int C, int heads, int S, int topk, int dtype);

/* Stream used by every later call from this host thread (a hipStream_t;
 * NULL = the null stream). Always returns BRA_OK. */
int bra_set_stream(void* stream);
void* bra_get_stream(void);

/* Bytes of library workspace bra_forward needs: two fp32 [N][S*S][C]
 * arrays (region means), the largest squared key norm per (image, region,
 * head of 32 channels) (fp32 [N][S*S][C/32]), then 490*C bytes of LCE
 * weights repacked for the attention kernels (pixel-pair, tap-major and
 * Toeplitz layouts); each part starts 256-byte aligned. Returns 0 for
 * invalid sizes. */
size_t bra_workspace_bytes(int N, int C, int S);

/* Frees the library workspace of every device (synchronises each device
 * that holds one first). The next bra_forward allocates again. */
void bra_release(void);

/* Static text for a status code; for BRA_ERR_HIP it includes the last HIP
 * error seen by this thread. */
const char* bra_error_string(int code);

/* Library version: 100 * major + minor. */
int bra_version(void);

/* Per-kernel timing with HIP events tied to the kernel dispatches.
 * bra_profile_begin(mask) records events around the kernels of every kind k
 * with bit (1 << k) set in mask (BRA_K_* below; up to 4096 launches per kind,
 * later ones are not recorded) and clears earlier records; mask 0 stops
 * recording. bra_profile_read waits for the recorded events, then writes for
 * each kind k < n the summed milliseconds and the launch count, and clears
 * the record. A recorded kernel is launched with hipExtLaunchKernelGGL, whose
 * start and stop events take the time stamps of that kernel's own dispatch
 * (no extra stream commands between kernels).
 * bra_profile_set_mask(mask) changes which kinds are recorded from the next
 * launch on without clearing the record (to sample some launches of a run). */
enum bra_kernel_kind {
  BRA_K_POOL = 0, BRA_K_ROUTE = 1, BRA_K_ATTN = 2, BRA_K_LCE = 3, BRA_K_LINEAR = 4,
  BRA_K_COUNT = 5
};
int bra_profile_begin(int mask);
int bra_profile_set_mask(int mask);
int bra_profile_read(double* ms, int* counts, int n);

/* A plain device-to-device copy kernel (bytes % 16 == 0, both pointers
 * 16-byte aligned), used to calibrate hardware byte counters against a
 * kernel of known traffic. */
int bra_calib_copy(const void* src, void* dst, size_t bytes);

#ifdef __cplusplus
}
#endif

#endif /* BRA_H_ */
