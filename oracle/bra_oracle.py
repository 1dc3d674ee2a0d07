"""Plain fp64 CPU oracle of the Bi-Level Routing Attention (BRA) forward pass.

TEST INFRASTRUCTURE ONLY. This module is the checker the GPU path is compared
against. Only the test suite, the smoke check and the benchmark's CPU-baseline
leg may import it; the product path never does. It shares no code with the
HIP kernels or their host library, and imports nothing from that package.

What it computes follows the walk-through of the authors' code at
TRANSFORMER.niftyadmin.cn/n/347023.html, section "BRA模块" (the equation bodies
of the paper are lost from that page; the code lines it pairs with Eq. 3-7 and
with Algorithm 1 survive), and page bernice.tw/posts/biformer, section
"Bi-Level Routing Attention" (its three parts: region partition, region-to-
region routing, token-to-token attention plus LCE).

Every step is written the plain way, in float64, in the page's order:

1. region partition      "n (j h) (i w) c -> n (j i) h w c"   (Algorithm 1)
2. region means          mean over each region's tokens        (Q^r, K^r)
3. region affinity       A = (Q^r * C^-1/2) @ K^r^T            (Eq. 4)
4. top-k routing         indices of the topk largest A per row (Eq. 5)
5. key/value gather      routed regions' tokens, rank-major    (Eq. 6)
6. token attention       per head softmax(q k^T hd^-1/2) v     (Eq. 7, 1st term)
7. LCE                   5x5 depthwise conv of V, zero pad 2   (Eq. 7, 2nd term)
8. merge                 out = attention + LCE

Readings taken where the pages are silent or garbled (each also listed in the
design notes of the repository):
* routing scale is C^-1/2 and attention scale head_dim^-1/2;
* one routing for all heads (the walk-through's route index has no head axis);
* the routing weights (softmax of the top-k logits) are not applied to the
  gathered keys/values: the gather is a pure index gather;
* top-k order is descending logit, exact ties go to the lower region index;
* the softmax runs jointly over all topk * T gathered keys;
* LCE runs on V over the whole re-assembled image (not per region), with zero
  padding and a bias, as a cross-correlation (no kernel flip), like a
  Conv2d(C, C, 5, padding=2, groups=C);
* H and W must be divisible by S (no padding branch);
* the key/value downsampling hook is the identity and qk_dim = C.

Parity pins for every function live in tests/oracle_pins.py (run by
tests/test_oracle.py).
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "check_shapes", "partition", "unpartition", "region_means",
    "region_affinity", "topk_routes", "gather_regions", "token_attention",
    "lce", "bra_forward", "linear", "round_bf16", "bra_block_forward",
    "dense_attention", "bra_forward_head_routed", "bra_backward",
]


def check_shapes(N, H, W, C, heads, S, topk):
    """Preconditions: the walk-through asserts H % S == 0 and W % S == 0
    (section BRA模块); the head split "(m c)" needs C % heads == 0; top-k needs
    1 <= topk <= S^2."""
    if min(N, H, W, C, heads, S) <= 0:
        raise ValueError("sizes must be positive")
    if H % S or W % S:
        raise ValueError("H and W must be divisible by S")
    if C % heads:
        raise ValueError("C must be divisible by heads")
    if not 1 <= topk <= S * S:
        raise ValueError("topk must lie in [1, S*S]")


def partition(x: np.ndarray, S: int) -> np.ndarray:
    """Algorithm 1 "patchify": (N, H, W, C) -> (N, S*S, (H/S)*(W/S), C).

    Region r = j*S + i, with j the region row (along H) and i the region column;
    inside a region the tokens are row-major, t = y'*(W/S) + x'. This is the
    walk-through's rearrange "n (j h) (i w) c -> n (j i) h w c" followed by
    "n p2 h w c -> n p2 (h w) c"."""
    N, H, W, C = x.shape
    rh, rw = H // S, W // S
    y = x.reshape(N, S, rh, S, rw, C)          # n j h i w c
    y = y.transpose(0, 1, 3, 2, 4, 5)          # n j i h w c
    return y.reshape(N, S * S, rh * rw, C)


def unpartition(xp: np.ndarray, S: int, H: int, W: int) -> np.ndarray:
    """Inverse of `partition`: (N, S*S, T, C) -> (N, H, W, C), the walk-through's
    "(n j i) m (h w) c -> n (j h) (i w) (m c)" without the head axis."""
    N, R, T, C = xp.shape
    rh, rw = H // S, W // S
    y = xp.reshape(N, S, S, rh, rw, C)          # n j i h w c
    y = y.transpose(0, 1, 3, 2, 4, 5)           # n j h i w c
    return y.reshape(N, H, W, C)


def region_means(xp: np.ndarray) -> np.ndarray:
    """Q^r or K^r: for each channel separately, the mean over the T tokens of
    the region; the channels are never averaged together (walk-through,
    section BRA模块, q_win / k_win). (N, R, T, C) -> (N, R, C)."""
    return xp.sum(axis=2) / xp.shape[2]


def region_affinity(qr: np.ndarray, kr: np.ndarray) -> np.ndarray:
    """Eq. 4: A = (Q^r * scale) @ K^r^T with scale = C^-1/2; the routing
    embedding is the identity. (N, R, C) x (N, R, C) -> (N, R, R)."""
    C = qr.shape[-1]
    return (qr * (1.0 / np.sqrt(C))) @ np.swapaxes(kr, -1, -2)


def topk_routes(A: np.ndarray, topk: int) -> np.ndarray:
    """Eq. 5: per row, the indices of the topk largest affinities, in
    descending order of affinity; equal affinities keep the lower region index
    first (a stable sort on the negated key). (N, R, R) -> (N, R, topk) int."""
    order = np.argsort(-A, axis=-1, kind="stable")
    return order[..., :topk].astype(np.int64)


def gather_regions(xp: np.ndarray, route: np.ndarray) -> np.ndarray:
    """Eq. 6: for every query region, the tokens of its routed regions,
    concatenated rank-major, token-minor (the "(k w2)" order of the
    walk-through). (N, R, T, C), (N, R, topk) -> (N, R, topk*T, C)."""
    N, R, T, C = xp.shape
    g = xp[np.arange(N)[:, None, None], route]       # (N, R, topk, T, C)
    return g.reshape(N, R, route.shape[-1] * T, C)


def token_attention(qp: np.ndarray, kg: np.ndarray, vg: np.ndarray, heads: int,
                    return_probs: bool = False):
    """Eq. 7, first term: multi-head softmax attention of each region's
    queries over its gathered keys/values. Head m owns channels
    [m*hd, (m+1)*hd) (the "(m c)" split); scores are (q * hd^-1/2) @ k^T; the
    softmax runs over the last axis, i.e. jointly over all gathered keys.
    qp (N, R, T, C), kg/vg (N, R, L, C) -> (N, R, T, C)."""
    N, R, T, C = qp.shape
    hd = C // heads
    scale = 1.0 / np.sqrt(hd)
    out = np.empty_like(qp)
    probs = [] if return_probs else None
    for m in range(heads):
        sl = slice(m * hd, (m + 1) * hd)
        s = (qp[..., sl] * scale) @ np.swapaxes(kg[..., sl], -1, -2)   # (N,R,T,L)
        s = s - s.max(axis=-1, keepdims=True)
        e = np.exp(s)
        p = e / e.sum(axis=-1, keepdims=True)
        out[..., sl] = p @ vg[..., sl]
        if return_probs:
            probs.append(p)
    if return_probs:
        return out, probs
    return out


def lce(v: np.ndarray, w: np.ndarray, b: np.ndarray | None) -> np.ndarray:
    """Eq. 7, second term, LCE(V): a 5x5 depthwise convolution of V over the
    whole (N, H, W, C) map, stride 1, zero padding 2, plus a per-channel bias
    -- the Conv2d(C, C, kernel_size=5, padding=2, groups=C) of the module
    print (section 网络结构). Cross-correlation orientation:
    l[n,y,x,c] = b[c] + sum_{a,e in 0..4} w[c,a,e] * v[n, y+a-2, x+e-2, c]."""
    N, H, W, C = v.shape
    vp = np.zeros((N, H + 4, W + 4, C))
    vp[:, 2:H + 2, 2:W + 2, :] = v
    out = np.zeros((N, H, W, C))
    for a in range(5):
        for e in range(5):
            out += w[:, a, e] * vp[:, a:a + H, e:e + W, :]
    if b is not None:
        out += b
    return out


def bra_forward(q, k, v, lce_w, lce_b, heads: int, S: int, topk: int,
                route_override: np.ndarray | None = None,
                return_probs: bool = False):
    """The whole forward pass on float64 copies of the inputs.

    q, k, v: (N, H, W, C); lce_w: (C, 5, 5); lce_b: (C,) or None.
    route_override: optional (N, S*S, topk) route indices to use instead of
    the ones this oracle selects (the near-tie protocol feeds the GPU's
    choice back here).
    Returns a dict with "out" (N,H,W,C), "route_idx" (N,R,topk) (the routes
    actually used), "route_oracle" (the oracle's own choice), "logits"
    (N,R,R) and, if asked, "probs" (per image, per head (R,T,L)).

    Images are independent (routing never crosses images), so the attention
    is evaluated one image at a time to bound memory."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, H, W, C = q.shape
    check_shapes(N, H, W, C, heads, S, topk)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    w = np.asarray(lce_w, dtype=np.float64).reshape(C, 5, 5)
    b = None if lce_b is None else np.asarray(lce_b, dtype=np.float64).reshape(C)

    qp, kp, vp = partition(q, S), partition(k, S), partition(v, S)
    A = region_affinity(region_means(qp), region_means(kp))
    route_own = topk_routes(A, topk)
    if route_override is not None:
        route = np.asarray(route_override, dtype=np.int64).reshape(N, S * S, topk)
        if route.min() < 0 or route.max() >= S * S:
            raise ValueError("route_override holds an index outside [0, S*S)")
    else:
        route = route_own

    att = np.empty_like(qp)
    probs = [] if return_probs else None
    for n in range(N):
        kg = gather_regions(kp[n:n + 1], route[n:n + 1])
        vg = gather_regions(vp[n:n + 1], route[n:n + 1])
        res = token_attention(qp[n:n + 1], kg, vg, heads, return_probs)
        if return_probs:
            att[n:n + 1], pr = res
            probs.append([p[0] for p in pr])
        else:
            att[n:n + 1] = res
    out = unpartition(att, S, H, W) + lce(v, w, b)
    res = {"out": out, "route_idx": route, "route_oracle": route_own, "logits": A}
    if return_probs:
        res["probs"] = probs
    return res


def linear(x, w, b=None) -> np.ndarray:
    """A Linear layer over the last axis: y = x w^T + b, in float64.

    x: (..., K); w: (Nout, K) as a Linear layer stores it; b: (Nout,) or None.
    The walk-through (section "BRA模块") projects the tokens with one
    Linear(C, 3C) (its module print in section "网络结构": QKVLinear holding
    Linear(64, 192)) and ends the block with wo = Linear(C, C)."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    y = x @ w.T
    if b is not None:
        y = y + np.asarray(b, dtype=np.float64)
    return y


def round_bf16(x) -> np.ndarray:
    """Rounds to bfloat16 (via float32, then to nearest even on the upper 16
    bits) and returns float64: the storage precision of a bf16 tensor between
    two steps of the block."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16 << 16
    return (u.astype(np.uint32)).view(np.float32).astype(np.float64)


def bra_block_forward(x, wqkv, bqkv, lce_w, lce_b, wo, bo, heads: int, S: int, topk: int,
                      store: str | None = None, route_override=None):
    """The BRA block around the operator, as the walk-through's forward pass
    (section "BRA模块") runs it: q, k, v = split(qkv(x)) in that order along the
    channels, the operator on them (steps 1-8 above), then wo.

    x: (N, H, W, C); wqkv: (3C, C); bqkv: (3C,) or None; wo: (C, C); bo: (C,)
    or None. store="bf16" rounds the tensors handed from one step to the next
    (q, k, v and the operator's output) to bfloat16, as a bf16 pipeline stores
    them; None keeps float64 throughout. Returns the operator's result dict
    with "out" replaced by the block output and "attn_out" added."""
    x = np.asarray(x, dtype=np.float64)
    C = x.shape[-1]
    keep = round_bf16 if store == "bf16" else (lambda t: t)
    qkv = linear(x, wqkv, bqkv)
    q, k, v = (keep(qkv[..., i * C:(i + 1) * C]) for i in range(3))
    res = bra_forward(q, k, v, lce_w, lce_b, heads, S, topk, route_override=route_override)
    o = keep(res["out"])
    res["attn_out"] = o
    res["out"] = linear(o, wo, bo)
    return res


def dense_attention(q, k, v, lce_w, lce_b, heads: int) -> np.ndarray:
    """The router-free attention of the last stage: every query attends to
    every token of its own image, plus the same 5x5 depthwise term on V.

    The walk-through's module print (section "网络结构") shows the last stage
    built from AttentionLePE blocks (a bias-free qkv Linear(C, 3C), a lepe
    Conv2d(C, C, 5, padding=2, groups=C) and a proj Linear), and page
    bernice.tw/posts/biformer, section "Biformer", gives that stage k = S^2:
    all regions routed, i.e. plain attention over the whole map. Per image n
    and head m (channels [m*hd, (m+1)*hd)), with the H*W tokens in raster
    order: o = softmax_u((q_t . k_u) * hd^-1/2) v_u over all u; out = o +
    lce(v). q, k, v: (N, H, W, C); lce_w: (C, 5, 5); lce_b: (C,) or None."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, H, W, C = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    if heads < 1 or C % heads:
        raise ValueError("heads must divide C")
    hd = C // heads
    w = np.asarray(lce_w, dtype=np.float64).reshape(C, 5, 5)
    b = None if lce_b is None else np.asarray(lce_b, dtype=np.float64).reshape(C)
    att = np.empty((N, H * W, C))
    for n in range(N):
        qn, kn, vn = (x[n].reshape(H * W, C) for x in (q, k, v))
        for m in range(heads):
            sl = slice(m * hd, (m + 1) * hd)
            s = (qn[:, sl] @ kn[:, sl].T) / np.sqrt(hd)      # (queries, keys)
            s = s - s.max(axis=1, keepdims=True)
            e = np.exp(s)
            att[n][:, sl] = (e / e.sum(axis=1, keepdims=True)) @ vn[:, sl]
    return att.reshape(N, H, W, C) + lce(v, w, b)


def bra_forward_head_routed(q, k, v, lce_w, lce_b, heads: int, S: int, topk: int,
                            route_override: np.ndarray | None = None):
    """The per-head routing variant: every head routes on its own channels.

    The hand-written BRA class of the qqiyuan.cn blog (its forward, section on
    the region-level routing) splits q and k into heads first and then takes
    region means, region scores (scaled by its self.scale = head_dim^-1/2) and
    the top-k per head, so each head gathers its own regions. This function
    keeps everything else of the operator as bra_forward computes it (joint
    softmax over the gathered keys, LCE on V over the whole image) and changes
    only the routing: for head m (channels [m*hd, (m+1)*hd)), steps 2-6 run
    on that head's channel slice alone -- region_affinity scales by the last
    axis' size^-1/2, which on a head's slice is head_dim^-1/2.
    Returns "out" (N,H,W,C), "route_idx" (N,heads,R,topk) (the routes used),
    "route_oracle" and "logits" (N,heads,R,R). route_override, if given, is
    (N, heads, R, topk)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, H, W, C = q.shape
    check_shapes(N, H, W, C, heads, S, topk)
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v must have the same shape")
    R, hd = S * S, C // heads
    w = np.asarray(lce_w, dtype=np.float64).reshape(C, 5, 5)
    b = None if lce_b is None else np.asarray(lce_b, dtype=np.float64).reshape(C)
    if route_override is not None:
        route_override = np.asarray(route_override, dtype=np.int64).reshape(N, heads, R, topk)
        if route_override.min() < 0 or route_override.max() >= R:
            raise ValueError("route_override holds an index outside [0, S*S)")
    logits = np.empty((N, heads, R, R))
    own = np.empty((N, heads, R, topk), dtype=np.int64)
    used = np.empty_like(own)
    att = np.empty((N, H, W, C))
    for m in range(heads):
        sl = slice(m * hd, (m + 1) * hd)
        qp, kp, vp = partition(q[..., sl], S), partition(k[..., sl], S), partition(v[..., sl], S)
        A = region_affinity(region_means(qp), region_means(kp))
        logits[:, m], own[:, m] = A, topk_routes(A, topk)
        route = own[:, m] if route_override is None else route_override[:, m]
        used[:, m] = route
        o = np.empty_like(qp)
        for n in range(N):
            o[n:n + 1] = token_attention(qp[n:n + 1], gather_regions(kp[n:n + 1], route[n:n + 1]),
                                         gather_regions(vp[n:n + 1], route[n:n + 1]), 1)
        att[..., sl] = unpartition(o, S, H, W)
    return {"out": att + lce(v, w, b), "route_idx": used, "route_oracle": own, "logits": logits}


def bra_backward(q, k, v, lce_w, route, dout, heads: int, S: int):
    """Gradients of bra_forward's output with respect to q, k, v and the LCE
    weights and bias, for given routes.

    The walk-through's router (section "BRA模块") detaches the region means
    before the affinity, so no gradient flows through the routing: the
    routes are fixed indices here, as the forward used them. For image n,
    head m and query region r with gathered keys/values K, V (rank-major, as
    in gather_regions), queries Q and output gradient G (the rows of dout):
      s = hd^-1/2 Q K^T,  P = softmax over each row,  O = P V;
      dP = G V^T,  D = rowsum(P * dP) (= rowsum(G * O)),  dS = P * (dP - D);
      dQ = hd^-1/2 dS K,  dK = hd^-1/2 dS^T Q,  dV = P^T G,
    and the rows of dK, dV are added back to the regions they were gathered
    from (a region routed by several query regions collects all their
    contributions). LCE(v) = b + sum_{a,e} w[c,a,e] v[y+a-2, x+e-2] adds
    dv[y', x'] = sum_{a,e} w[c,a,e] dout[y'-a+2, x'-e+2] (zero outside the
    image), dw[c,a,e] = sum over pixels of dout[y,x,c] v[y+a-2, x+e-2, c] and
    db[c] = sum over pixels of dout[.., c].
    q, k, v, dout: (N, H, W, C); lce_w: (C, 5, 5); route: (N, S*S, topk).
    Returns a dict with dq, dk, dv (N,H,W,C), dlce_w (C,5,5), dlce_b (C,)."""
    q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
    N, H, W, C = q.shape
    route = np.asarray(route, dtype=np.int64)
    topk = route.shape[-1]
    check_shapes(N, H, W, C, heads, S, topk)
    R, hd = S * S, C // heads
    scale = 1.0 / np.sqrt(hd)
    w = np.asarray(lce_w, dtype=np.float64).reshape(C, 5, 5)
    qp, kp, vp, gp = (partition(x, S) for x in (q, k, v, g))
    T = qp.shape[2]
    dqp, dkp, dvp = np.zeros_like(qp), np.zeros_like(kp), np.zeros_like(vp)
    for n in range(N):
        for m in range(heads):
            sl = slice(m * hd, (m + 1) * hd)
            for r in range(R):
                Q, G = qp[n, r, :, sl], gp[n, r, :, sl]
                Kg = np.concatenate([kp[n, s, :, sl] for s in route[n, r]])
                Vg = np.concatenate([vp[n, s, :, sl] for s in route[n, r]])
                sc = (Q @ Kg.T) * scale
                P = np.exp(sc - sc.max(axis=1, keepdims=True))
                P /= P.sum(axis=1, keepdims=True)
                dP = G @ Vg.T
                dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
                dqp[n, r, :, sl] += scale * (dS @ Kg)
                dK, dV = scale * (dS.T @ Q), P.T @ G
                for i, s in enumerate(route[n, r]):
                    dkp[n, s, :, sl] += dK[i * T:(i + 1) * T]
                    dvp[n, s, :, sl] += dV[i * T:(i + 1) * T]
    dq, dk, dv = (unpartition(x, S, H, W) for x in (dqp, dkp, dvp))
    gpad = np.zeros((N, H + 4, W + 4, C))
    gpad[:, 2:H + 2, 2:W + 2, :] = g
    vpad = np.zeros((N, H + 4, W + 4, C))
    vpad[:, 2:H + 2, 2:W + 2, :] = v
    dw = np.zeros((C, 5, 5))
    for a in range(5):
        for e in range(5):
            # output (y, x) read v[y+a-2, x+e-2]: that pixel receives w * dout[y, x]
            dv += w[:, a, e] * gpad[:, 4 - a:4 - a + H, 4 - e:4 - e + W, :]
            dw[:, a, e] = (g * vpad[:, a:a + H, e:e + W, :]).sum(axis=(0, 1, 2))
    return {"dq": dq, "dk": dk, "dv": dv, "dlce_w": dw, "dlce_b": g.sum(axis=(0, 1, 2))}
