"""Pins of the fp64 oracle to facts that do not come from the oracle itself.

Each pin takes the oracle module and raises AssertionError when the oracle
disagrees with the pages' definitions, a closed form, a library routine that
computes a special case, or a brute-force evaluation on a tiny input.
tests/test_oracle.py runs every pin on the real oracle; tests/
test_oracle_mutations.py plants plausible mistakes in the oracle and checks
that some pin fails for each of them.
"""
from __future__ import annotations

import itertools
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- partition
def pin_partition_matches_page_rearrange(O):
    """The walk-through (section BRA模块) partitions with the einops pattern
    "n (j h) (i w) c -> n (j i) h w c" and flattens tokens with
    "n p2 h w c -> n p2 (h w) c"; einops executes those strings here."""
    from einops import rearrange
    for (N, H, W, C, S) in [(2, 6, 6, 3, 3), (1, 8, 4, 2, 2), (1, 5, 5, 1, 1), (1, 4, 8, 2, 4)]:
        x = _rng(1).standard_normal((N, H, W, C))
        want = rearrange(x, "n (j h) (i w) c -> n (j i) h w c", j=S, i=S)
        want = rearrange(want, "n p2 h w c -> n p2 (h w) c")
        got = O.partition(x, S)
        assert got.shape == want.shape, (got.shape, want.shape)
        assert np.array_equal(got, want)
        back = O.unpartition(got, S, H, W)
        assert np.array_equal(back, x)


def pin_unpartition_matches_page_rearrange(O):
    """Output re-assembly "(n j i) m (h w) c -> n (j h) (i w) (m c)"."""
    from einops import rearrange
    N, H, W, S, m, c = 2, 6, 9, 3, 2, 3
    rh, rw = H // S, W // S
    x = _rng(2).standard_normal((N * S * S, m, rh * rw, c))
    want = rearrange(x, "(n j i) m (h w) c -> n (j h) (i w) (m c)", j=S, i=S, h=rh, w=rw)
    xp = rearrange(x, "(n p2) m t c -> n p2 t (m c)", n=N)
    assert np.array_equal(O.unpartition(xp, S, H, W), want)


# ---------------------------------------------------------------- means
def pin_region_means_closed_form(O):
    """q[n,y,x,c] = a_c*y + b_c*x + g_c has region means
    a_c*(j*rh + (rh-1)/2) + b_c*(i*rw + (rw-1)/2) + g_c, exactly in fp64 for
    small integer coefficients."""
    N, H, W, C, S = 2, 12, 8, 3, 4
    rh, rw = H // S, W // S
    a = np.array([1.0, -2.0, 3.0])
    b = np.array([5.0, 0.0, -1.0])
    g = np.array([0.5, 7.0, -3.0])
    y = np.arange(H)[:, None, None]
    x = np.arange(W)[None, :, None]
    q = np.broadcast_to(a * y + b * x + g, (N, H, W, C)).copy()
    got = O.region_means(O.partition(q, S))
    for n in range(N):
        for j in range(S):
            for i in range(S):
                want = a * (j * rh + (rh - 1) / 2) + b * (i * rw + (rw - 1) / 2) + g
                assert np.array_equal(got[n, j * S + i], want), (j, i, got[n, j * S + i], want)


def pin_region_means_constant(O):
    """A region filled with one vector has that vector as its mean
    (means over tokens, not over channels)."""
    N, S, rh, rw, C = 1, 3, 2, 5, 4
    vals = _rng(3).integers(-8, 8, size=(N, S, S, C)).astype(np.float64)
    q = np.repeat(np.repeat(vals, rh, axis=1), rw, axis=2)
    got = O.region_means(O.partition(q, S))
    assert np.array_equal(got, vals.reshape(N, S * S, C))


# ---------------------------------------------------------------- routing
def _constant_regions(vals, rh, rw):
    return np.repeat(np.repeat(vals, rh, axis=1), rw, axis=2)


def pin_affinity_known_answer(O):
    """Regions of constant tokens: q region r = e_(r mod C), k region s =
    val[s, :]. Then A[r, s] = C^-1/2 * val[s, r mod C] exactly (C = 4, so the
    scale is 1/2), and row r's routes are the regions sorted by
    val[:, r mod C] descending."""
    S, C, rh, rw, topk = 3, 4, 2, 2, 4
    R = S * S
    perms = [[3, 7, 1, 0, 8, 2, 6, 4, 5], [0, 1, 2, 3, 4, 5, 6, 7, 8],
             [8, 7, 6, 5, 4, 3, 2, 1, 0], [4, 0, 8, 1, 7, 2, 6, 3, 5]]
    val = np.array(perms, dtype=np.float64).T + 1.0            # (R, C)
    uq = np.zeros((1, S, S, C))
    for r in range(R):
        uq[0, r // S, r % S, r % C] = 1.0
    q = _constant_regions(uq, rh, rw)
    k = _constant_regions(val.reshape(1, S, S, C), rh, rw)
    qr = O.region_means(O.partition(q, S))
    kr = O.region_means(O.partition(k, S))
    A = O.region_affinity(qr, kr)
    for r in range(R):
        for s in range(R):
            assert A[0, r, s] == 0.5 * val[s, r % C], (r, s, A[0, r, s])
    route = O.topk_routes(A, topk)
    for r in range(R):
        col = val[:, r % C]
        want = sorted(range(R), key=lambda s: -col[s])[:topk]
        assert list(route[0, r]) == want, (r, list(route[0, r]), want)


def pin_routing_brute_force(O):
    """Tiny random inputs: means, affinities and routes evaluated with
    explicit Python loops (no numpy reductions) and a full sort by the key
    (-A, s)."""
    for seed, (N, H, W, C, S, topk) in enumerate([(2, 4, 4, 3, 2, 2), (1, 6, 3, 2, 3, 5), (1, 2, 2, 5, 2, 4)]):
        rng = _rng(100 + seed)
        q = rng.standard_normal((N, H, W, C))
        k = rng.standard_normal((N, H, W, C))
        rh, rw = H // S, W // S
        R = S * S

        def mean(x, n, r):
            j, i = divmod(r, S)
            acc = [0.0] * C
            for yy in range(j * rh, (j + 1) * rh):
                for xx in range(i * rw, (i + 1) * rw):
                    for c in range(C):
                        acc[c] += x[n, yy, xx, c]
            return [a / (rh * rw) for a in acc]

        A = O.region_affinity(O.region_means(O.partition(q, S)), O.region_means(O.partition(k, S)))
        route = O.topk_routes(A, topk)
        for n in range(N):
            for r in range(R):
                qm = mean(q, n, r)
                row = []
                for s in range(R):
                    km = mean(k, n, s)
                    row.append(sum(qm[c] * km[c] for c in range(C)) / C ** 0.5)
                assert np.allclose(A[n, r], row, rtol=1e-13, atol=1e-13)
                want = sorted(range(R), key=lambda s: (-row[s], s))[:topk]
                assert list(route[n, r]) == want, (n, r, list(route[n, r]), want)


def pin_routing_exact_ties(O):
    """Copy region s' of k bit-for-bit into a later region s: both get the
    same affinity with every query region, and the lower index must come
    first."""
    N, H, W, C, S = 1, 8, 8, 4, 4
    rng = _rng(7)
    q = rng.standard_normal((N, H, W, C))
    k = rng.standard_normal((N, H, W, C))
    rh = H // S
    # region 2 (j=0,i=2) copied into region 9 (j=2,i=1) and region 13 (j=3,i=1)
    src = k[:, 0:rh, 4:6, :].copy()
    k[:, 4:6, 2:4, :] = src
    k[:, 6:8, 2:4, :] = src
    A = O.region_affinity(O.region_means(O.partition(q, S)), O.region_means(O.partition(k, S)))
    assert np.array_equal(A[..., 2], A[..., 9]) and np.array_equal(A[..., 2], A[..., 13])
    R = S * S
    full = O.topk_routes(A, R)
    for r in range(R):
        lst = list(full[0, r])
        assert lst.index(2) < lst.index(9) < lst.index(13), (r, lst)
        assert sorted(lst) == list(range(R))
    # all-equal affinities: routes are 0..topk-1
    z = np.zeros((1, 5, 5))
    assert np.array_equal(O.topk_routes(z, 3)[0], np.tile(np.arange(3), (5, 1)))


def pin_route_is_permutation_at_full_topk(O):
    A = _rng(8).standard_normal((2, 9, 9))
    route = O.topk_routes(A, 9)
    for n in range(2):
        for r in range(9):
            assert sorted(route[n, r]) == list(range(9))
            vals = A[n, r, route[n, r]]
            assert np.all(np.diff(vals) <= 0)


# ---------------------------------------------------------------- attention
def _dense_reference(q, k, v, w, b, heads):
    """Dense multi-head attention over all H*W tokens (torch's
    scaled_dot_product_attention, which scales by head_dim^-1/2, in fp64 on
    the CPU) plus LCE from torch's grouped conv2d. Heads are split with the
    page's "(m c)" pattern via einops."""
    import torch
    import torch.nn.functional as F
    from einops import rearrange
    N, H, W, C = q.shape
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x))
    qh = rearrange(t(q), "n h w (m c) -> n m (h w) c", m=heads)
    kh = rearrange(t(k), "n h w (m c) -> n m (h w) c", m=heads)
    vh = rearrange(t(v), "n h w (m c) -> n m (h w) c", m=heads)
    o = F.scaled_dot_product_attention(qh, kh, vh)
    o = rearrange(o, "n m (h w) c -> n h w (m c)", h=H, w=W)
    vv = rearrange(t(v), "n h w c -> n c h w")
    l = F.conv2d(vv, t(w).reshape(C, 1, 5, 5), t(b), padding=2, groups=C)
    l = rearrange(l, "n c h w -> n h w c")
    return (o + l).numpy()


def pin_dense_when_all_regions_routed(O):
    """topk = S^2 routes every region to every query region, so BRA equals
    dense attention over all H*W tokens plus LCE (the dense-attention
    invariant); S = 1 is the same special case with one region."""
    cases = [(2, 6, 6, 8, 2, 3, 9), (1, 4, 8, 4, 1, 2, 4), (1, 5, 5, 6, 3, 1, 1), (1, 8, 8, 8, 2, 4, 16)]
    for seed, (N, H, W, C, heads, S, topk) in enumerate(cases):
        rng = _rng(200 + seed)
        q, k, v = (rng.standard_normal((N, H, W, C)) for _ in range(3))
        w = rng.standard_normal((C, 5, 5)) * 0.2
        b = rng.standard_normal(C) * 0.1
        got = O.bra_forward(q, k, v, w, b, heads, S, topk)["out"]
        want = _dense_reference(q, k, v, w, b, heads)
        assert np.allclose(got, want, rtol=1e-11, atol=1e-11), np.abs(got - want).max()


def pin_softmax_rows_sum_to_one(O):
    """Softmax rows: every query's probabilities over its gathered keys sum
    to 1, are non-negative, and are zero nowhere."""
    rng = _rng(9)
    q, k, v = (rng.standard_normal((2, 6, 6, 4)) for _ in range(3))
    res = O.bra_forward(q, k, v, np.zeros((4, 5, 5)), None, 2, 3, 2, return_probs=True)
    for per_img in res["probs"]:
        for p in per_img:
            assert p.shape == (9, 4, 2 * 4)
            assert np.all(p > 0)
            assert np.allclose(p.sum(-1), 1.0, atol=1e-12, rtol=0)


def pin_route_order_invariance(O):
    """Route-order invariance: permuting the order of each row's routed
    regions does not change the output (the softmax runs over the union)."""
    rng = _rng(10)
    N, H, W, C, heads, S, topk = 2, 8, 8, 4, 2, 4, 5
    q, k, v = (rng.standard_normal((N, H, W, C)) for _ in range(3))
    w = rng.standard_normal((C, 5, 5)) * 0.2
    b = rng.standard_normal(C) * 0.1
    base = O.bra_forward(q, k, v, w, b, heads, S, topk)
    perm = base["route_idx"].copy()
    for n in range(N):
        for r in range(S * S):
            perm[n, r] = rng.permutation(perm[n, r])
    again = O.bra_forward(q, k, v, w, b, heads, S, topk, route_override=perm)
    assert np.allclose(again["out"], base["out"], rtol=0, atol=1e-12)


def pin_identical_keys_give_mean_of_values(O):
    """All keys equal: the softmax is uniform, so each query's output is the
    plain mean of its gathered values (LCE zeroed). Values are one constant
    per region, so the output reveals which regions were gathered."""
    N, H, W, C, heads, S, topk = 1, 6, 6, 4, 2, 3, 3
    rh = H // S
    k = np.ones((N, H, W, C))
    q = _rng(11).standard_normal((N, H, W, C))
    cval = np.arange(S * S, dtype=np.float64) * 8.0 + 1.0           # one value per region
    v = np.repeat(np.repeat(cval.reshape(1, S, S, 1), rh, 1), rh, 2) * np.ones((1, 1, 1, C))
    route = np.array([[[(r + 1) % 9, (r * 4) % 9, (r + 5) % 9] for r in range(9)]])
    res = O.bra_forward(q, k, v, np.zeros((C, 5, 5)), None, heads, S, topk, route_override=route)
    out = res["out"]
    for r in range(9):
        j, i = divmod(r, S)
        want = np.mean([cval[s] for s in route[0, r]])
        assert np.allclose(out[0, j * rh:(j + 1) * rh, i * rh:(i + 1) * rh, :], want, rtol=0, atol=1e-12)


def pin_single_token_regions(O):
    """T = 1 (one token per region) and topk = 1: each query attends to one
    key, so out = v of the routed token (LCE zeroed)."""
    N, H, W, C, heads = 1, 3, 4, 4, 2
    rng = _rng(12)
    q, k, v = (rng.standard_normal((N, H, W, C)) for _ in range(3))
    # S must divide both H and W with one token per region: use H = W = S.
    H = W = S = 3
    q, k, v = (x[:, :3, :3, :] for x in (q, k, v))
    res = O.bra_forward(q, k, v, np.zeros((C, 5, 5)), None, heads, S, 1)
    route = res["route_idx"]
    for r in range(9):
        s = route[0, r, 0]
        assert np.allclose(res["out"][0, r // 3, r % 3], v[0, s // 3, s % 3], rtol=0, atol=1e-14)
        # the routed region is the argmax of q_r . k_s over s
        dots = [q[0, r // 3, r % 3] @ k[0, t // 3, t % 3] for t in range(9)]
        assert s == int(np.argmax(dots))


def pin_dense_attention_matches_library(O):
    """The router-free path against torch's scaled_dot_product_attention and
    grouped conv2d in fp64 (a library routine computing the same thing)."""
    cases = [(2, 7, 7, 8, 2), (1, 3, 5, 12, 3), (1, 4, 4, 4, 1)]
    for seed, (N, H, W, C, heads) in enumerate(cases):
        rng = _rng(600 + seed)
        q, k, v = (rng.standard_normal((N, H, W, C)) for _ in range(3))
        w = rng.standard_normal((C, 5, 5)) * 0.2
        b = rng.standard_normal(C) * 0.1
        got = O.dense_attention(q, k, v, w, b, heads)
        want = _dense_reference(q, k, v, w, b, heads)
        assert np.allclose(got, want, rtol=1e-11, atol=1e-11), np.abs(got - want).max()


def pin_dense_attention_equals_full_routing(O):
    """The dense-attention invariant from the other side: BRA with every region routed
    (topk = S^2, S > 1, so the keys arrive in routing order, region by region)
    equals the dense path."""
    for seed, (N, H, W, C, heads, S) in enumerate([(1, 6, 6, 8, 2, 3), (2, 4, 8, 4, 2, 2)]):
        rng = _rng(610 + seed)
        q, k, v = (rng.standard_normal((N, H, W, C)) for _ in range(3))
        w = rng.standard_normal((C, 5, 5)) * 0.2
        b = rng.standard_normal(C) * 0.1
        got = O.dense_attention(q, k, v, w, b, heads)
        want = O.bra_forward(q, k, v, w, b, heads, S, S * S)["out"]
        assert np.allclose(got, want, rtol=1e-11, atol=1e-11), np.abs(got - want).max()


def pin_dense_attention_single_token(O):
    """A 1x1 map: the one key gets probability 1 and only the centre tap of
    the 5x5 window sees the image, so out = v + w[:, 2, 2] * v + b."""
    rng = _rng(620)
    C = 6
    q, k, v = (rng.standard_normal((3, 1, 1, C)) for _ in range(3))
    w = rng.standard_normal((C, 5, 5))
    b = rng.standard_normal(C)
    got = O.dense_attention(q, k, v, w, b, 2)
    assert np.allclose(got, v + w[:, 2, 2] * v + b, rtol=0, atol=1e-13)


def pin_dense_attention_uniform_keys(O):
    """All keys equal: the softmax is uniform over the image, so with the
    LCE weights zero each output is the mean of V over all tokens (per
    channel) plus the bias; queries do not matter."""
    rng = _rng(621)
    N, H, W, C = 2, 3, 4, 4
    q = rng.standard_normal((N, H, W, C))
    v = rng.standard_normal((N, H, W, C))
    b = rng.standard_normal(C)
    got = O.dense_attention(q, np.ones((N, H, W, C)), v, np.zeros((C, 5, 5)), b, 2)
    want = v.mean(axis=(1, 2), keepdims=True) + b
    assert np.allclose(got, np.broadcast_to(want, got.shape), rtol=0, atol=1e-13)


def pin_head_routed_one_head_is_the_operator(O):
    """With one head, routing per head is routing over all channels: the
    variant equals bra_forward (routes, logits and output)."""
    rng = _rng(630)
    N, H, W, C, S, topk = 2, 6, 6, 8, 3, 4
    q, k, v = (rng.standard_normal((N, H, W, C)) for _ in range(3))
    w = rng.standard_normal((C, 5, 5)) * 0.2
    b = rng.standard_normal(C) * 0.1
    got = O.bra_forward_head_routed(q, k, v, w, b, 1, S, topk)
    want = O.bra_forward(q, k, v, w, b, 1, S, topk)
    assert np.array_equal(got["route_idx"][:, 0], want["route_idx"])
    assert np.allclose(got["logits"][:, 0], want["logits"], rtol=0, atol=1e-13)
    assert np.allclose(got["out"], want["out"], rtol=0, atol=1e-12)


def pin_head_routed_brute_force_routes(O):
    """Per-head routes and logits from plain Python loops on a tiny input:
    head m's region means over its own channels, logits scaled by
    head_dim^-1/2, descending order with ties to the lower index."""
    rng = _rng(631)
    N, H, W, C, heads, S, topk = 1, 4, 4, 6, 3, 2, 3
    q, k, v = (rng.standard_normal((N, H, W, C)) for _ in range(3))
    res = O.bra_forward_head_routed(q, k, v, np.zeros((C, 5, 5)), None, heads, S, topk)
    hd, rh, R = C // heads, H // S, S * S
    for m in range(heads):
        def mean(x, r):
            j, i = divmod(r, S)
            return [sum(x[0, j * rh + a, i * rh + e, m * hd + c] for a in range(rh) for e in range(rh)) / (rh * rh)
                    for c in range(hd)]
        for r in range(R):
            qm = mean(q, r)
            row = [sum(a * c for a, c in zip(qm, mean(k, t))) / hd ** 0.5 for t in range(R)]
            assert np.allclose(res["logits"][0, m, r], row, rtol=0, atol=1e-12)
            order = sorted(range(R), key=lambda t: (-row[t], t))[:topk]
            assert list(res["route_idx"][0, m, r]) == order


def pin_head_routed_heads_route_apart(O):
    """A known answer where the heads must disagree: head 0's channels make
    every region prefer region 1, head 1's prefer region 2 (k's channels of a
    head are large only in that region). Shared routing could not give both."""
    N, H, W, C, heads, S = 1, 4, 4, 4, 2, 2
    q = np.ones((N, H, W, C))
    k = np.zeros((N, H, W, C))
    k[0, 0:2, 2:4, 0:2] = 5.0      # region 1 (j = 0, i = 1), head 0's channels
    k[0, 2:4, 0:2, 2:4] = 3.0      # region 2 (j = 1, i = 0), head 1's channels
    v = _rng(632).standard_normal((N, H, W, C))
    res = O.bra_forward_head_routed(q, k, v, np.zeros((C, 5, 5)), None, heads, S, 1)
    assert np.all(res["route_idx"][0, 0, :, 0] == 1)
    assert np.all(res["route_idx"][0, 1, :, 0] == 2)


def pin_head_routed_all_regions_is_dense(O):
    """topk = S^2 routes every region for every head: the variant equals the
    dense attention (pinned to torch's SDPA)."""
    rng = _rng(633)
    N, H, W, C, heads, S = 2, 6, 6, 8, 2, 3
    q, k, v = (rng.standard_normal((N, H, W, C)) for _ in range(3))
    w = rng.standard_normal((C, 5, 5)) * 0.2
    b = rng.standard_normal(C) * 0.1
    got = O.bra_forward_head_routed(q, k, v, w, b, heads, S, S * S)["out"]
    assert np.allclose(got, _dense_reference(q, k, v, w, b, heads), rtol=1e-11, atol=1e-11)


def _fd_check(O, N, H, W, C, heads, S, topk, seed, h=1e-6, rtol=1e-6):
    """Directional finite differences of sum(bra_forward(...)["out"] * dout)
    against bra_backward, for q, k, v, the LCE weights and bias."""
    rng = _rng(seed)
    q, k, v, g = (rng.standard_normal((N, H, W, C)) for _ in range(4))
    w = rng.standard_normal((C, 5, 5)) * 0.3
    b = rng.standard_normal(C) * 0.1
    route = O.bra_forward(q, k, v, w, b, heads, S, topk)["route_idx"]
    res = O.bra_backward(q, k, v, w, route, g, heads, S)
    args = {"q": q, "k": k, "v": v, "w": w, "b": b}
    f = lambda a: (O.bra_forward(a["q"], a["k"], a["v"], a["w"], a["b"], heads, S, topk,
                                 route_override=route)["out"] * g).sum()
    for name, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("w", "dlce_w"), ("b", "dlce_b")):
        d = rng.standard_normal(args[name].shape)
        ap, am = dict(args), dict(args)
        ap[name], am[name] = args[name] + h * d, args[name] - h * d
        fd = (f(ap) - f(am)) / (2 * h)
        an = (res[key] * d).sum()
        assert abs(fd - an) <= rtol * max(1.0, abs(fd)), (name, fd, an)


def pin_backward_finite_differences(O):
    """The routed gradients against central finite differences of the
    forward (routes held fixed, as the detached router does): regions
    routed by several query regions, topk 1 and S^2, one and three heads."""
    for i, case in enumerate([(1, 4, 4, 4, 2, 2, 2), (2, 6, 6, 6, 3, 3, 3), (1, 4, 6, 4, 1, 2, 4),
                              (1, 6, 6, 4, 2, 3, 1)]):
        _fd_check(O, *case, seed=640 + i)


def pin_backward_one_region_is_autograd(O):
    """One region routed to itself (S = 1) is dense attention: the gradients
    equal torch.autograd through scaled_dot_product_attention and the grouped
    conv2d, in fp64."""
    import torch
    import torch.nn.functional as F
    from einops import rearrange
    rng = _rng(650)
    N, H, W, C, heads = 2, 5, 4, 6, 3
    q, k, v, g = (rng.standard_normal((N, H, W, C)) for _ in range(4))
    w = rng.standard_normal((C, 5, 5)) * 0.3
    b = rng.standard_normal(C) * 0.1
    res = O.bra_backward(q, k, v, w, np.zeros((N, 1, 1), dtype=np.int64), g, heads, 1)
    t = {n: torch.tensor(x, requires_grad=True) for n, x in (("q", q), ("k", k), ("v", v), ("w", w), ("b", b))}
    split = lambda x: rearrange(x, "n h w (m c) -> n m (h w) c", m=heads)
    o = rearrange(F.scaled_dot_product_attention(split(t["q"]), split(t["k"]), split(t["v"])),
                  "n m (h w) c -> n h w (m c)", h=H)
    l = F.conv2d(t["v"].permute(0, 3, 1, 2), t["w"].reshape(C, 1, 5, 5), t["b"], padding=2, groups=C)
    ((o + l.permute(0, 2, 3, 1)) * torch.tensor(g)).sum().backward()
    for n, key in (("q", "dq"), ("k", "dk"), ("v", "dv"), ("w", "dlce_w"), ("b", "dlce_b")):
        assert np.allclose(res[key], t[n].grad.numpy(), rtol=1e-10, atol=1e-10), n


def pin_backward_value_gradient_sums(O):
    """With the LCE weights zero, every query's probabilities sum to 1, so
    the value gradients of an image sum (over all pixels, per channel) to the
    sum of dout; the bias gradient is the sum of dout over the batch."""
    rng = _rng(651)
    N, H, W, C, heads, S, topk = 2, 6, 6, 4, 2, 3, 2
    q, k, v, g = (rng.standard_normal((N, H, W, C)) for _ in range(4))
    route = O.bra_forward(q, k, v, np.zeros((C, 5, 5)), None, heads, S, topk)["route_idx"]
    res = O.bra_backward(q, k, v, np.zeros((C, 5, 5)), route, g, heads, S)
    assert np.allclose(res["dv"].sum(axis=(1, 2)), g.sum(axis=(1, 2)), rtol=0, atol=1e-11)
    assert np.allclose(res["dlce_b"], g.sum(axis=(0, 1, 2)), rtol=0, atol=1e-11)


# ---------------------------------------------------------------- LCE
def pin_lce_delta_kernel(O):
    rng = _rng(13)
    v = rng.standard_normal((2, 5, 7, 3))
    w = np.zeros((3, 5, 5))
    w[:, 2, 2] = 1.0
    b = np.array([0.5, -1.0, 2.0])
    assert np.array_equal(O.lce(v, w, b), v + b)


def pin_lce_ones_count_closed_form(O):
    """v = 1, w = 1, b = 0: each output counts the in-image taps,
    (#rows of [y-2, y+2] inside) * (#cols of [x-2, x+2] inside): 25 inside,
    15 on an edge, 9 in a corner."""
    H, W = 6, 7
    out = O.lce(np.ones((1, H, W, 2)), np.ones((2, 5, 5)), None)
    for y in range(H):
        for x in range(W):
            ny = min(y + 2, H - 1) - max(y - 2, 0) + 1
            nx = min(x + 2, W - 1) - max(x - 2, 0) + 1
            assert out[0, y, x, 0] == ny * nx == out[0, y, x, 1]
    assert out[0, 3, 3, 0] == 25 and out[0, 0, 3, 0] == 15 and out[0, 0, 0, 0] == 9


def pin_lce_orientation(O):
    """Cross-correlation, like Conv2d: with only w[c, 0, 0] = 1 the output at
    (y, x) is v at (y-2, x-2) (zero outside the image)."""
    v = _rng(14).standard_normal((1, 6, 6, 2))
    w = np.zeros((2, 5, 5))
    w[:, 0, 0] = 1.0
    out = O.lce(v, w, None)
    want = np.zeros_like(v)
    want[:, 2:, 2:, :] = v[:, :-2, :-2, :]
    assert np.array_equal(out, want)


def pin_lce_matches_scipy_correlate(O):
    from scipy.signal import correlate2d
    rng = _rng(15)
    v = rng.standard_normal((2, 7, 9, 3))
    w = rng.standard_normal((3, 5, 5))
    b = rng.standard_normal(3)
    out = O.lce(v, w, b)
    for n in range(2):
        for c in range(3):
            want = correlate2d(v[n, :, :, c], w[c], mode="same", boundary="fill") + b[c]
            assert np.allclose(out[n, :, :, c], want, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------- shapes
def pin_c0_shape_trace(O):
    """The walk-through's tensor trace at stage 1 (golden file; section
    BRA模块): (1,56,56,64) -> 49 regions of 64 tokens -> means (1,49,64) ->
    logits (1,49,49) -> r_idx (1,49,1) -> gathered (1,49,1,64,64) per K and V ->
    attention weights (49,2,64,64) -> out (1,56,56,64)."""
    import json
    with open(os.path.join(GOLDEN, "c0_shape_trace.json")) as f:
        trace = json.load(f)["shapes"]
    N, H, W, C, heads, S, topk = 1, 56, 56, 64, 2, 7, 1
    rng = _rng(16)
    q, k, v = (rng.standard_normal((N, H, W, C)) for _ in range(3))
    qp = O.partition(q, S)
    assert tuple(qp.reshape(N, S * S, 8, 8, C).shape) == tuple(trace["patchify"])
    assert tuple(qp.shape) == tuple(trace["q_pix"])
    qr = O.region_means(qp)
    assert tuple(qr.shape) == tuple(trace["q_win"])
    A = O.region_affinity(qr, O.region_means(O.partition(k, S)))
    assert tuple(A.shape) == tuple(trace["attn_logit"])
    route = O.topk_routes(A, topk)
    assert tuple(route.shape) == tuple(trace["r_idx"])
    kg = O.gather_regions(O.partition(k, S), route)
    assert tuple(kg.reshape(N, S * S, topk, 64, C).shape) == tuple(trace["k_pix_sel"])
    res = O.bra_forward(q, k, v, np.zeros((C, 5, 5)), None, heads, S, topk, return_probs=True)
    p = np.stack(res["probs"][0], axis=1)          # (R, heads, T, L)
    assert tuple(p.shape) == tuple(trace["attn_weight"])
    assert tuple(res["out"].shape) == tuple(trace["out"])


# ---------------------------------------------------------------- projections
def pin_linear_hand_example(O):
    """A Linear layer computes x w^T + b with w stored (out, in) (the
    walk-through's Linear(64, 192) maps 64 channels to 192): worked by hand
    for a 2 x 3 input, a 2 x 3 weight and a bias."""
    x = np.array([[1.0, 2.0, 3.0], [4.0, 5.0, 6.0]])
    w = np.array([[1.0, 0.0, -1.0], [2.0, 1.0, 0.0]])
    b = np.array([0.5, -1.0])
    want = np.array([[-1.5, 3.0], [-1.5, 12.0]])
    assert np.array_equal(O.linear(x, w, b), want)
    assert np.array_equal(O.linear(x, w, None), want - b)


def pin_linear_brute_force(O):
    """Every output of a small Linear equals its sum of products written out
    one term at a time (leading axes kept: (2, 3, K) tokens)."""
    rng = _rng(41)
    x = rng.standard_normal((2, 3, 5))
    w = rng.standard_normal((7, 5))
    b = rng.standard_normal(7)
    y = O.linear(x, w, b)
    assert y.shape == (2, 3, 7)
    for i in range(2):
        for j in range(3):
            for f in range(7):
                acc = b[f]
                for c in range(5):
                    acc += x[i, j, c] * w[f, c]
                assert abs(y[i, j, f] - acc) < 1e-12


def pin_round_bf16_known_values(O):
    """bfloat16 keeps 8 significant bits and rounds to nearest, ties to even:
    at 1 the spacing is 2^-7, so 1 + 2^-8 (a tie) stays 1, 1 + 3*2^-8 (a tie)
    goes to the even 1 + 2^-6, anything above a half spacing rounds up, and
    the sign is kept."""
    x = np.array([1.0, 1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 1 + 2.0 ** -8 + 2.0 ** -20,
                  -(1 + 2.0 ** -8 + 2.0 ** -20), 3.0, 0.0, 2.0 ** -130])
    want = np.array([1.0, 1.0, 1 + 2.0 ** -6, 1 + 2.0 ** -7, -(1 + 2.0 ** -7), 3.0, 0.0, 2.0 ** -130])
    assert np.array_equal(O.round_bf16(x), want)


def _block_inputs(seed, N=1, H=8, W=8, C=8):
    rng = _rng(seed)
    x = rng.standard_normal((N, H, W, C))
    lw = rng.standard_normal((C, 5, 5)) * 0.2
    lb = rng.standard_normal(C) * 0.1
    return x, lw, lb


def pin_block_identity_projections(O):
    """With qkv = three stacked identities (zero bias) and wo = diag(d) plus a
    bias, the block is the operator on (x, x, x), scaled per channel and
    shifted (section BRA模块: q, kv = qkv(x), then the operator, then wo)."""
    x, lw, lb = _block_inputs(42)
    C = x.shape[-1]
    eye = np.eye(C)
    d = np.arange(1.0, C + 1)
    bo = np.linspace(-1, 1, C)
    res = O.bra_block_forward(x, np.vstack([eye, eye, eye]), None, lw, lb, np.diag(d), bo,
                              heads=2, S=2, topk=2)
    op = O.bra_forward(x, x, x, lw, lb, 2, 2, 2)
    assert np.allclose(res["out"], op["out"] * d + bo, rtol=0, atol=1e-12)
    assert np.array_equal(res["route_idx"], op["route_idx"])


def pin_block_split_order(O):
    """qkv's 3C outputs are q, then k, then v: with the blocks 2I, 3I, 5I
    and wo = I the block equals the operator on (2x, 3x, 5x)."""
    x, lw, lb = _block_inputs(43)
    C = x.shape[-1]
    eye = np.eye(C)
    bq = np.concatenate([np.full(C, 0.1), np.full(C, -0.2), np.full(C, 0.3)])
    res = O.bra_block_forward(x, np.vstack([2 * eye, 3 * eye, 5 * eye]), bq, lw, lb, eye, None,
                              heads=2, S=2, topk=1)
    op = O.bra_forward(2 * x + 0.1, 3 * x - 0.2, 5 * x + 0.3, lw, lb, 2, 2, 1)
    assert np.allclose(res["out"], op["out"], rtol=0, atol=1e-12)


def pin_block_bf16_store_rounds_handoffs(O):
    """store="bf16" rounds q, k, v and the operator's output and nothing else:
    fed x already on the bf16 grid with identity projections, the block equals
    wo applied to the rounded operator output."""
    x, lw, lb = _block_inputs(44)
    x = O.round_bf16(x)
    C = x.shape[-1]
    eye = np.eye(C)
    res = O.bra_block_forward(x, np.vstack([eye, eye, eye]), None, lw, lb, eye, None,
                              heads=2, S=2, topk=2, store="bf16")
    op = O.bra_forward(x, x, x, lw, lb, 2, 2, 2)
    assert np.array_equal(res["out"], O.round_bf16(op["out"]))
    assert not np.array_equal(res["out"], op["out"])


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
