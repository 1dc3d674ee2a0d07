"""Parity of the HIP path (through the C ABI) with the fp64 oracle.

Every case prints its name before touching the GPU. Inputs come from the
seeded generator in synth/, which both sides read bit for bit.
"""
from __future__ import annotations

import sys
import zlib

import numpy as np
import pytest

import oracle
from oracle import bra_oracle as O
from synth import CONFIGS, draw, draw_config
from tests.parity import check_output, compare_routes

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def oracle_routing(inp, S, topk):
    A = O.region_affinity(O.region_means(O.partition(inp["q"], S)),
                          O.region_means(O.partition(inp["k"], S)))
    return A, O.topk_routes(A, topk)


def run_forward(bra, inp, heads, S, topk, dtype, images=None, name=""):
    say(name, "forward", inp["q"].shape, f"heads={heads} S={S} topk={topk} {dtype}")
    out, route = bra.forward(dev(inp["q"], dtype), dev(inp["k"], dtype), dev(inp["v"], dtype),
                             dev(inp["lce_w"], dtype), dev(inp["lce_b"], dtype), heads, S, topk)
    out, route = host(out), host(route)
    A, own = oracle_routing(inp, S, topk)
    exact, near, fails = compare_routes(route, A, own)
    assert not fails, fails[:5]
    N = inp["q"].shape[0]
    imgs = list(range(N)) if images is None else images
    ref = oracle.bra_forward(inp["q"][imgs], inp["k"][imgs], inp["v"][imgs], inp["lce_w"],
                             inp["lce_b"], heads, S, topk, route_override=route[imgs])
    rep = check_output(out[imgs], ref["out"], dtype)
    rep.update(exact_rows=exact, near_tie_rows=near)
    say(name, rep)
    return out, route, rep


SMALL_CASES = [
    # name, N, H, W, C, heads, S, topk, dtype, offset_std
    ("c1_like_b2", 2, 28, 28, 128, 4, 7, 4, "bf16", 0.0),
    ("c2_like_b3", 3, 14, 14, 256, 8, 7, 16, "bf16", 0.0),
    ("t64_l192", 1, 32, 32, 64, 2, 4, 3, "bf16", 0.7),
    ("t256_l512", 1, 64, 64, 64, 2, 4, 2, "bf16", 0.7),
    ("ragged_t6_l18", 2, 15, 10, 64, 2, 5, 3, "bf16", 0.0),
    ("t20_qblocks", 1, 20, 25, 64, 2, 5, 2, "bf16", 0.0),
    ("t1_single_token", 1, 8, 8, 32, 1, 8, 5, "bf16", 0.0),
    ("dense_topk_eq_R", 1, 12, 12, 64, 2, 3, 9, "bf16", 0.0),
    ("s1_one_region", 2, 8, 8, 32, 1, 1, 1, "bf16", 0.0),
    ("nonsquare_t24", 1, 16, 24, 96, 3, 4, 5, "bf16", 0.0),
    ("r1024_router", 1, 32, 32, 32, 1, 32, 16, "bf16", 0.0),
    ("r400_router", 1, 40, 40, 64, 2, 20, 7, "bf16", 0.7),
    ("r100_router", 2, 20, 20, 64, 2, 10, 6, "bf16", 0.0),
    ("r36_three_col_tiles", 2, 24, 24, 96, 3, 6, 5, "bf16", 0.0),
    # small-region kernel: T = 16 / G key tiles side by side in the score columns
    ("t8_2x4_regions_l24", 1, 8, 16, 128, 4, 4, 3, "bf16", 0.0),
    ("t8_4x2_regions_h8_l40", 2, 16, 8, 256, 8, 4, 5, "bf16", 0.7),
    ("t8_l128_two_chunks", 1, 16, 32, 64, 2, 8, 16, "bf16", 0.7),
    ("t4_l96_two_chunks", 1, 16, 16, 128, 4, 8, 24, "bf16", 0.7),
    ("t2_1x2_regions_l14", 1, 6, 12, 64, 2, 6, 7, "bf16", 0.0),
    ("t1_1x1_regions_l40", 1, 8, 8, 64, 2, 8, 40, "bf16", 0.7),
    # 4x4 regions of an image too large for the image-resident kernel
    ("t16_region_kernel_64px", 1, 64, 64, 128, 4, 16, 4, "bf16", 0.7),
    # the one-kernel 4x4 path (pooling and routing in the attention kernel):
    # region counts 1..36, topk 1..4 (= S^2 too), C 64/128, 2 and 4 heads,
    # whole and partial prefetch slots
    ("fused_s4_c64_t2", 2, 16, 16, 64, 2, 4, 2, "bf16", 0.7),
    ("fused_s5_c128_t3", 3, 20, 20, 128, 4, 5, 3, "bf16", 0.0),
    ("fused_s3_c64_t1", 2, 12, 12, 64, 2, 3, 1, "bf16", 0.7),
    ("fused_s6_c64_t4", 1, 24, 24, 64, 2, 6, 4, "bf16", 0.0),
    ("fused_s2_topk_eq_R", 1, 8, 8, 128, 4, 2, 4, "bf16", 0.0),
    ("fused_s1_one_region", 2, 4, 4, 64, 2, 1, 1, "bf16", 0.0),
    ("f32_c0_like", 1, 56, 56, 64, 2, 7, 1, "f32", 0.0),
    ("f32_ragged", 2, 15, 10, 64, 2, 5, 3, "f32", 0.0),
    ("f32_t256", 1, 64, 64, 64, 2, 4, 2, "f32", 0.7),
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=[c[0] for c in SMALL_CASES])
def test_forward_small(gpu_lib, case):
    name, N, H, W, C, heads, S, topk, dtype, off = case
    inp = draw(N, H, W, C, S, dtype, seed=zlib.crc32(name.encode()) % 10000, offset_std=off)
    run_forward(gpu_lib, inp, heads, S, topk, dtype, name=name)


# Full-size workloads, in the launch configuration the benchmark times:
# routes and outputs of every image are compared with the oracle's, and the
# exact and near-tie route rows are reported.
@pytest.mark.parametrize("cfg", CONFIGS, ids=[c.name for c in CONFIGS])
def test_forward_full_config(gpu_lib, cfg):
    inp = draw_config(cfg)
    _, _, rep = run_forward(gpu_lib, inp, cfg.heads, cfg.S, cfg.topk, cfg.dtype, name=cfg.name)
    assert rep["exact_rows"] + rep["near_tie_rows"] == cfg.N * cfg.R


@pytest.mark.parametrize("cfg", CONFIGS, ids=[c.name for c in CONFIGS])
def test_region_means(gpu_lib, cfg):
    inp = draw_config(cfg, N=min(cfg.N, 4))
    say(cfg.name, "region_means")
    qr, kr = gpu_lib.region_means(dev(inp["q"], cfg.dtype), dev(inp["k"], cfg.dtype), cfg.S)
    qr, kr = host(qr), host(kr)
    want_q = O.region_means(O.partition(inp["q"], cfg.S))
    want_k = O.region_means(O.partition(inp["k"], cfg.S))
    assert np.allclose(qr, want_q, rtol=1e-5, atol=1e-6), np.abs(qr - want_q).max()
    assert np.allclose(kr, want_k, rtol=1e-5, atol=1e-6), np.abs(kr - want_k).max()


@pytest.mark.parametrize("cfg", CONFIGS, ids=[c.name for c in CONFIGS])
def test_router_from_oracle_means(gpu_lib, cfg):
    """Routing alone, fed the oracle's means rounded to fp32."""
    import torch
    inp = draw_config(cfg)  # full batch: large batches take the per-image routing kernel
    qr = O.region_means(O.partition(inp["q"], cfg.S)).astype(np.float32)
    kr = O.region_means(O.partition(inp["k"], cfg.S)).astype(np.float32)
    say(cfg.name, "route")
    ri = host(gpu_lib.route(torch.from_numpy(qr).cuda(), torch.from_numpy(kr).cuda(), cfg.topk))
    A = O.region_affinity(qr.astype(np.float64), kr.astype(np.float64))
    exact, near, fails = compare_routes(ri, A, O.topk_routes(A, cfg.topk))
    assert not fails, fails[:5]


@pytest.mark.parametrize("case", [SMALL_CASES[i] for i in (0, 1, 2, 4, 12)], ids=lambda c: c[0])
def test_attend_with_oracle_routes(gpu_lib, case):
    """Attention + LCE alone, on the oracle's own routes."""
    import torch
    name, N, H, W, C, heads, S, topk, dtype, off = case
    inp = draw(N, H, W, C, S, dtype, seed=7 + zlib.crc32(name.encode()) % 1000, offset_std=off)
    ref = oracle.bra_forward(inp["q"], inp["k"], inp["v"], inp["lce_w"], inp["lce_b"], heads, S, topk)
    say(name, "attend")
    out = gpu_lib.attend(dev(inp["q"], dtype), dev(inp["k"], dtype), dev(inp["v"], dtype),
                         dev(inp["lce_w"], dtype), dev(inp["lce_b"], dtype),
                         torch.from_numpy(ref["route_idx"].astype(np.int32)).cuda(), heads, S)
    check_output(host(out), ref["out"], dtype)


@pytest.mark.parametrize("H,rside", [(32, 8), (64, 16)], ids=["8x8_regions", "16x16_regions"])
def test_attend_late_large_scores(gpu_lib, H, rside):
    """The last routed region holds keys whose scaled scores exceed all
    earlier ones by about 163 (base-2 exponent units): past fp32's range, so
    the large-region kernel must raise its running maximum after the first
    key tile (the rescale path that ordinary inputs never take) to match the
    oracle rather than overflow."""
    import torch
    N, C, heads, S, topk = 1, 64, 2, 4, 4
    R = S * S
    inp = draw(N, H, H, C, S, "bf16", seed=4242)
    q = np.full_like(inp["q"], 1.0)      # every score = sum of the key's channels
    k = inp["k"].copy()
    X = 5                                # region routed last, half its keys at +20
    jx, ix = divmod(X, S)
    k[:, jx * rside:(jx + 1) * rside, ix * rside:ix * rside + rside // 2, :] = 20.0
    others = [s_ for s_ in range(R) if s_ != X]
    route = np.array([[others[(r + 1) % (R - 1)], others[(r + 2) % (R - 1)],
                       others[(r + 7) % (R - 1)], X] for r in range(R)], dtype=np.int32)[None]
    assert all(len(set(row)) == topk for row in route[0])
    ref = oracle.bra_forward(q, k, inp["v"], inp["lce_w"], inp["lce_b"], heads, S, topk,
                             route_override=route)
    say("late large scores", H)
    out = gpu_lib.attend(dev(q, "bf16"), dev(k, "bf16"), dev(inp["v"], "bf16"),
                         dev(inp["lce_w"], "bf16"), dev(inp["lce_b"], "bf16"),
                         torch.from_numpy(route).cuda(), heads, S)
    check_output(host(out), ref["out"], "bf16")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_lce_alone(gpu_lib, dtype):
    inp = draw(2, 20, 12, 96, 4, dtype, seed=55)
    say("lce", dtype)
    got = host(gpu_lib.lce(dev(inp["v"], dtype), dev(inp["lce_w"], dtype), dev(inp["lce_b"], dtype)))
    want = O.lce(inp["v"], inp["lce_w"], inp["lce_b"])
    assert np.allclose(got, want, rtol=0, atol=2e-5), np.abs(got - want).max()
    say("lce no bias", dtype)
    got = host(gpu_lib.lce(dev(inp["v"], dtype), dev(inp["lce_w"], dtype), None))
    want = O.lce(inp["v"], inp["lce_w"], None)
    assert np.allclose(got, want, rtol=0, atol=2e-5)


def test_exact_ties_go_to_lower_index(gpu_lib):
    """Bit-identical regions of k tie exactly on both sides: the lower index
    must win, with no near-tie slack."""
    N, H, W, C, heads, S = 2, 16, 16, 64, 2, 4
    inp = draw(N, H, W, C, S, "bf16", seed=99)
    k = inp["k"]
    k[:, 4:8, 8:12, :] = k[:, 0:4, 4:8, :]      # region 6 := region 1
    k[:, 12:16, 0:4, :] = k[:, 0:4, 4:8, :]     # region 12 := region 1
    say("ties")
    _, route = gpu_lib.forward(dev(inp["q"], "bf16"), dev(k, "bf16"), dev(inp["v"], "bf16"),
                              dev(inp["lce_w"], "bf16"), None, heads, S, 16)
    route = host(route)
    for n in range(N):
        for r in range(16):
            lst = list(route[n, r])
            assert sorted(lst) == list(range(16))
            assert lst.index(1) < lst.index(6) < lst.index(12), (n, r, lst)


def test_exact_ties_one_kernel_path(gpu_lib):
    """The routing inside the 4x4-region attention kernel on exact ties:
    regions 6 and 12 of k are copies of region 1 and outweigh every other
    region for every query (q is all ones), so each row's first three routes
    are exactly 1, 6, 12 in that order and the fourth is the best of the rest."""
    N, H, W, C, heads, S, topk = 2, 16, 16, 64, 2, 4, 4
    inp = draw(N, H, W, C, S, "bf16", seed=1234)
    q = np.ones_like(inp["q"])
    k = inp["k"].copy()
    k[:, 0:4, 4:8, :] = 3.0 + 0.25 * np.sign(k[:, 0:4, 4:8, :])  # region 1: large means
    k[:, 4:8, 8:12, :] = k[:, 0:4, 4:8, :]      # region 6 := region 1
    k[:, 12:16, 0:4, :] = k[:, 0:4, 4:8, :]     # region 12 := region 1
    inp = dict(inp, q=q, k=k)
    say("ties, one-kernel path")
    _, route, _ = run_forward(gpu_lib, inp, heads, S, topk, "bf16", name="ties_one_kernel")
    for n in range(N):
        for r in range(S * S):
            assert list(route[n, r, :3]) == [1, 6, 12], (n, r, list(route[n, r]))


def test_one_kernel_path_without_bias(gpu_lib):
    """The 4x4-region one-kernel path with lce_b = None (no LCE bias)."""
    N, H, W, C, heads, S, topk = 2, 20, 20, 128, 4, 5, 4
    inp = draw(N, H, W, C, S, "bf16", seed=4321, offset_std=0.7)
    say("one-kernel path, no bias")
    out, route = gpu_lib.forward(dev(inp["q"], "bf16"), dev(inp["k"], "bf16"), dev(inp["v"], "bf16"),
                                 dev(inp["lce_w"], "bf16"), None, heads, S, topk)
    out, route = host(out), host(route)
    A, own = oracle_routing(inp, S, topk)
    exact, near, fails = compare_routes(route, A, own)
    assert not fails, fails[:5]
    ref = oracle.bra_forward(inp["q"], inp["k"], inp["v"], inp["lce_w"], None, heads, S, topk,
                             route_override=route)
    check_output(out, ref["out"], "bf16")


def test_deterministic(gpu_lib):
    cfg = CONFIGS[1]
    inp = draw_config(cfg, N=16)
    args = [dev(inp[x], cfg.dtype) for x in ("q", "k", "v", "lce_w", "lce_b")]
    say("determinism")
    o1, r1 = gpu_lib.forward(*args, cfg.heads, cfg.S, cfg.topk)
    o2, r2 = gpu_lib.forward(*args, cfg.heads, cfg.S, cfg.topk)
    import torch
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(r1, r2)


def test_host_pointer_rejected(gpu_lib):
    import ctypes
    lib = gpu_lib.load()
    buf = np.zeros(8 * 8 * 32, dtype=np.float32)
    hp = ctypes.c_void_p(buf.ctypes.data)
    say("host pointer")
    assert lib.bra_lce(hp, hp, None, 1, 8, 8, 32, 0, hp) == -7


@pytest.mark.parametrize("ci,pools,routes", [(3, 3, 3), (2, 3, 3), (4, 3, 0), (0, 3, 0), (1, 0, 0)])
def test_profile_counts(gpu_lib, ci, pools, routes):
    """Launches per forward: pool, route and attention for 8x8 regions with
    S*S = 256 (the detection shape) and for 2x2 regions (the 14x14 stage);
    with S*S <= 64 the attention kernels of 16x16 regions (the segmentation
    shape) and of fp32 8x8 regions (the 56x56 stage) choose their regions'
    routes themselves, so no route kernel runs; with 4x4 regions (the 28x28
    stage) one kernel pools, routes and attends."""
    cfg = CONFIGS[ci]
    inp = draw_config(cfg, N=4)
    args = [dev(inp[x], cfg.dtype) for x in ("q", "k", "v", "lce_w", "lce_b")]
    say(f"profile {cfg.name}")
    gpu_lib.profile_begin()
    for _ in range(3):
        gpu_lib.forward(*args, cfg.heads, cfg.S, cfg.topk)
    rec = gpu_lib.profile_read()
    gpu_lib.profile_begin(())
    assert rec["pool"][1] == pools and rec["route"][1] == routes and rec["attn"][1] == 3
    assert rec["attn"][0] > 0


def test_profile_sampling(gpu_lib):
    """profile_set_mask switches recording on and off between launches
    without discarding the record: only the sampled launches are counted."""
    cfg = CONFIGS[1]
    inp = draw_config(cfg, N=2)
    args = [dev(inp[x], cfg.dtype) for x in ("q", "k", "v", "lce_w", "lce_b")]
    say("profile sampling")
    gpu_lib.profile_begin(())
    for i in range(6):
        gpu_lib.profile_set_mask(["attn"] if i % 3 == 0 else ())
        gpu_lib.forward(*args, cfg.heads, cfg.S, cfg.topk)
    gpu_lib.profile_set_mask(())
    rec = gpu_lib.profile_read()
    assert rec["attn"][1] == 2 and rec["pool"][1] == 0 and rec["route"][1] == 0
    assert rec["attn"][0] > 0


@pytest.mark.parametrize("cfg", CONFIGS, ids=[c.name for c in CONFIGS])
def test_stage_routes_equal_forward_routes(gpu_lib, cfg):
    """bra_route(bra_region_means(q, k)) gives the same route bits as the
    routing inside bra_forward."""
    import torch
    inp = draw_config(cfg)  # full batch: large batches take the per-image routing kernel
    args = [dev(inp[x], cfg.dtype) for x in ("q", "k", "v", "lce_w", "lce_b")]
    say(cfg.name, "stage routes")
    _, r_fwd = gpu_lib.forward(*args, cfg.heads, cfg.S, cfg.topk)
    qr, kr = gpu_lib.region_means(args[0], args[1], cfg.S)
    r_stage = gpu_lib.route(qr, kr, cfg.topk)
    torch.cuda.synchronize()
    assert torch.equal(r_fwd, r_stage)


STAGE_ROUTE_CASES = [
    # name, N, H, W, C, heads, S, topk, dtype: attention kernels that route
    # their own regions, with C over several 128-channel phases of the route
    # kernel (and a partial last phase)
    ("tile16_c256", 2, 64, 64, 256, 8, 4, 2, "bf16"),
    ("tile8_c160_r64", 1, 64, 64, 160, 5, 8, 3, "bf16"),
    ("f32_c192", 2, 32, 32, 192, 6, 4, 2, "f32"),
]


@pytest.mark.parametrize("case", STAGE_ROUTE_CASES, ids=[c[0] for c in STAGE_ROUTE_CASES])
def test_stage_routes_equal_forward_routes_wide_c(gpu_lib, case):
    """The route kernel's logits (channels split into LDS a phase at a time)
    equal those of the routing inside the attention kernels bit for bit, at
    channel counts past one phase: the same route bits either way."""
    import torch
    name, N, H, W, C, heads, S, topk, dtype = case
    inp = draw(N, H, W, C, S, dtype, seed=zlib.crc32(name.encode()) % 10000, offset_std=0.7)
    args = [dev(inp[x], dtype) for x in ("q", "k", "v", "lce_w", "lce_b")]
    say(name, "stage routes")
    gpu_lib.profile_begin()
    _, r_fwd = gpu_lib.forward(*args, heads, S, topk)
    rec = gpu_lib.profile_read()
    gpu_lib.profile_begin(())
    assert rec["route"][1] == 0 and rec["attn"][1] == 1  # routed inside the attention kernel
    qr, kr = gpu_lib.region_means(args[0], args[1], S)
    r_stage = gpu_lib.route(qr, kr, topk)
    torch.cuda.synchronize()
    assert torch.equal(r_fwd, r_stage)


def test_failed_workspace_allocation_leaves_outputs_untouched(gpu_lib, monkeypatch):
    """With BRA_TEST_FAIL_ALLOC=1 the library's workspace request fails as an
    out-of-memory allocation would: bra_forward returns BRA_ERR_HIP, its
    error text names the HIP failure, and out / route_idx keep their previous
    contents (nothing was launched). Without the hook the same call works."""
    import torch
    N, H, W, C, heads, S, topk = 2, 32, 32, 64, 2, 4, 2   # 8x8 regions: pool + route + attend
    inp = draw(N, H, W, C, S, "bf16", seed=808)
    args = [dev(inp[x], "bf16") for x in ("q", "k", "v", "lce_w", "lce_b")]
    out = torch.full((N, H, W, C), 7.0, dtype=torch.bfloat16, device="cuda")
    route = torch.full((N, S * S, topk), -5, dtype=torch.int32, device="cuda")
    gpu_lib.release()                      # the next call must ask for a workspace
    monkeypatch.setenv("BRA_TEST_FAIL_ALLOC", "1")
    say("workspace allocation failure")
    with pytest.raises(gpu_lib.BraError) as ei:
        gpu_lib.forward(*args, heads, S, topk, out=out, route_idx=route)
    assert ei.value.code == -6 and "HIP failure" in str(ei.value)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all()) and bool((route == -5).all())
    monkeypatch.delenv("BRA_TEST_FAIL_ALLOC")
    gpu_lib.forward(*args, heads, S, topk, out=out, route_idx=route)
    got, r = host(out), host(route)
    ref = oracle.bra_forward(inp["q"], inp["k"], inp["v"], inp["lce_w"], inp["lce_b"], heads, S,
                             topk, route_override=r)
    check_output(got, ref["out"], "bf16")


@pytest.mark.parametrize("H,S", [(64, 4), (32, 4)], ids=["16x16_regions", "8x8_regions"])
def test_forward_bound_far_above_scores(gpu_lib, H, S):
    """Queries long along one channel of each head, keys long along another:
    |q| |k| (the bound the large-region kernel takes as its softmax maximum)
    lies hundreds of base-2 units above every real score, so the P of the
    first pass underflow and the kernel must take its exact two-pass way
    (each query's maximum score first). Routes and outputs against the
    oracle."""
    N, C, heads, topk = 2, 64, 2, 2
    inp = draw(N, H, H, C, S, "bf16", seed=5151)
    q, k = inp["q"].copy(), inp["k"].copy()
    for hh in range(heads):
        q[..., 32 * hh] = 40.0
        k[..., 32 * hh + 1] = 40.0
    inp = dict(inp, q=q, k=k)
    run_forward(gpu_lib, inp, heads, S, topk, "bf16", name=f"bound_far_{H}")
