"""Parity of the projections around the operator (bra_linear, and the block
qkv -> operator -> wo) with the fp64 oracle, through the C ABI.

Linear alone, bf16: the GPU accumulates in fp32 and rounds once to bf16, so
every output lies within half a bf16 spacing of the exact value plus the fp32
accumulation error, bounded by K * 2^-23 * sum_k |x_k w_k| + 2^-24 |b|; the test
checks that bound element by element. f32: max-abs 1e-4.

The block: q, k, v and the operator's output are stored in the compute dtype
between the calls, so the oracle rounds them the same way (store="bf16");
routes then follow the near-tie protocol on the oracle's logits of the rounded
q and k, and the block output the bf16 / f32 output tolerances.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest

from oracle import bra_oracle as O
from synth import CONFIGS, draw_block, draw_linear
from tests.parity import check_output, compare_routes, half_ulp_bf16

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


def check_linear(y, x, w, b, dtype):
    ref = O.linear(x, w, b)
    if dtype == "f32":
        return check_output(y, ref, "f32")
    K = x.shape[-1]
    mag = O.linear(np.abs(x), np.abs(w), None) + np.abs(b)
    bound = half_ulp_bf16(ref) + K * 2.0 ** -23 * mag + 2.0 ** -24 * np.abs(b)
    err = np.abs(y - ref)
    bad = err > bound
    assert not bad.any(), dict(n_bad=int(bad.sum()), first=np.argwhere(bad)[:5].tolist(),
                               worst=float((err - bound).max()))
    return {"max_abs": float(err.max()), "max_over_half_ulp": float((err / half_ulp_bf16(ref)).max())}


# (name, M, K, Nout, split, dtype): ragged token counts (one token, a partial
# 64-token wave, a partial 256-token workgroup), feature counts that leave a
# partial 64-feature block, one to three outputs, K from one to several steps
LINEAR_CASES = [
    ("qkv_c64_ragged", 300, 64, 192, 64, "bf16"),
    ("qkv_c128", 1024, 128, 384, 128, "bf16"),
    ("one_token", 1, 32, 96, 32, "bf16"),
    ("wo_c64_partial_wave", 77, 64, 64, 64, "bf16"),
    ("nout_72_one_part", 257, 96, 72, 72, "bf16"),
    ("two_parts", 130, 160, 48, 24, "bf16"),
    ("k_256_max", 200, 256, 128, 128, "bf16"),
    ("qkv_c64_f32", 300, 64, 192, 64, "f32"),
    ("nout_72_f32", 257, 96, 72, 72, "f32"),
    ("one_token_f32", 1, 32, 24, 8, "f32"),
]


@pytest.mark.parametrize("case", LINEAR_CASES, ids=[c[0] for c in LINEAR_CASES])
def test_linear(gpu_lib, case):
    name, M, K, Nout, split, dtype = case
    say(name, "linear", dict(M=M, K=K, Nout=Nout, split=split, dtype=dtype))
    d = draw_linear(M, K, Nout, dtype, seed=3000 + len(name))
    ys = gpu_lib.linear(dev(d["x"], dtype), dev(d["w"], dtype), dev(d["b"], dtype), split=split)
    assert len(ys) == Nout // split
    y = np.concatenate([host(t) for t in ys], axis=-1)
    rep = check_linear(y, d["x"], d["w"], d["b"], dtype)
    say(name, rep)


def test_linear_without_bias(gpu_lib):
    say("linear_no_bias", "M=200 K=64 Nout=64 bf16")
    d = draw_linear(200, 64, 64, "bf16", seed=3100)
    (y,) = gpu_lib.linear(dev(d["x"], "bf16"), dev(d["w"], "bf16"), None)
    check_linear(host(y), d["x"], d["w"], np.zeros(64), "bf16")


@pytest.mark.parametrize("K", [96, 160])
def test_linear_infinite_weight(gpu_lib, K):
    """K % 64 == 32 (the pipelined loop's last step is a half step): a weight
    of +Inf among the first 32 columns must give +-Inf, never NaN, in its
    feature (0 * Inf would make NaN if zero rows were ever multiplied by
    step-0 weights); every other output stays within the bf16 bound."""
    M, Nout = 130, 64
    say("linear_inf_weight", dict(M=M, K=K, Nout=Nout))
    d = draw_linear(M, K, Nout, "bf16", seed=3150 + K)
    w = d["w"].copy()
    w[5, 3] = np.inf
    (y,) = gpu_lib.linear(dev(d["x"], "bf16"), dev(w, "bf16"), dev(d["b"], "bf16"))
    y = host(y)
    ref = O.linear(d["x"], w, d["b"])
    assert not np.isnan(y).any()
    assert np.array_equal(y[:, 5], ref[:, 5]), (y[:5, 5], ref[:5, 5])
    keep = [f for f in range(Nout) if f != 5]
    check_linear(y[:, keep], d["x"], d["w"][keep], d["b"][keep], "bf16")


def test_linear_full_size_qkv(gpu_lib):
    """The qkv projection at the size of the 28x28 classification stage
    (batch 128, C = 128: 100352 tokens -> 384 features), every output."""
    cfg = CONFIGS[1]
    M = cfg.N * cfg.H * cfg.W
    say("linear_full_qkv", dict(M=M, K=cfg.C, Nout=3 * cfg.C))
    d = draw_linear(M, cfg.C, 3 * cfg.C, "bf16", seed=3200)
    ys = gpu_lib.linear(dev(d["x"], "bf16"), dev(d["w"], "bf16"), dev(d["b"], "bf16"), split=cfg.C)
    y = np.concatenate([host(t) for t in ys], axis=-1)
    say("linear_full_qkv", check_linear(y, d["x"], d["w"], d["b"], "bf16"))


def test_linear_rejects_bad_shapes(gpu_lib):
    import torch
    x = torch.zeros((10, 48), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, 48), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu_lib.BraError):
        gpu_lib.linear(x, w, None)                      # K % 32 != 0
    x = torch.zeros((10, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        gpu_lib.linear(x, w, None, split=16)            # four parts
    w = torch.zeros((12, 64), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu_lib.BraError):
        gpu_lib.linear(x, w, None, split=4)             # split % 8 != 0
    x = torch.zeros((10, 288), dtype=torch.bfloat16, device="cuda")
    w = torch.zeros((64, 288), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(gpu_lib.BraError):
        gpu_lib.linear(x, w, None)                      # bf16 K > 256


def test_block_rejects_bad_arguments(gpu_lib):
    """bra_block_forward's checks return their codes before any launch and
    leave the outputs untouched: a missing weight, an unsupported width, a
    misaligned output, topk above S^2."""
    import ctypes
    import torch
    lib = gpu_lib.load()
    N, H, C, heads, S, topk = 1, 16, 64, 2, 2, 2
    dt = torch.bfloat16
    x = torch.zeros((N, H, H, C), dtype=dt, device="cuda")
    wqkv = torch.zeros((3 * C, C), dtype=dt, device="cuda")
    wo = torch.zeros((C, C), dtype=dt, device="cuda")
    lw = torch.zeros((C, 5, 5), dtype=dt, device="cuda")
    y = torch.full((N, H, H, C + 8), 3.0, dtype=dt, device="cuda")
    route = torch.full((N, S * S, topk), -9, dtype=torch.int32, device="cuda")
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    say("block argument checks")

    def call(xp, wq, wop, yp, c=C, h=heads, k=topk):
        return lib.bra_block_forward(xp, wq, None, p(lw), None, wop, None, N, H, H, c, h, S, k, 1, yp,
                                     p(route))
    # codes of include/bra.h: -1 NULL, -3 TOPK, -5 UNSUPPORTED, -8 ALIGN
    assert call(p(x), None, p(wo), p(y)) == -1                               # no qkv weight
    assert call(p(x), p(wqkv), p(wo), ctypes.c_void_p(y.data_ptr() + 8)) == -8  # y not 16-byte aligned
    assert call(p(x), p(wqkv), p(wo), p(y), k=S * S + 1) == -3              # topk > S^2
    assert call(p(x), p(wqkv), p(wo), p(y), c=288, h=9) == -5               # bf16 C > 256
    torch.cuda.synchronize()
    assert bool((y == 3.0).all()) and bool((route == -9).all())


def run_block(bra, d, heads, S, topk, dtype, images=None, name=""):
    x = d["x"]
    say(name, "block", x.shape, f"heads={heads} S={S} topk={topk} {dtype}")
    args = [dev(d[k], dtype) for k in ("x", "wqkv", "bqkv", "lce_w", "lce_b", "wo", "bo")]
    y, route = bra.block_forward(*args, heads, S, topk)
    y, route = host(y), host(route)
    imgs = list(range(x.shape[0])) if images is None else images
    store = "bf16" if dtype == "bf16" else None
    blk = (x[imgs], d["wqkv"], d["bqkv"], d["lce_w"], d["lce_b"], d["wo"], d["bo"], heads, S, topk)
    own = O.bra_block_forward(*blk, store=store)
    exact, near, fails = compare_routes(route[imgs], own["logits"], own["route_oracle"])
    assert not fails, fails[:5]
    ref = O.bra_block_forward(*blk, store=store, route_override=route[imgs])
    rep = check_output(y[imgs], ref["out"], dtype)
    rep.update(exact_rows=exact, near_tie_rows=near)
    say(name, rep)
    return rep


# (name, N, H, C, heads, S, topk, dtype, fused): the one-kernel 4x4-region
# path (S = 7 at H = 28) and fp32 run as three steps; two heads with 8x8 or
# 16x16 regions run fused (qkv + pooling, routing, attention + wo): a token
# count that leaves the last projection workgroup partly empty (24x24, 8x8
# regions), whole-region routing (topk = S^2), 16x16 regions with two slabs
# and a ragged topk
BLOCK_CASES = [
    ("block_4x4_c128_t4", 2, 28, 128, 4, 7, 4, "bf16", False),
    ("block_f32_c64_t1", 1, 16, 64, 2, 2, 1, "f32", False),
    ("block_8x8_c128_t2", 1, 32, 128, 4, 4, 2, "bf16", False),
    ("block_fused_8x8_t2", 1, 32, 64, 2, 4, 2, "bf16", True),
    ("block_fused_8x8_ragged", 1, 24, 64, 2, 3, 4, "bf16", True),
    ("block_fused_8x8_all", 2, 16, 64, 2, 2, 4, "bf16", True),
    ("block_fused_16x16_t3", 2, 48, 64, 2, 3, 3, "bf16", True),
    ("block_fused_16x16_t1", 1, 32, 64, 2, 2, 1, "bf16", True),
]


@pytest.mark.parametrize("case", BLOCK_CASES, ids=[c[0] for c in BLOCK_CASES])
def test_block_small(gpu_lib, case):
    import torch
    name, N, H, C, heads, S, topk, dtype, fused = case
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    assert gpu_lib.block_fused(N, H, H, C, heads, S, topk, tdt) == fused
    d = draw_block(N, H, H, C, S, dtype, seed=3300 + len(name))
    run_block(gpu_lib, d, heads, S, topk, dtype, name=name)


def test_block_fused_full_size(gpu_lib):
    """The fused block at the segmentation workload's shape (8 images of
    128x128 tokens, C = 64, two heads, 16x16 regions, topk 4); the oracle
    checks every image, routes and outputs."""
    import torch
    cfg = CONFIGS[4]
    assert gpu_lib.block_fused(cfg.N, cfg.H, cfg.W, cfg.C, cfg.heads, cfg.S, cfg.topk, torch.bfloat16)
    d = draw_block(cfg.N, cfg.H, cfg.W, cfg.C, cfg.S, "bf16", seed=3500, offset_std=cfg.offset_std,
                   w_std=cfg.w_std, b_std=cfg.b_std)
    run_block(gpu_lib, d, cfg.heads, cfg.S, cfg.topk, "bf16", name="block_full_c4")


def test_block_full_size(gpu_lib):
    """The block at the 28x28 classification stage's full batch (128 images);
    the oracle checks every image, routes and outputs."""
    cfg = CONFIGS[1]
    d = draw_block(cfg.N, cfg.H, cfg.W, cfg.C, cfg.S, "bf16", seed=3400, w_std=cfg.w_std,
                   b_std=cfg.b_std)
    run_block(gpu_lib, d, cfg.heads, cfg.S, cfg.topk, "bf16", name="block_full_c1")
