"""The backward for given routes (bra_backward) against the fp64 oracle's
bra_backward, through the C ABI. Routes come from the GPU forward on the
same inputs and are handed to both sides (the router gets no gradient).

Tolerances: dq, dk, dv are bf16 outputs and take the bf16 rule of the
forward (per element 2e-2, relative L2 5e-3). dlce_w and dlce_b are fp32 sums
over every pixel of the batch: per element |gpu - oracle| <= 1e-4 times the
sum of the absolute products (fp32 accumulation of up to 1.3e5 terms in a
fixed order; the worst case n * 2^-24 would be 8e-3).

Every case prints its name before touching the GPU."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from synth import CONFIGS, draw, draw_config
from tests.parity import check_output

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def dev(x, dtype="bf16"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def host(t):
    import torch
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def lce_grad_bounds(v, g):
    """Sum over pixels of |dout * v shifted| per (channel, tap), and of |dout|."""
    N, H, W, C = v.shape
    vp = np.zeros((N, H + 4, W + 4, C))
    vp[:, 2:H + 2, 2:W + 2] = np.abs(v)
    ag = np.abs(g)
    bw = np.stack([(ag * vp[:, a:a + H, e:e + W]).sum(axis=(0, 1, 2)) for a in range(5) for e in range(5)], 1)
    return bw, ag.sum(axis=(0, 1, 2))


def run_backward(bra, inp, dout, heads, S, topk, name):
    say(name, "backward", inp["q"].shape, f"heads={heads} S={S} topk={topk}")
    t = {x: dev(inp[x]) for x in ("q", "k", "v", "lce_w", "lce_b")}
    _, route = bra.forward(t["q"], t["k"], t["v"], t["lce_w"], t["lce_b"], heads, S, topk)
    dq, dk, dv, dw, db = bra.backward(t["q"], t["k"], t["v"], t["lce_w"], route, dev(dout), heads, S)
    route = host(route)
    ref = oracle.bra_backward(inp["q"], inp["k"], inp["v"], inp["lce_w"], route, dout, heads, S)
    rep = {}
    for key, got in (("dq", dq), ("dk", dk), ("dv", dv)):
        rep[key] = check_output(host(got), ref[key], "bf16")
    bw, bb = lce_grad_bounds(inp["v"], dout)
    ew = np.abs(host(dw) - ref["dlce_w"].reshape(-1, 25))
    eb = np.abs(host(db) - ref["dlce_b"])
    assert np.all(ew <= 1e-4 * bw + 1e-6), float((ew / (bw + 1e-30)).max())
    assert np.all(eb <= 1e-4 * bb + 1e-6), float((eb / (bb + 1e-30)).max())
    rep["dlce_w_rel_max"] = float((ew / (bw + 1e-30)).max())
    say(name, rep)


def dout_for(inp, seed):
    return draw(*inp["q"].shape[:3], inp["q"].shape[3], 1, "bf16", seed=seed)["q"]


# (N, H, W, C, heads, S, topk): 4x4 regions (T = 16; topk odd -> a half key
# tile), 8x8 and 16x16 regions, regions that nobody routes to (topk 1)
CASES = [
    (2, 16, 16, 64, 2, 4, 3),
    (1, 32, 32, 64, 2, 4, 4),
    (1, 32, 32, 32, 1, 2, 2),
    (2, 28, 28, 128, 4, 7, 4),
    (1, 24, 24, 64, 2, 3, 1),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_backward_small(gpu_lib, case):
    N, H, W, C, heads, S, topk = case
    inp = draw(N, H, W, C, S, "bf16", seed=900 + H + C + topk, offset_std=0.7)
    run_backward(gpu_lib, inp, dout_for(inp, 950 + H + topk), heads, S, topk, f"backward {case}")


@pytest.mark.parametrize("ci,N", [(4, None), (1, 8)])
def test_backward_config(gpu_lib, ci, N):
    """The segmentation workload (c4, every image) and the 28x28
    classification stage (c1's shape, 8 images)."""
    cfg = CONFIGS[ci]
    inp = draw_config(cfg, N=N)
    run_backward(gpu_lib, inp, dout_for(inp, 990 + ci), cfg.heads, cfg.S, cfg.topk, f"{cfg.name} backward")


def test_backward_deterministic(gpu_lib):
    import torch
    N, H, W, C, heads, S, topk = 2, 32, 32, 64, 2, 4, 4
    inp = draw(N, H, W, C, S, "bf16", seed=961)
    t = {x: dev(inp[x]) for x in ("q", "k", "v", "lce_w", "lce_b")}
    say("backward determinism")
    _, route = gpu_lib.forward(t["q"], t["k"], t["v"], t["lce_w"], t["lce_b"], heads, S, topk)
    g = dev(dout_for(inp, 962))
    a = gpu_lib.backward(t["q"], t["k"], t["v"], t["lce_w"], route, g, heads, S)
    b = gpu_lib.backward(t["q"], t["k"], t["v"], t["lce_w"], route, g, heads, S)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))


def test_backward_unsupported_shapes(gpu_lib):
    """2x2 regions (T = 4) and fp32 are outside the backward kernels."""
    say("backward unsupported")
    for dtype, (H, S) in (("bf16", (14, 7)), ("f32", (16, 4))):
        inp = draw(1, H, H, 64, S, dtype, seed=963)
        t = {x: dev(inp[x], dtype) for x in ("q", "k", "v", "lce_w")}
        import torch
        route = torch.zeros((1, S * S, 1), dtype=torch.int32, device="cuda")
        with pytest.raises(gpu_lib.BraError) as ei:
            gpu_lib.backward(t["q"], t["k"], t["v"], t["lce_w"], route, t["q"], 2, S)
        assert ei.value.code == -5
