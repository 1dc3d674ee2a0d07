"""The per-head routing variant (bra_forward_head_routed) against the fp64
oracle's bra_forward_head_routed, through the C ABI: every head's routes
under the near-tie protocol (accepted rows fed back to the oracle), then the
outputs at the stated tolerances.

Every case prints its name before touching the GPU."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
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


def run_head_routed(bra, inp, heads, S, topk, dtype, name):
    say(name, "head-routed", inp["q"].shape, f"heads={heads} S={S} topk={topk} {dtype}")
    out, route = bra.forward_head_routed(*[dev(inp[x], dtype) for x in ("q", "k", "v", "lce_w", "lce_b")],
                                         heads, S, topk)
    out, route = host(out), host(route)
    ref = oracle.bra_forward_head_routed(inp["q"], inp["k"], inp["v"], inp["lce_w"], inp["lce_b"],
                                         heads, S, topk)
    exact = near = 0
    for m in range(heads):
        e, nr, fails = compare_routes(route[:, m], ref["logits"][:, m], ref["route_oracle"][:, m])
        assert not fails, (m, fails[:5])
        exact, near = exact + e, near + nr
    assert exact + near == route.shape[0] * heads * S * S
    if near:
        ref = oracle.bra_forward_head_routed(inp["q"], inp["k"], inp["v"], inp["lce_w"], inp["lce_b"],
                                             heads, S, topk, route_override=route)
    rep = check_output(out, ref["out"], dtype)
    rep.update(exact_rows=exact, near_tie_rows=near)
    say(name, rep)
    return out, route


# (N, H, W, C, heads, S, topk, dtype): ragged region counts, topk = 1 and S^2,
# 4x4, 8x8 and 16x16 regions, fp32 and bf16; the bf16 8x8 / 16x16 cases with
# S*S <= 64 run the one-pass path (the attention kernel routes each head)
CASES = [
    (2, 16, 16, 64, 2, 4, 3, "bf16"),
    (1, 12, 12, 96, 3, 3, 9, "f32"),
    (2, 28, 28, 128, 4, 7, 4, "bf16"),
    (1, 32, 32, 64, 2, 2, 1, "f32"),
    (1, 40, 40, 64, 2, 5, 2, "bf16"),
    (2, 14, 14, 96, 3, 7, 16, "bf16"),
    (1, 32, 32, 96, 3, 2, 2, "bf16"),
    (1, 24, 24, 64, 2, 3, 9, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:7])) + "_" + c[7])
def test_head_routed_small(gpu_lib, case):
    N, H, W, C, heads, S, topk, dtype = case
    inp = draw(N, H, W, C, S, dtype, seed=800 + H + C + topk)
    run_head_routed(gpu_lib, inp, heads, S, topk, dtype, f"head-routed {case}")


@pytest.mark.parametrize("ci", [4, 2])
def test_head_routed_full_config(gpu_lib, ci):
    """The segmentation (c4) and 14x14 classification (c2) shapes with every
    head routed on its own channels, every image against the oracle."""
    cfg = CONFIGS[ci]
    inp = draw_config(cfg)
    run_head_routed(gpu_lib, inp, cfg.heads, cfg.S, cfg.topk, cfg.dtype, f"{cfg.name} head-routed")


def test_head_routed_one_head_equals_forward(gpu_lib):
    """With one head the variant is the operator: same route bits and the
    same output bits as bra_forward."""
    import torch
    N, H, W, C, S, topk = 2, 32, 32, 32, 4, 3
    inp = draw(N, H, W, C, S, "bf16", seed=851)
    args = [dev(inp[x], "bf16") for x in ("q", "k", "v", "lce_w", "lce_b")]
    say("head-routed one head vs forward")
    o1, r1 = gpu_lib.forward_head_routed(*args, 1, S, topk)
    o2, r2 = gpu_lib.forward(*args, 1, S, topk)
    torch.cuda.synchronize()
    assert torch.equal(r1[:, 0], r2) and torch.equal(o1, o2)


def test_head_routed_one_pass_launches(gpu_lib):
    """On the large-region shapes with S*S <= 64 the variant is one pooling
    and one attention launch (no per-head copies or launches)."""
    cfg = CONFIGS[4]
    inp = draw_config(cfg, N=2)
    args = [dev(inp[x], "bf16") for x in ("q", "k", "v", "lce_w", "lce_b")]
    say("head-routed launches")
    gpu_lib.profile_begin()
    gpu_lib.forward_head_routed(*args, cfg.heads, cfg.S, cfg.topk)
    rec = gpu_lib.profile_read()
    gpu_lib.profile_begin(())
    assert rec["pool"][1] == 1 and rec["attn"][1] == 1 and rec["route"][1] == 0
