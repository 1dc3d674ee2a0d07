"""The router-free last-stage attention (bra_attention_dense) against the
fp64 oracle's dense_attention, through the C ABI.

Every case prints its name before touching the GPU. Inputs come from the
seeded generator in synth/ (S = 1: the whole map is one region)."""
from __future__ import annotations

import sys

import numpy as np
import pytest

import oracle
from synth import STAGE4, draw, draw_config
from tests.parity import check_output

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
    return t.float().cpu().numpy().astype(np.float64)


def run_dense(bra, inp, heads, dtype, name):
    say(name, "dense", inp["q"].shape, f"heads={heads} {dtype}")
    args = [dev(inp[x], dtype) for x in ("q", "k", "v", "lce_w", "lce_b")]
    out = host(bra.attention_dense(*args, heads))
    ref = oracle.dense_attention(inp["q"], inp["k"], inp["v"], inp["lce_w"], inp["lce_b"], heads)
    rep = check_output(out, ref, dtype)
    say(name, rep)
    return out


# (N, H, W, C, heads, dtype): the dense kernel's range (bf16, <= 256 tokens) with
# ragged query and key tiles, 1x1 and 16x16 maps; then the routed fallback
# (fp32, and a bf16 map of more than 256 tokens)
CASES = [
    (2, 7, 7, 64, 2, "bf16"),
    (3, 5, 9, 96, 3, "bf16"),
    (2, 1, 1, 32, 1, "bf16"),
    (1, 16, 16, 64, 2, "bf16"),
    (2, 12, 12, 128, 4, "bf16"),
    (1, 3, 20, 64, 2, "bf16"),
    (2, 2, 17, 32, 1, "bf16"),
    (2, 7, 7, 64, 2, "f32"),
    (1, 20, 20, 64, 2, "bf16"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c[:5])) + "_" + c[5])
def test_dense_small(gpu_lib, case):
    N, H, W, C, heads, dtype = case
    inp = draw(N, H, W, C, 1, dtype, seed=700 + H * W + C)
    run_dense(gpu_lib, inp, heads, dtype, f"dense {case}")


def test_dense_stage4_full(gpu_lib):
    """The full last-stage workload (128 images of 7x7 tokens, C = 512, 16
    heads), every image against the oracle."""
    inp = draw_config(STAGE4)
    run_dense(gpu_lib, inp, STAGE4.heads, STAGE4.dtype, "stage-4 full")


def test_dense_equals_all_regions_routed(gpu_lib):
    """bra_forward with every region routed (S = 7 on a 7x7 map: one token a
    region, topk = 49) computes the same attention in another key order: both
    agree with the oracle and with each other to the bf16 bound."""
    import torch
    N, H, W, C, heads = 4, 7, 7, 64, 2
    inp = draw(N, H, W, C, 7, "bf16", seed=731)
    args = [dev(inp[x], "bf16") for x in ("q", "k", "v", "lce_w", "lce_b")]
    say("dense vs routed topk=S^2")
    dense = host(gpu_lib.attention_dense(*args, heads))
    routed, route = gpu_lib.forward(*args, heads, 7, 49)
    routed = host(routed)
    torch.cuda.synchronize()
    ref = oracle.dense_attention(inp["q"], inp["k"], inp["v"], inp["lce_w"], inp["lce_b"], heads)
    check_output(dense, ref, "bf16")
    check_output(routed, ref, "bf16")
    assert np.abs(dense - routed).max() <= 2e-2


def test_dense_deterministic_and_no_write_past_out(gpu_lib):
    """Two calls give the same bits, and the bytes after out stay untouched."""
    import torch
    N, H, W, C, heads = 3, 7, 7, 64, 2
    inp = draw(N, H, W, C, 1, "bf16", seed=732)
    args = [dev(inp[x], "bf16") for x in ("q", "k", "v", "lce_w", "lce_b")]
    say("dense determinism")
    buf = torch.full((N * H * W * C + 4096,), 3.0, dtype=torch.bfloat16, device="cuda")
    out = buf[:N * H * W * C].view(N, H, W, C)
    gpu_lib.attention_dense(*args, heads, out=out)
    o1 = out.clone()
    gpu_lib.attention_dense(*args, heads, out=out)
    torch.cuda.synchronize()
    assert torch.equal(o1, out)
    assert torch.all(buf[N * H * W * C:] == 3.0)


def test_dense_rejects_bad_heads(gpu_lib):
    inp = draw(1, 7, 7, 64, 1, "bf16", seed=733)
    args = [dev(inp[x], "bf16") for x in ("q", "k", "v", "lce_w", "lce_b")]
    say("dense bad heads")
    with pytest.raises(gpu_lib.BraError) as ei:
        gpu_lib.attention_dense(*args, 3)
    assert ei.value.code == -2
    with pytest.raises(gpu_lib.BraError) as ei:
        gpu_lib.attention_dense(*args, 1)   # head_dim 64: outside the compiled envelope
    assert ei.value.code == -5
