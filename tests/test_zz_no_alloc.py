"""bra_forward_noalloc (the forward for callers that cannot allocate) against
bra_forward, through the C ABI: the same kernels run on a static device
scratch array instead of the library's allocated workspace, so routes and
outputs must be bit-identical, on two calls in a row (the second smaller, so
it runs over the first call's leftovers in the array), and a shape whose
workspace exceeds the array is refused before any launch."""
from __future__ import annotations

import ctypes
import sys

import numpy as np
import pytest

from synth import draw

pytestmark = pytest.mark.gpu


def say(*a):
    print("[case]", *a, file=sys.stderr, flush=True)


def dev(x, dtype="bf16"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float32)))
    return t.to(device="cuda", dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)


def call(lib, name, t, heads, S, topk, dtype, out, route):
    import torch
    from vision_transformer_sparse_amd import bra
    N, H, W, C = t["q"].shape
    with torch.cuda.device(t["q"].device):
        lib.bra_set_stream(ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        p = [ctypes.c_void_p(t[x].data_ptr()) for x in ("q", "k", "v", "lce_w", "lce_b")]
        return getattr(lib, name)(*p, N, H, W, C, heads, S, topk,
                                  bra.BF16 if dtype == "bf16" else bra.F32,
                                  ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(route.data_ptr()))


def both(gpu_lib, shape, seed, dtype="bf16", off=0.0):
    import torch
    N, H, W, C, heads, S, topk = shape
    lib = gpu_lib.load()
    inp = draw(N, H, W, C, S, dtype, seed=seed, offset_std=off)
    t = {k: dev(v, dtype) for k, v in inp.items()}
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    o_ref = torch.empty((N, H, W, C), dtype=tdt, device="cuda")
    r_ref = torch.empty((N, S * S, topk), dtype=torch.int32, device="cuda")
    o_na = torch.full_like(o_ref, 3.0)
    r_na = torch.full_like(r_ref, -1)
    say("noalloc", shape, dtype)
    assert call(lib, "bra_forward", t, heads, S, topk, dtype, o_ref, r_ref) == 0
    assert call(lib, "bra_forward_noalloc", t, heads, S, topk, dtype, o_na, r_na) == 0
    torch.cuda.synchronize()
    assert torch.equal(r_na, r_ref)
    assert torch.equal(o_na.view(torch.int16 if dtype == "bf16" else torch.int32),
                       o_ref.view(torch.int16 if dtype == "bf16" else torch.int32))


@pytest.mark.parametrize("big,small", [
    # 2x2 regions of 14x14 images (pool + route + image-resident attention):
    # 16 images, then 4
    ((16, 14, 14, 256, 8, 7, 16), (4, 14, 14, 256, 8, 7, 16)),
    # 16x16 regions (the large-region kernel), then 8x8 regions
    ((2, 64, 64, 64, 2, 4, 4), (1, 32, 32, 64, 2, 4, 2)),
    # fp32, then a ragged smaller fp32 shape
    ((1, 56, 56, 64, 2, 7, 1), (2, 15, 10, 64, 2, 5, 3)),
], ids=["2x2_regions", "16x16_then_8x8", "f32"])
def test_noalloc_matches_forward_twice(gpu_lib, big, small):
    dtype = "f32" if big[0] == 1 and big[1] == 56 else "bf16"
    both(gpu_lib, big, seed=61, dtype=dtype, off=0.7)
    both(gpu_lib, small, seed=62, dtype=dtype)


def test_noalloc_one_kernel_shape(gpu_lib):
    """4x4 regions run as one kernel with no workspace at all."""
    both(gpu_lib, (4, 28, 28, 128, 4, 7, 4), seed=63)


def test_noalloc_refuses_oversized_workspace(gpu_lib):
    """256 images of 14x14x256 need 2*256*49*256*4 bytes of region means
    (25.7 MB) > BRA_NOALLOC_SCRATCH_BYTES (16 MiB): BRA_ERR_SCRATCH, nothing
    launched, outputs untouched."""
    import torch
    N, H, W, C, heads, S, topk = 256, 14, 14, 256, 8, 7, 16
    lib = gpu_lib.load()
    assert lib.bra_workspace_bytes(N, C, S) > (16 << 20)
    z = torch.zeros((N, H, W, C), dtype=torch.bfloat16, device="cuda")
    t = {"q": z, "k": z, "v": z, "lce_w": torch.zeros((C, 5, 5), dtype=torch.bfloat16, device="cuda"),
         "lce_b": torch.zeros((C,), dtype=torch.bfloat16, device="cuda")}
    out = torch.full_like(z, 5.0)
    route = torch.full((N, S * S, topk), -2, dtype=torch.int32, device="cuda")
    say("noalloc oversized")
    assert call(lib, "bra_forward_noalloc", t, heads, S, topk, "bf16", out, route) == -9
    assert b"scratch" in lib.bra_error_string(-9)
    torch.cuda.synchronize()
    assert bool((out == 5.0).all()) and bool((route == -2).all())


def test_noalloc_records_no_events(gpu_lib):
    """With every kernel kind profiled, the allocation-free call creates and
    records no events (bra_forward would record its three launches)."""
    import torch
    N, H, W, C, heads, S, topk = 2, 32, 32, 64, 2, 4, 2
    lib = gpu_lib.load()
    t = {k: dev(v) for k, v in draw(N, H, W, C, S, "bf16", seed=64).items()}
    out = torch.empty((N, H, W, C), dtype=torch.bfloat16, device="cuda")
    route = torch.empty((N, S * S, topk), dtype=torch.int32, device="cuda")
    say("noalloc no events")
    gpu_lib.profile_begin()
    assert call(lib, "bra_forward_noalloc", t, heads, S, topk, "bf16", out, route) == 0
    rec = gpu_lib.profile_read()
    gpu_lib.profile_begin(())
    assert all(cnt == 0 for _, cnt in rec.values()), rec
