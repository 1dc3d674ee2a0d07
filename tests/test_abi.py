"""The C-ABI library without a GPU: it loads, exports every entry point that
include/bra.h declares, and rejects invalid arguments with the documented
status codes before any HIP call (no compute is launched here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bra.h")
LIB = os.path.join(ROOT, "vision_transformer_sparse_amd", "libbra.so")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(bra_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(LIB):
        pytest.fail("libbra.so not built (python -m vision_transformer_sparse_amd.build)")
    from vision_transformer_sparse_amd import bra
    return bra.load()


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("bra_forward", "bra_set_stream", "bra_workspace_bytes",
                     "bra_release", "bra_error_string"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", LIB], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(bra_\w+)", out))
    missing = [n for n in declared_functions() if n not in exported]
    assert not missing, missing
    from vision_transformer_sparse_amd import bra
    assert sorted(bra.EXPORTED) == declared_functions()


def test_version_and_strings(lib):
    assert lib.bra_version() >= 100
    for code in (0, -1, -2, -3, -4, -5, -7, 42):
        assert lib.bra_error_string(code)


def test_workspace_bytes(lib):
    # region means of q and k, the per-(image, region, head) key norms, then
    # the packed LCE weights (30*C + 25*C/2 + 80*C dwords); parts 256-aligned
    assert lib.bra_workspace_bytes(128, 128, 7) == 2 * 128 * 49 * 128 * 4 + 128 * 49 * 4 * 4 + 490 * 128
    # 2*1*4*64*4 = 2048 bytes of means, 1*4*2*4 = 32 bytes of norms padded to 256
    assert lib.bra_workspace_bytes(1, 64, 2) == 2048 + 256 + 490 * 64
    assert lib.bra_workspace_bytes(0, 128, 7) == 0


P = ctypes.c_void_p(4096)  # never dereferenced: every case fails before HIP


@pytest.mark.parametrize("args,code", [
    # q, k, v, w, b, N, H, W, C, heads, S, topk, dtype, out, route
    ((None, P, P, P, None, 1, 8, 8, 64, 2, 2, 1, 1, P, P), -1),
    ((P, P, P, None, None, 1, 8, 8, 64, 2, 2, 1, 1, P, P), -1),
    ((P, P, P, P, None, 1, 8, 8, 64, 2, 2, 1, 1, None, P), -1),
    ((P, P, P, P, None, 1, 8, 8, 64, 2, 2, 1, 1, P, None), -1),
    ((P, P, P, P, None, 0, 8, 8, 64, 2, 2, 1, 1, P, P), -2),
    ((P, P, P, P, None, 1, 9, 8, 64, 2, 2, 1, 1, P, P), -2),
    ((P, P, P, P, None, 1, 8, 9, 64, 2, 2, 1, 1, P, P), -2),
    ((P, P, P, P, None, 1, 8, 8, 64, 3, 2, 1, 1, P, P), -2),
    ((P, P, P, P, None, 1, 8, 8, 64, 2, 0, 1, 1, P, P), -2),
    ((P, P, P, P, None, 1, 8, 8, 64, 2, 2, 0, 1, P, P), -3),
    ((P, P, P, P, None, 1, 8, 8, 64, 2, 2, 5, 1, P, P), -3),
    ((P, P, P, P, None, 1, 8, 8, 64, 2, 2, 1, 7, P, P), -4),
    ((P, P, P, P, None, 1, 8, 8, 128, 2, 2, 1, 1, P, P), -5),   # head_dim 64
    ((P, P, P, P, None, 1, 64, 64, 64, 2, 64, 1, 1, P, P), -5),  # S*S > 1024
])
def test_forward_rejects(lib, args, code):
    assert lib.bra_forward(*args) == code


def test_misaligned_pointers_rejected(lib):
    M = ctypes.c_void_p(4096 + 2)
    assert lib.bra_forward(M, P, P, P, None, 1, 8, 8, 64, 2, 2, 1, 1, P, P) == -8
    assert lib.bra_forward(P, P, P, P, ctypes.c_void_p(4097), 1, 8, 8, 64, 2, 2, 1, 1, P, P) == -8
    assert lib.bra_forward(P, P, P, P, None, 1, 8, 8, 64, 2, 2, 1, 1, P, ctypes.c_void_p(4098)) == -8
    assert lib.bra_lce(P, P, None, 1, 8, 8, 64, 1, M) == -8


def test_stage_entry_points_reject(lib):
    assert lib.bra_route(None, P, 1, 4, 32, 1, P) == -1
    assert lib.bra_route(P, P, 1, 4, 32, 5, P) == -3
    assert lib.bra_route(P, P, 1, 2048, 32, 1, P) == -5
    assert lib.bra_region_means(P, P, 1, 8, 8, 64, 3, 1, P, P) == -2
    assert lib.bra_attend(P, P, P, P, None, None, 1, 8, 8, 64, 2, 2, 1, 1, P) == -1
    assert lib.bra_lce(P, P, None, 1, 8, 8, 64, 3, P) == -4
    assert lib.bra_calib_copy(P, P, 15) == -2


def test_stream_roundtrip(lib):
    assert lib.bra_set_stream(None) == 0
    assert lib.bra_get_stream() is None


def test_binding_refuses_host_tensors():
    import torch
    from vision_transformer_sparse_amd import bra
    x = torch.zeros(1, 8, 8, 32)
    with pytest.raises(ValueError):
        bra.forward(x, x, x, torch.zeros(32, 5, 5), None, 1, 2, 1)
