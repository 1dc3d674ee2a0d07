"""The comparison rules themselves (CPU only)."""
import numpy as np
import pytest

from tests.parity import check_output, compare_routes, half_ulp_bf16


def test_routes_exact_and_near_tie():
    A = np.array([[[3.0, 2.0, 2.0 + 5e-6, 0.0]]])
    own = np.array([[[0, 2]]])
    assert compare_routes(own, A, own) == (1, 0, [])
    # GPU picked region 1, within 1e-5 of region 2: accepted
    ex, near, fails = compare_routes(np.array([[[0, 1]]]), A, own)
    assert (ex, near, fails) == (0, 1, [])
    # GPU picked region 3, far below: rejected
    ex, near, fails = compare_routes(np.array([[[0, 3]]]), A, own)
    assert near == 0 and len(fails) == 1
    # duplicated index: rejected
    assert compare_routes(np.array([[[0, 0]]]), A, own)[2]
    # out-of-range index: rejected
    assert compare_routes(np.array([[[0, 4]]]), A, own)[2]
    # swapped order of well-separated logits: rejected
    assert compare_routes(np.array([[[2, 0]]]), A, own)[2]


def test_half_ulp():
    assert half_ulp_bf16(np.array([1.0]))[0] == 2.0 ** -8
    assert half_ulp_bf16(np.array([-9.5]))[0] == 2.0 ** -5


def test_output_tolerances():
    ref = np.concatenate([[0.5, -3.0, 9.0], np.full(100, 2.0)])
    d = np.zeros_like(ref)
    d[:3] = [0.019, -0.019, 0.04]
    check_output(ref + d, ref, "bf16")
    d[:3] = [0.021, 0.0, 0.0]
    with pytest.raises(AssertionError):
        check_output(ref + d, ref, "bf16")
    d[:3] = [0.0, 0.0, 0.06]
    with pytest.raises(AssertionError):
        check_output(ref + d, ref, "bf16")
    with pytest.raises(AssertionError):   # small everywhere, but too large in L2
        check_output(ref + 0.015, ref, "bf16")
    check_output(ref + 9e-5, ref, "f32")
    with pytest.raises(AssertionError):
        check_output(ref + 2e-4, ref, "f32")
