"""The kernels' division by a fixed d through one multiply-high (FastDiv in
bra_internal.h): floor(n * ceil(2^32 / d) / 2^32) == n // d for every n and
d in [1, 2^16) (d = 1 divides by identity). Checked at every d, at the
values where a truncation error would first show: each multiple of d and the
value just below it, and the largest n."""
import numpy as np


def _fdiv(n, d):
    m = (np.uint64(1 << 32) + d - np.uint64(1)) // d
    return (n * m) >> np.uint64(32)


def test_fastdiv_exact_below_2_16():
    top = np.uint64((1 << 16) - 1)
    for d in range(2, 1 << 16):
        du = np.uint64(d)
        k = np.arange(1, (1 << 16) // d + 1, dtype=np.uint64)
        n = np.concatenate([k * du, k * du - np.uint64(1), np.array([top, 0], dtype=np.uint64)])
        n = n[n <= top]
        assert np.array_equal(_fdiv(n, du), n // du), d
