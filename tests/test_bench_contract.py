"""bench.py's host-side contract, without a GPU: more than one GPU is refused
with a message, and the roofline arithmetic follows its definition
(algorithmic bytes or flops per launch over the launch time)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr and r.stdout == ""


def test_roofline_arithmetic():
    import bench
    from synth import CONFIGS
    cfgs = {c.name: c for c in CONFIGS}
    c1 = cfgs["c1"]
    # c1: q, k, v read and out written once (bf16), routes and LCE parameters
    E = c1.N * c1.H * c1.W * c1.C
    alg = bench.algorithmic(c1)["attn"]["bytes"]
    assert alg == 4 * E * 2 + c1.N * c1.R * c1.topk * 4 + c1.C * 26 * 2
    r = bench.roofline_for("attn", c1, 0.05, None)  # 50 us a launch
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["achieved"] - alg / 50e-6 / 1e9) < 1e-6
    assert abs(r["frac"] - r["achieved"] / 8000.0) < 1e-12
    # c4 is past the bf16 ridge point: it is priced against the matrix cores
    c4 = cfgs["c4"]
    r4 = bench.roofline_for("attn", c4, 0.07, None)
    assert r4["bound"] == "mfma" and r4["unit"] == "TFLOP/s" and r4["peak"] == 2500.0
    flops = 4 * c4.N * c4.H * c4.W * c4.C * c4.L
    assert abs(r4["achieved"] - flops / 70e-6 / 1e12) < 1e-6


def test_projection_roofline_arithmetic():
    """The block's two projections per step: qkv reads x (E elements) and
    writes q, k, v (3E), wo reads o and writes y (2E), plus 4C^2 weights and 4C
    biases; 8EC flops. Reported per launch (half of that) against HBM: at
    C = 128 the intensity (about 2C/3 flop per byte) is far below the ridge."""
    import bench
    from synth import CONFIGS
    c1 = CONFIGS[1]
    E = c1.N * c1.H * c1.W * c1.C
    alg = bench.algorithmic(c1)["linear"]
    assert alg["bytes"] == (6 * E + 4 * c1.C * c1.C + 4 * c1.C) * 2 / 2
    assert alg["flops"] == 8 * E * c1.C / 2
    r = bench.roofline_for("linear", c1, 0.01, None)
    assert r["bound"] == "hbm" and abs(r["achieved"] - alg["bytes"] / 10e-6 / 1e9) < 1e-6
