"""Throughput of the BRA forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c1]

A step is one bra_forward call -- region pooling, routing, gathered attention
and LCE -- over one batch of seeded synthetic input already resident in HBM.
W untimed steps, then K steps timed between two device synchronisations.
One JSON line is printed. It carries:
  value      whole-job queries/s (a query is one token position, N*H*W per step)
  roofline   the attention kernel's (the dominant kernel's) algorithmic bytes
             (or flops) per launch over its mean launch time, measured with HIP
             events on the launch stream on every PROFILE_EVERY-th step of the
             timed region (the library launches a timed kernel with
             hipExtLaunchKernelGGL, which ties the event pair to that dispatch);
             the other kernels are timed the same way in a separate pass after
             it (the "kernels" object)
  cpu_baseline  the fp64 CPU oracle timed on whole-batch passes of the same
             workload (about 10 s of CPU work)
Other workloads: --config c0..c4 (c1 is the default).
--op block times the block around the operator instead: the qkv projection
(Linear C -> 3C, bra_linear), bra_forward, and the output projection (Linear
C -> C); "kernels" then also holds the projection kernel's roofline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "BRA forward queries/sec at 1 MI355X; % of MFMA peak (attn) and HBM GB/s (route)"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
FP32_PEAK_TFLOPS = 157.3
PROFILE_EVERY = 4
ATTN_SOURCES = ("attn_image.hip", "attn_region.hip", "attn_tile.hip", "attn_mfma.hip", "attn_valu.hip",
                "attn_f32.hip", "bra_internal.h", "route_common.h")


def algorithmic(cfg):
    """Per-launch algorithmic traffic / work of each kernel (what the method
    must move or compute, not what a dense method would)."""
    b = 2 if cfg.dtype == "bf16" else 4
    E = cfg.N * cfg.H * cfg.W * cfg.C
    means = 2 * cfg.N * cfg.R * cfg.C * 4
    routes = cfg.N * cfg.R * cfg.topk * 4
    lce_params = cfg.C * 26 * b
    return {
        "pool": {"bytes": 2 * E * b + means},
        "route": {"bytes": means + routes, "flops": 2 * cfg.N * cfg.R * cfg.R * cfg.C},
        "attn": {"bytes": 4 * E * b + routes + lce_params, "flops": 4 * E * cfg.L + 50 * E},
        # the block's two projections, averaged per launch: qkv reads x and
        # writes q, k, v; wo reads o and writes y (weights and biases once)
        "linear": {"bytes": (4 * E + 4 * cfg.C * (cfg.C + 1) + 2 * E) * b / 2,
                   "flops": 2 * E * 4 * cfg.C / 2},
    }


def roofline_for(kind, cfg, ms_per_launch, traffic):
    alg = algorithmic(cfg)[kind]
    t = ms_per_launch * 1e-3
    if kind == "linear" and cfg.dtype == "bf16":
        ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        if alg["flops"] / alg["bytes"] > ridge:
            achieved = alg["flops"] / t / 1e12
            return {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                    "traffic": traffic, "kernel": kind}
    if kind == "attn":
        mfma_flops = 4 * cfg.N * cfg.H * cfg.W * cfg.C * cfg.L
        if cfg.dtype == "bf16":
            ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
            if mfma_flops / alg["bytes"] > ridge:
                achieved = mfma_flops / t / 1e12
                return {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                        "traffic": traffic, "kernel": kind}
    achieved = alg["bytes"] / t / 1e9
    return {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic, "kernel": kind}


def source_digest(names=ATTN_SOURCES) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "vision_transformer_sparse_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(cfg_name: str):
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, or None if it is absent or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", f"attn_{cfg_name}_hbm_counters.txt")
    if not os.path.exists(path):
        return None
    vals = {}
    with open(path) as f:
        for line in f:
            if ":" in line:
                k, v = line.split(":", 1)
                vals[k.strip()] = v.strip()
    if vals.get("attention_source_sha256_16") != source_digest():
        return None
    try:
        return float(vals["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(inp, cfg, budget_s: float, op: str = "forward"):
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info, threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    ncores = len(os.sched_getaffinity(0))
    ncores = min(ncores, 16)
    ctx = threadpool_limits(limits=ncores) if threadpool_limits else None
    passes, t0 = 0, time.perf_counter()
    try:
        while True:
            if op == "block":
                oracle.bra_block_forward(inp["x"], inp["wqkv"], inp["bqkv"], inp["lce_w"],
                                         inp["lce_b"], inp["wo"], inp["bo"], cfg.heads, cfg.S,
                                         cfg.topk)
            else:
                oracle.bra_forward(inp["q"], inp["k"], inp["v"], inp["lce_w"], inp["lce_b"],
                                   cfg.heads, cfg.S, cfg.topk)
            passes += 1
            if time.perf_counter() - t0 >= budget_s:
                break
    finally:
        if ctx is not None:
            ctx.__exit__(None, None, None)
    dt = time.perf_counter() - t0
    return {"value": passes * cfg.queries / dt, "unit": "queries/s", "cores": ncores,
            "kind": "oracle",
            "sample": f"{passes} full {op} pass(es) of the {cfg.name} batch (N={cfg.N}, "
                      f"{cfg.queries} queries each), fp64 numpy, {dt:.1f} s"}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the GPU's clocks settle over tens of milliseconds of load: the defaults
    # warm up for ~50 ms and time ~100 ms
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--config", default="c1")
    ap.add_argument("--op", choices=("forward", "block"), default="forward",
                    help="forward: bra_forward alone; block: qkv projection, bra_forward, wo")
    ap.add_argument("--cpu-budget", type=float, default=10.0,
                    help="seconds of oracle work for the CPU baseline (0 = skip)")
    ap.add_argument("--calib-copy-mb", type=int, default=0,
                    help="after timing, run one copy kernel of this many MiB (counter calibration)")
    a = ap.parse_args(argv)
    if a.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {a.gpus} is not supported "
              "(each image is independent, so batch sharding needs no collective, "
              "but this build runs on one device)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from synth import CONFIGS, draw_block, draw_config
    from vision_transformer_sparse_amd import bra

    cfg = {c.name: c for c in CONFIGS}[a.config]
    bra.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if a.op == "block":
        inp = draw_block(cfg.N, cfg.H, cfg.W, cfg.C, cfg.S, cfg.dtype, 2000 + CONFIGS.index(cfg),
                         cfg.offset_std, cfg.w_std, cfg.b_std)
    else:
        inp = draw_config(cfg)
    tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    t = {k: torch.from_numpy(v.astype(np.float32)).to(dev, tdt) for k, v in inp.items()}
    shape = (cfg.N, cfg.H, cfg.W, cfg.C)
    out = torch.empty(shape, dtype=tdt, device=dev)
    route = torch.empty((cfg.N, cfg.R, cfg.topk), dtype=torch.int32, device=dev)
    if a.op == "block":
        qkv = [torch.empty(shape, dtype=tdt, device=dev) for _ in range(3)]
        y = torch.empty(shape, dtype=tdt, device=dev)

        def step():
            bra.linear(t["x"], t["wqkv"], t["bqkv"], split=cfg.C, outs=qkv)
            bra.forward(*qkv, t["lce_w"], t["lce_b"], cfg.heads, cfg.S, cfg.topk,
                        out=out, route_idx=route)
            bra.linear(out, t["wo"], t["bo"], outs=[y])
    else:
        def step():
            bra.forward(t["q"], t["k"], t["v"], t["lce_w"], t["lce_b"], cfg.heads, cfg.S,
                        cfg.topk, out=out, route_idx=route)

    for _ in range(a.warmup):
        step()
    torch.cuda.synchronize()
    print(f"[bench] {cfg.name} warmup done", file=sys.stderr, flush=True)
    # attention launches are timed with HIP events on one step in
    # PROFILE_EVERY (two event records per timed launch perturb the loop)
    bra.profile_begin(())
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(a.steps):
        if i % PROFILE_EVERY == 0:
            bra.profile_set_mask(["attn"])
            step()
            bra.profile_set_mask(())
        else:
            step()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    prof_timed = bra.profile_read()
    bra.profile_begin(())
    print(f"[bench] {cfg.name} timed {a.steps} steps in {elapsed:.3f} s", file=sys.stderr, flush=True)

    # every kernel kind, in a separate (untimed) pass
    bra.profile_begin(bra.KERNEL_NAMES)
    for _ in range(max(10, a.steps // 4)):
        step()
    prof_all = bra.profile_read()
    bra.profile_begin(())

    if a.calib_copy_mb > 0:
        nbytes = a.calib_copy_mb * 1024 * 1024
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        bra.calib_copy(src, dst)
        torch.cuda.synchronize()
        del src, dst

    ms_step = elapsed * 1e3 / a.steps
    kernels = {}
    for kind, (ms, cnt) in prof_all.items():
        if cnt:
            kernels[kind] = {"us_per_launch": ms * 1e3 / cnt, "launches": cnt}
    attn_ms, attn_cnt = prof_timed["attn"]
    attn_ms_per_launch = attn_ms / attn_cnt
    roof = roofline_for("attn", cfg, attn_ms_per_launch, measured_traffic(cfg.name))
    roof["us_per_launch"] = attn_ms_per_launch * 1e3
    roof["launches"] = attn_cnt
    for kind in kernels:
        r = roofline_for(kind, cfg, kernels[kind]["us_per_launch"] * 1e-3, None)
        kernels[kind].update(bound=r["bound"], achieved=round(r["achieved"], 2), unit=r["unit"],
                             frac=round(r["frac"], 4))

    cpu = cpu_baseline(inp, cfg, a.cpu_budget, a.op) if a.cpu_budget > 0 else None
    value = cfg.queries * a.steps / elapsed
    line = {
        "metric": METRIC,
        "value": value,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": a.steps,
        "warmup": a.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) q/k/v; see synth/)",
        "config": {"workload": f"{cfg.name}: {cfg.what}"
                               + (" -- block: qkv Linear, BRA, wo Linear" if a.op == "block" else ""),
                   "N": cfg.N, "H": cfg.H, "W": cfg.W,
                   "C": cfg.C, "heads": cfg.heads, "S": cfg.S, "topk": cfg.topk,
                   "queries_per_step": cfg.queries, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "attention_source_sha256_16": source_digest(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
