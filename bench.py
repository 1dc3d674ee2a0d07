"""Throughput of the BRA forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config c4]

A step is one bra_forward call -- region pooling, routing, gathered attention
and LCE -- over one batch of seeded synthetic input already resident in HBM.
The headline workload is c4 (segmentation stage 1: 8 images of 128x128, 64
channels, 2 heads, 8x8 regions of 256 tokens, topk 4): the largest single-GPU
workload, and the one whose attention is bound by the matrix cores.

Order of the run:
  1. per_config: every workload c0..c4 is measured in turn -- warm steps
     timed back to back, every kernel kind timed with HIP events, and cold
     steps (each after a 1 GiB write that flushes L2 and the memory-side
     cache) timed with events around the whole step and around the
     attention kernel. This also brings the GPU's clocks to steady state.
  2. headline: W untimed warm-up steps of the headline workload, then K
     steps timed between two device synchronisations.
One JSON line is printed. It carries:
  value      whole-job queries/s of the K timed steps (a query is one token
             position, N*H*W per step)
  roofline   the attention kernel's (the dominant kernel's) algorithmic flops
             (c4; bytes for the HBM-bound workloads) per launch over its mean
             launch time, measured with HIP events on the launch stream on
             every PROFILE_EVERY-th step of the timed region (the library
             launches a timed kernel with hipExtLaunchKernelGGL, which ties
             the event pair to that dispatch)
  per_config per workload: warm ms/step and queries/s, cold step and
             attention medians (p10, p90), and each kernel kind's us per
             launch and fraction of the roofline that bounds it
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the headline
             workload (about 10 s of CPU work), threads and CPU model stated
--op block times the block around the operator instead, one
bra_block_forward call a step: the qkv projection (Linear C -> 3C), the
operator and the output projection (Linear C -> C), fused on the shapes
bra_block_fused reports (there "linear" is the qkv projection with the
region pooling and "attn" the attention with the output projection);
"kernels" then also holds the projection kernel's roofline. The router-free last stage (s4: 128 images of 7x7 tokens, C = 512,
16 heads) is measured in per_config as its own workload: a step is one
bra_attention_dense call. `--config s4` makes it the headline. The per-head
routing variant on the c4 shape (c4h: one bra_forward_head_routed call a
step), the backward for given routes on the c4 and c1 shapes (c4b, c1b: one
bra_backward call a step) and the block on the c4 and c1 shapes (c4blk,
c1blk) are measured there too.
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
FLUSH_BYTES = 1 << 30
ATTN_SOURCES = ("attn_image.hip", "attn_region.hip", "attn_tile.hip", "attn_mfma.hip", "attn_valu.hip",
                "attn_f32.hip", "attn_dense.hip", "bra_internal.h", "route_common.h")


def dense(cfg) -> bool:
    """The router-free workload: its step is bra_attention_dense."""
    return cfg.name == "s4"


def algorithmic(cfg):
    """Per-launch algorithmic traffic / work of each kernel (what the method
    must move or compute, not what a dense method would)."""
    b = 2 if cfg.dtype == "bf16" else 4
    E = cfg.N * cfg.H * cfg.W * cfg.C
    means = 2 * cfg.N * cfg.R * cfg.C * 4
    routes = 0 if dense(cfg) else cfg.N * cfg.R * cfg.topk * 4
    lce_params = cfg.C * 26 * b
    return {
        "pool": {"bytes": 2 * E * b + means},
        "route": {"bytes": means + routes, "flops": 2 * cfg.N * cfg.R * cfg.R * cfg.C},
        "attn": {"bytes": 4 * E * b + routes + lce_params, "flops": 4 * E * cfg.L + 50 * E},
        # backward for given routes: reads q, k, v, dout, writes dq, dk, dv; the
        # five products S (recomputed), dP, dV, dQ, dK, and the LCE's two
        "attn_bwd": {"bytes": 7 * E * b + routes + lce_params + cfg.C * 26 * 4,
                     "flops": 10 * E * cfg.L + 100 * E},
        # the block's two projections, averaged per launch: qkv reads x and
        # writes q, k, v; wo reads o and writes y (weights and biases once)
        "linear": {"bytes": (4 * E + 4 * cfg.C * (cfg.C + 1) + 2 * E) * b / 2,
                   "flops": 2 * E * 4 * cfg.C / 2},
        # the fused block: the qkv projection that also writes the region
        # means and key norms; the attention that applies wo before it stores
        # (reads q, k, v, writes y)
        "linear_qkv": {"bytes": 4 * E * b + 3 * cfg.C * (cfg.C + 1) * b + means
                       + cfg.N * cfg.R * (cfg.C // 32) * 4,
                       "flops": 2 * E * 3 * cfg.C},
        "attn_block": {"bytes": 4 * E * b + routes + lce_params + cfg.C * (cfg.C + 1) * b,
                       "flops": 4 * E * cfg.L + 50 * E + 2 * E * cfg.C},
    }


def roofline_for(kind, cfg, ms_per_launch, traffic, share=1.0, backward=False, fused_block=False):
    """share: the fraction of the workload one launch processes (1/heads
    for the per-head routing variant, which launches each kernel per head).
    backward: the attention kind is the backward's kernels (one bra_backward
    call, priced by its own algorithmic work). fused_block: the kinds are
    the fused block's kernels (qkv + pooling, routing, attention + wo)."""
    akind = kind
    if backward and kind == "attn":
        akind = "attn_bwd"
    elif fused_block:
        akind = {"attn": "attn_block", "linear": "linear_qkv"}.get(kind, kind)
    alg = {k: v * share for k, v in algorithmic(cfg)[akind].items()}
    t = ms_per_launch * 1e-3
    if kind == "linear" and cfg.dtype == "bf16":
        ridge = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)
        if alg["flops"] / alg["bytes"] > ridge:
            achieved = alg["flops"] / t / 1e12
            return {"bound": "mfma", "achieved": achieved, "peak": MFMA_BF16_PEAK_TFLOPS,
                    "unit": "TFLOP/s", "frac": achieved / MFMA_BF16_PEAK_TFLOPS,
                    "traffic": traffic, "kernel": kind}
    if kind == "attn":
        E = cfg.N * cfg.H * cfg.W * cfg.C
        mfma_flops = (10 if backward else 4) * E * cfg.L * share + (2 * E * cfg.C if fused_block else 0)
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


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_threads() -> int:
    """Threads for the oracle's BLAS pool: every core of the process's
    affinity set, capped by OMP_NUM_THREADS where the host sets it (a shared
    host states the share of its cores a job may use that way)."""
    n = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.isdigit() and int(env) > 0:
        n = min(n, int(env))
    return n


def cpu_baseline(inp, cfg, budget_s: float, op: str = "forward"):
    import oracle
    try:
        from threadpoolctl import threadpool_limits
    except ImportError:  # pragma: no cover
        threadpool_limits = None
    ncores = cpu_threads()
    ctx = threadpool_limits(limits=ncores) if threadpool_limits else None
    passes, t0 = 0, time.perf_counter()
    try:
        while True:
            if op == "block":
                oracle.bra_block_forward(inp["x"], inp["wqkv"], inp["bqkv"], inp["lce_w"],
                                         inp["lce_b"], inp["wo"], inp["bo"], cfg.heads, cfg.S,
                                         cfg.topk)
            elif op == "backward":
                oracle.bra_backward(inp["q"], inp["k"], inp["v"], inp["lce_w"], inp["route"],
                                    inp["g"], cfg.heads, cfg.S)
            elif op == "head_routed":
                oracle.bra_forward_head_routed(inp["q"], inp["k"], inp["v"], inp["lce_w"], inp["lce_b"],
                                               cfg.heads, cfg.S, cfg.topk)
            elif op == "dense":
                oracle.dense_attention(inp["q"], inp["k"], inp["v"], inp["lce_w"], inp["lce_b"],
                                       cfg.heads)
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
            "kind": "oracle", "cpu_model": cpu_model(),
            "affinity_cores": len(os.sched_getaffinity(0)),
            "sample": f"{passes} full {op} pass(es) of the {cfg.name} batch (N={cfg.N}, "
                      f"{cfg.queries} queries each), fp64 numpy, {dt:.1f} s"}


def pctl(xs, p):
    xs = sorted(xs)
    if not xs:
        return None
    i = min(len(xs) - 1, max(0, int(round(p / 100.0 * (len(xs) - 1)))))
    return xs[i]


class Workload:
    """Device tensors and the step function of one workload."""

    def __init__(self, cfg, op, dev, inputs=None):
        import numpy as np
        import torch

        from synth import CONFIGS, draw, draw_block, draw_config
        from vision_transformer_sparse_amd import bra

        self.cfg = cfg
        if dense(cfg) and op == "forward":
            op = "dense"
        self.op = op
        if inputs is None:
            if op == "block":
                inputs = draw_block(cfg.N, cfg.H, cfg.W, cfg.C, cfg.S, cfg.dtype,
                                    2000 + CONFIGS.index(cfg), cfg.offset_std, cfg.w_std, cfg.b_std)
            else:
                inputs = draw_config(cfg)
        self.inputs = inputs
        tdt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
        t = {k: torch.from_numpy(v.astype(np.float32)).to(dev, tdt) for k, v in inputs.items()}
        shape = (cfg.N, cfg.H, cfg.W, cfg.C)
        out = torch.empty(shape, dtype=tdt, device=dev)
        route = torch.empty((cfg.N, cfg.heads, cfg.R, cfg.topk) if op == "head_routed" else (cfg.N, cfg.R, cfg.topk),
                            dtype=torch.int32, device=dev)
        self.fused = op == "block" and bra.block_fused(cfg.N, cfg.H, cfg.W, cfg.C, cfg.heads, cfg.S,
                                                       cfg.topk, tdt)
        if op == "block":
            def step():
                bra.block_forward(t["x"], t["wqkv"], t["bqkv"], t["lce_w"], t["lce_b"], t["wo"], t["bo"],
                                  cfg.heads, cfg.S, cfg.topk, out=out, route_idx=route)
        elif op == "dense":
            def step():
                bra.attention_dense(t["q"], t["k"], t["v"], t["lce_w"], t["lce_b"], cfg.heads, out=out)
        elif op == "backward":
            g_np = draw(cfg.N, cfg.H, cfg.W, cfg.C, cfg.S, cfg.dtype, 3000 + CONFIGS.index(cfg))["q"]
            g = torch.from_numpy(g_np.astype(np.float32)).to(dev, tdt)
            bra.forward(t["q"], t["k"], t["v"], t["lce_w"], t["lce_b"], cfg.heads, cfg.S, cfg.topk,
                        out=out, route_idx=route)
            # the CPU baseline differentiates for the same routes and dout
            self.inputs = dict(inputs, route=route.cpu().numpy(), g=g_np)

            def step():
                bra.backward(t["q"], t["k"], t["v"], t["lce_w"], route, g, cfg.heads, cfg.S)
        elif op == "head_routed":
            def step():
                bra.forward_head_routed(t["q"], t["k"], t["v"], t["lce_w"], t["lce_b"], cfg.heads, cfg.S,
                                        cfg.topk, out=out, route_idx=route)
        else:
            def step():
                bra.forward(t["q"], t["k"], t["v"], t["lce_w"], t["lce_b"], cfg.heads, cfg.S,
                            cfg.topk, out=out, route_idx=route)
        self.step = step


def attn_share(prof, steps: int) -> float:
    """The fraction of a step's work one attention launch does: a step of
    the per-head routing variant launches the attention kernel once per head
    where it runs the operator per head, once where one kernel routes every
    head."""
    cnt = prof.get("attn", (0.0, 0))[1]
    return steps / cnt if cnt else 1.0


def kernel_rooflines(prof, cfg, share=1.0, backward=False, fused_block=False):
    kernels = {}
    for kind, (ms, cnt) in prof.items():
        if cnt:
            us = ms * 1e3 / cnt
            r = roofline_for(kind, cfg, us * 1e-3, None, share, backward, fused_block)
            kernels[kind] = {"us_per_launch": round(us, 3), "launches": cnt, "bound": r["bound"],
                             "achieved": round(r["achieved"], 2), "unit": r["unit"],
                             "frac": round(r["frac"], 4)}
    return kernels


def measure_config(w, flush, n_warm, n_cold):
    """Warm and cold timings of one workload (see the module docstring)."""
    import torch

    from vision_transformer_sparse_amd import bra

    cfg = w.cfg
    bwd = w.op == "backward"
    fb = w.fused
    for _ in range(n_warm // 2):
        w.step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(n_warm):
        w.step()
    torch.cuda.synchronize()
    warm_ms = (time.perf_counter() - t0) * 1e3 / n_warm
    bra.profile_begin(bra.KERNEL_NAMES)
    nprof = max(20, n_warm // 4)
    for _ in range(nprof):
        w.step()
    prof = bra.profile_read()
    share = attn_share(prof, nprof)
    kernels = kernel_rooflines(prof, cfg, share, bwd, fb)
    bra.profile_begin(())
    # cold: a 1 GiB write before each step; events around the step (torch's
    # current stream, which the binding hands to the library) and around the
    # attention kernel (the library's event pair on its dispatch)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(n_cold)]
    attn_us = []
    for a, b in ev:
        flush.zero_()
        bra.profile_begin(["attn"])
        a.record()
        w.step()
        b.record()
        ms, cnt = bra.profile_read()["attn"]
        if cnt:
            attn_us.append(ms * 1e3 / cnt)
    bra.profile_begin(())
    torch.cuda.synchronize()
    cold_us = [a.elapsed_time(b) * 1e3 for a, b in ev]
    cold = {"step_us_median": round(pctl(cold_us, 50), 3), "step_us_p10": round(pctl(cold_us, 10), 3),
            "step_us_p90": round(pctl(cold_us, 90), 3), "calls": n_cold,
            "queries_per_s": cfg.queries / (pctl(cold_us, 50) * 1e-6)}
    if attn_us:
        med = pctl(attn_us, 50)
        r = roofline_for("attn", cfg, med * 1e-3, None, share, bwd, fb)
        cold.update(attn_us_median=round(med, 3), attn_us_p10=round(pctl(attn_us, 10), 3),
                    attn_us_p90=round(pctl(attn_us, 90), 3), attn_frac=round(r["frac"], 4))
    return {"ms_per_step": round(warm_ms, 5), "queries_per_s": cfg.queries / (warm_ms * 1e-3),
            "queries_per_step": cfg.queries, "kernels": kernels, "cold": cold}


def main(argv=None) -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=500)
    ap.add_argument("--config", default="c4", help="headline workload (c0..c4, or s4)")
    ap.add_argument("--op", choices=("forward", "block", "backward", "head_routed"), default="forward",
                    help="forward: bra_forward alone; block: qkv projection, bra_forward, wo; "
                         "backward: bra_backward for the forward's routes; head_routed: "
                         "bra_forward_head_routed")
    ap.add_argument("--per-config", choices=("all", "none"), default="all",
                    help="all: measure every workload first (per_config); none: the headline only")
    ap.add_argument("--cold", type=int, default=100, help="cold calls per workload in per_config")
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

    import torch

    from synth import CONFIGS, STAGE4
    from vision_transformer_sparse_amd import bra

    workloads = CONFIGS + [STAGE4] if a.op == "forward" else CONFIGS
    if a.op in ("backward", "head_routed") and a.per_config == "all":
        print(f"--op {a.op} is measured with --per-config none (per_config already holds it)",
              file=sys.stderr)
        return 2
    by_name = {c.name: c for c in workloads}
    cfg = by_name[a.config]
    bra.load()
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    per_config = {}
    head = None
    if a.per_config == "all":
        flush = torch.empty(FLUSH_BYTES // 4, dtype=torch.float32, device=dev)
        runs = [(c.name, c, a.op) for c in workloads]
        if a.op == "forward":
            runs.append(("c4h", by_name["c4"], "head_routed"))
            runs.append(("c4b", by_name["c4"], "backward"))
            runs.append(("c1b", by_name["c1"], "backward"))
            runs.append(("c4blk", by_name["c4"], "block"))
            runs.append(("c1blk", by_name["c1"], "block"))
        for name, c, op in runs:
            w = Workload(c, op, dev)
            per_config[name] = measure_config(w, flush, n_warm=1000, n_cold=a.cold)
            if op == "head_routed":
                per_config[name]["op"] = "bra_forward_head_routed (every head routed on its own channels)"
            if op == "backward":
                per_config[name]["op"] = "bra_backward (gradients for the forward's routes)"
            if op == "block":
                per_config[name]["op"] = ("bra_block_forward (qkv Linear, BRA, wo Linear; "
                                          + ("fused)" if w.fused else "three steps)"))
            print(f"[bench] per_config {name}: {per_config[name]['ms_per_step'] * 1e3:.2f} us/step warm, "
                  f"{per_config[name]['cold']['step_us_median']:.2f} us cold", file=sys.stderr, flush=True)
            if c is cfg and op == a.op:
                head = w
            else:
                del w
        del flush
        torch.cuda.synchronize()
    if head is None:
        head = Workload(cfg, a.op, dev)

    step = head.step
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
    print(f"[bench] {cfg.name} timed {a.steps} steps in {elapsed:.4f} s", file=sys.stderr, flush=True)

    # every kernel kind, in a separate (untimed) pass
    bra.profile_begin(bra.KERNEL_NAMES)
    nprof = max(10, a.steps // 4)
    for _ in range(nprof):
        step()
    prof = bra.profile_read()
    share = attn_share(prof, nprof)
    bwd = head.op == "backward"
    kernels = kernel_rooflines(prof, cfg, share, bwd, head.fused)
    bra.profile_begin(())

    if a.calib_copy_mb > 0:
        nbytes = a.calib_copy_mb * 1024 * 1024
        src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        bra.calib_copy(src, dst)
        torch.cuda.synchronize()
        del src, dst

    ms_step = elapsed * 1e3 / a.steps
    attn_ms, attn_cnt = prof_timed["attn"]
    attn_ms_per_launch = attn_ms / attn_cnt
    traffic = measured_traffic(cfg.name) if head.op in ("forward", "dense") else None
    roof = roofline_for("attn", cfg, attn_ms_per_launch, traffic, share, bwd, head.fused)
    roof["us_per_launch"] = attn_ms_per_launch * 1e3
    roof["launches"] = attn_cnt

    cpu = cpu_baseline(head.inputs, cfg, a.cpu_budget, head.op) if a.cpu_budget > 0 else None
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
                               + ((" -- block: qkv Linear, BRA, wo Linear"
                                   + (" (fused)" if head.fused else "")) if a.op == "block" else "")
                               + (" -- bra_attention_dense" if head.op == "dense" else "")
                               + (" -- bra_backward for given routes" if bwd else "")
                               + (" -- bra_forward_head_routed" if head.op == "head_routed" else ""),
                   "N": cfg.N, "H": cfg.H, "W": cfg.W,
                   "C": cfg.C, "heads": cfg.heads, "S": cfg.S, "topk": cfg.topk,
                   "queries_per_step": cfg.queries, "parallelism": "single GPU"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "per_config": per_config,
        "attention_source_sha256_16": source_digest(),
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
