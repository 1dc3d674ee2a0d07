"""Seeded synthetic inputs for the Bi-Level Routing Attention forward pass.

This module draws random tensors and rounds them to the storage dtype. It
holds none of the method's arithmetic: no pooling, routing, attention or
convolution happens here. Both the fp64 oracle and the HIP path receive the
arrays it returns (the oracle as float64, the GPU as the same values stored in
fp32 or bf16), so the two sides see bit-identical inputs.

Shapes follow the stages the pages describe (page bernice.tw/posts/biformer,
sections "Biformer" and "實驗": S = 7 for 224x224 classification, 16 for
detection, 8 for segmentation; topk 1/4/16 per stage; and the tensor trace of
the walk-through at TRANSFORMER.niftyadmin.cn/n/347023.html, section BRA模块:
stage 1 is (1, 56, 56, 64) with 7x7 regions of 8x8 tokens). The value
distributions are the plainest reading of the workload statement: N(mu, var)
notation, so N(0, 1/25) has standard deviation 0.2.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

__all__ = ["Config", "CONFIGS", "STAGE4", "draw", "round_to_bf16", "draw_config", "draw_linear",
           "draw_block"]


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    what: str
    dtype: str          # "f32" or "bf16"
    N: int
    H: int
    W: int
    C: int
    heads: int
    S: int
    topk: int
    offset_std: float   # std of the per-(image, region, channel) offsets, 0 = none
    w_std: float        # std of the 5x5 depthwise LCE weights
    b_std: float        # std of the LCE bias, 0 = zero bias

    @property
    def R(self) -> int:
        return self.S * self.S

    @property
    def T(self) -> int:
        return (self.H // self.S) * (self.W // self.S)

    @property
    def L(self) -> int:
        return self.topk * self.T

    @property
    def head_dim(self) -> int:
        return self.C // self.heads

    @property
    def queries(self) -> int:
        return self.N * self.H * self.W


CONFIGS = [
    Config("c0", "classification stage 1 (224x224 input /4)", "f32",
           1, 56, 56, 64, 2, 7, 1, 0.0, 0.2, 0.0),
    Config("c1", "classification stage 2 (224x224 input /8)", "bf16",
           128, 28, 28, 128, 4, 7, 4, 0.0, 0.2, 0.1),
    Config("c2", "classification stage 3 (224x224 input /16)", "bf16",
           128, 14, 14, 256, 8, 7, 16, 0.0, 0.2, 0.1),
    Config("c3", "detection stage 2 (1024x1024 input /8), S=16", "bf16",
           2, 128, 128, 128, 4, 16, 4, math.sqrt(0.5), 0.2, 0.1),
    Config("c4", "segmentation stage 1 (512x512 input /4), S=8", "bf16",
           8, 128, 128, 64, 2, 8, 4, math.sqrt(0.5), 0.2, 0.1),
]


# The router-free last stage (every region routed, k = S^2 on page
# bernice.tw/posts/biformer, section "Biformer"; AttentionLePE with C = 512 in
# the walk-through's module print, section 网络结构): 7x7 tokens at 224x224
# input /32, 16 heads of 32. S = 1 (the whole map is one region) and topk = 1
# describe the same computation for the routed entry points.
STAGE4 = Config("s4", "classification stage 4 (224x224 input /32), dense", "bf16",
                128, 7, 7, 512, 16, 1, 1, 0.0, 0.2, 0.1)


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to bf16 (via fp32, round-to-nearest-even both times)
    and return them as float64 holding exactly the bf16 values."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    bits = x32.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) >> 16) & 0xFFFF
    out = (rounded.astype(np.uint32) << 16).view(np.float32)
    return out.astype(np.float64)


def _round(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return x.astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_to_bf16(x)
    raise ValueError(f"unknown dtype {dtype!r}")


def draw(N: int, H: int, W: int, C: int, S: int, dtype: str, seed: int,
         offset_std: float = 0.0, w_std: float = 0.2, b_std: float = 0.1):
    """Draw q, k, v (N,H,W,C), lce_w (C,5,5), lce_b (C,) from PCG64(seed).

    Order of draws: q, k, v standard normals; then (if offset_std > 0) one
    offset per (image, region row, region col, channel) for each of q, k, v,
    added to every token of that region; then lce_w; then lce_b (if b_std > 0,
    else zeros). Every array is rounded to `dtype` and returned as float64.
    """
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((N, H, W, C))
    k = rng.standard_normal((N, H, W, C))
    v = rng.standard_normal((N, H, W, C))
    if offset_std > 0.0:
        rh, rw = H // S, W // S
        for x in (q, k, v):
            off = rng.standard_normal((N, S, S, C)) * offset_std
            x += np.repeat(np.repeat(off, rh, axis=1), rw, axis=2)
    w = rng.standard_normal((C, 5, 5)) * w_std
    b = rng.standard_normal((C,)) * b_std if b_std > 0.0 else np.zeros((C,))
    return {"q": _round(q, dtype), "k": _round(k, dtype), "v": _round(v, dtype),
            "lce_w": _round(w, dtype), "lce_b": _round(b, dtype)}


def draw_config(cfg: Config | int, seed: int | None = None, N: int | None = None):
    """Inputs of one named workload. The seed defaults to 1000 + its index.
    `N` optionally truncates the batch (the first N images of the same draw
    are NOT preserved; a smaller batch is a different draw)."""
    if isinstance(cfg, int):
        idx, cfg = cfg, CONFIGS[cfg]
    else:
        idx = len(CONFIGS) if cfg == STAGE4 else CONFIGS.index(cfg)
    if seed is None:
        seed = 1000 + idx
    return draw(N if N is not None else cfg.N, cfg.H, cfg.W, cfg.C, cfg.S,
                cfg.dtype, seed, cfg.offset_std, cfg.w_std, cfg.b_std)


def _linear_init(rng, nout: int, nin: int):
    """A Linear layer's weight (nout, nin) and bias (nout,), each uniform on
    [-1/sqrt(nin), 1/sqrt(nin)] (the usual default initialisation of such a
    layer; the pages train their weights, which no synthetic run has)."""
    bound = 1.0 / math.sqrt(nin)
    w = rng.uniform(-bound, bound, (nout, nin))
    b = rng.uniform(-bound, bound, (nout,))
    return w, b


def draw_linear(M: int, K: int, Nout: int, dtype: str, seed: int):
    """x (M, K) standard normal, then w (Nout, K) and b (Nout,) as a Linear
    layer's initialisation, from PCG64(seed), rounded to `dtype`."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K))
    w, b = _linear_init(rng, Nout, K)
    return {"x": _round(x, dtype), "w": _round(w, dtype), "b": _round(b, dtype)}


def draw_block(N: int, H: int, W: int, C: int, S: int, dtype: str, seed: int,
               offset_std: float = 0.0, w_std: float = 0.2, b_std: float = 0.1):
    """Inputs of the block around the operator, from PCG64(seed): x
    (N, H, W, C) standard normal (plus, if offset_std > 0, one offset per
    image, region and channel added to the region's tokens), then the qkv
    Linear(C, 3C), then the output Linear(C, C), then lce_w (C,5,5) ~
    N(0, w_std^2) and lce_b (C,) ~ N(0, b_std^2) (zeros if b_std is 0). Every
    array is rounded to `dtype`."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((N, H, W, C))
    if offset_std > 0.0:
        off = rng.standard_normal((N, S, S, C)) * offset_std
        x += np.repeat(np.repeat(off, H // S, axis=1), W // S, axis=2)
    wqkv, bqkv = _linear_init(rng, 3 * C, C)
    wo, bo = _linear_init(rng, C, C)
    w = rng.standard_normal((C, 5, 5)) * w_std
    b = rng.standard_normal((C,)) * b_std if b_std > 0.0 else np.zeros((C,))
    out = {"x": x, "wqkv": wqkv, "bqkv": bqkv, "wo": wo, "bo": bo, "lce_w": w, "lce_b": b}
    return {name: _round(a, dtype) for name, a in out.items()}
