"""Python binding of libbra.so (include/bra.h): argument marshalling only.

Every function takes torch tensors that live on a ROCm device, passes their
device pointers and sizes to the C ABI, and enqueues the work on torch's
current stream of that device. All computation happens in the HIP kernels of
the library; there is no fallback: if the library is missing, `load()`
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbra.so")

F32, BF16 = 0, 1
K_POOL, K_ROUTE, K_ATTN, K_LCE = 0, 1, 2, 3
KERNEL_NAMES = ("pool", "route", "attn", "lce", "linear")

_lib = None

_vp, _i, _sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_SIGS = {
    "bra_forward": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _vp]),
    "bra_forward_noalloc": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _vp]),
    "bra_attention_dense": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _vp]),
    "bra_forward_head_routed": (_i, [_vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp, _vp]),
    "bra_backward": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                          _vp, _vp, _vp, _vp, _vp]),
    "bra_region_means": (_i, [_vp, _vp, _i, _i, _i, _i, _i, _i, _vp, _vp]),
    "bra_route": (_i, [_vp, _vp, _i, _i, _i, _i, _vp]),
    "bra_attend": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i, _vp]),
    "bra_lce": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp]),
    "bra_linear": (_i, [_vp, _vp, _vp, _i, _i, _i, _i, _i, _vp, _vp, _vp]),
    "bra_block_forward": (_i, [_vp, _vp, _vp, _vp, _vp, _vp, _vp, _i, _i, _i, _i, _i, _i, _i, _i,
                               _vp, _vp]),
    "bra_block_fused": (_i, [_i, _i, _i, _i, _i, _i, _i, _i]),
    "bra_set_stream": (_i, [_vp]),
    "bra_get_stream": (_vp, []),
    "bra_workspace_bytes": (_sz, [_i, _i, _i]),
    "bra_release": (None, []),
    "bra_error_string": (ctypes.c_char_p, [_i]),
    "bra_version": (_i, []),
    "bra_profile_begin": (_i, [_i]),
    "bra_profile_set_mask": (_i, [_i]),
    "bra_profile_read": (_i, [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int), _i]),
    "bra_calib_copy": (_i, [_vp, _vp, _sz]),
}
EXPORTED = tuple(_SIGS)


class BraError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: status {code}: {error_string(code)}")


def load() -> ctypes.CDLL:
    """Loads the in-tree libbra.so (built by vision_transformer_sparse_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m vision_transformer_sparse_amd.build`")
        lib = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            fn = getattr(lib, name)
            fn.restype = res
            fn.argtypes = args
        _lib = lib
    return _lib


def error_string(code: int) -> str:
    return load().bra_error_string(code).decode()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return F32
    if t.dtype == torch.bfloat16:
        return BF16
    raise TypeError(f"unsupported dtype {t.dtype} (float32 or bfloat16)")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _check(t: torch.Tensor, name: str, dtype=None, device=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


def _stream(device) -> None:
    load().bra_set_stream(ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream))


def _call(name, *args):
    rc = getattr(load(), name)(*args)
    if rc != 0:
        raise BraError(rc, name)


def forward(q, k, v, lce_w, lce_b, heads: int, S: int, topk: int, out=None, route_idx=None):
    """bra_forward: returns (out, route_idx). q, k, v: (N, H, W, C) float32 or
    bfloat16; lce_w: (C, 5, 5) or (C, 1, 5, 5) of the same dtype; lce_b: (C,)
    or None."""
    _check(q, "q")
    dev, dt = q.device, q.dtype
    for name, t in (("k", k), ("v", v), ("lce_w", lce_w)):
        _check(t, name, dt, dev)
    if lce_b is not None:
        _check(lce_b, "lce_b", dt, dev)
    N, H, W, C = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v shapes differ")
    if lce_w.numel() != C * 25 or (lce_b is not None and lce_b.numel() != C):
        raise ValueError("lce_w must hold C*25 and lce_b C elements")
    if out is None:
        out = torch.empty_like(q)
    if route_idx is None:
        route_idx = torch.empty((N, S * S, topk) if S > 0 and topk > 0 else (0,),
                                dtype=torch.int32, device=dev)
    _check(out, "out", dt, dev)
    _check(route_idx, "route_idx", torch.int32, dev)
    if out.shape != q.shape or route_idx.numel() != N * S * S * topk:
        raise ValueError("out / route_idx have the wrong size")
    with torch.cuda.device(dev):
        _stream(dev)
        _call("bra_forward", _ptr(q), _ptr(k), _ptr(v), _ptr(lce_w), _ptr(lce_b),
              N, H, W, C, heads, S, topk, _dtype_code(q), _ptr(out), _ptr(route_idx))
    return out, route_idx


def backward(q, k, v, lce_w, route_idx, dout, heads: int, S: int, lce_b_grad: bool = True):
    """bra_backward: returns (dq, dk, dv, dlce_w, dlce_b) for the given routes
    (dlce_w fp32 (C, 25), dlce_b fp32 (C,) or None)."""
    _check(q, "q")
    dev, dt = q.device, q.dtype
    for name, t in (("k", k), ("v", v), ("lce_w", lce_w), ("dout", dout)):
        _check(t, name, dt, dev)
    _check(route_idx, "route_idx", torch.int32, dev)
    N, H, W, C = q.shape
    if k.shape != q.shape or v.shape != q.shape or dout.shape != q.shape:
        raise ValueError("q, k, v, dout shapes differ")
    if lce_w.numel() != C * 25:
        raise ValueError("lce_w must hold C*25 elements")
    topk = route_idx.shape[-1]
    if route_idx.numel() != N * S * S * topk:
        raise ValueError("route_idx must be (N, S*S, topk)")
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dw = torch.empty((C, 25), dtype=torch.float32, device=dev)
    db = torch.empty((C,), dtype=torch.float32, device=dev) if lce_b_grad else None
    with torch.cuda.device(dev):
        _stream(dev)
        _call("bra_backward", _ptr(q), _ptr(k), _ptr(v), _ptr(lce_w), _ptr(route_idx), _ptr(dout),
              N, H, W, C, heads, S, topk, _dtype_code(q), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dw), _ptr(db))
    return dq, dk, dv, dw, db


def forward_head_routed(q, k, v, lce_w, lce_b, heads: int, S: int, topk: int, out=None,
                        route_idx=None):
    """bra_forward_head_routed: returns (out, route_idx) with route_idx int32
    (N, heads, S*S, topk) -- every head routed on its own channels."""
    _check(q, "q")
    dev, dt = q.device, q.dtype
    for name, t in (("k", k), ("v", v), ("lce_w", lce_w)):
        _check(t, name, dt, dev)
    if lce_b is not None:
        _check(lce_b, "lce_b", dt, dev)
    N, H, W, C = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v shapes differ")
    if lce_w.numel() != C * 25 or (lce_b is not None and lce_b.numel() != C):
        raise ValueError("lce_w must hold C*25 and lce_b C elements")
    if out is None:
        out = torch.empty_like(q)
    if route_idx is None:
        route_idx = torch.empty((N, max(heads, 0), S * S, topk) if S > 0 and topk > 0 else (0,),
                                dtype=torch.int32, device=dev)
    _check(out, "out", dt, dev)
    _check(route_idx, "route_idx", torch.int32, dev)
    if out.shape != q.shape or route_idx.numel() != N * heads * S * S * topk:
        raise ValueError("out / route_idx have the wrong size")
    with torch.cuda.device(dev):
        _stream(dev)
        _call("bra_forward_head_routed", _ptr(q), _ptr(k), _ptr(v), _ptr(lce_w), _ptr(lce_b),
              N, H, W, C, heads, S, topk, _dtype_code(q), _ptr(out), _ptr(route_idx))
    return out, route_idx


def attention_dense(q, k, v, lce_w, lce_b, heads: int, out=None):
    """bra_attention_dense: the router-free attention of the last stage (every
    query over all H*W tokens of its image) plus LCE; returns out."""
    _check(q, "q")
    dev, dt = q.device, q.dtype
    for name, t in (("k", k), ("v", v), ("lce_w", lce_w)):
        _check(t, name, dt, dev)
    if lce_b is not None:
        _check(lce_b, "lce_b", dt, dev)
    N, H, W, C = q.shape
    if k.shape != q.shape or v.shape != q.shape:
        raise ValueError("q, k, v shapes differ")
    if lce_w.numel() != C * 25 or (lce_b is not None and lce_b.numel() != C):
        raise ValueError("lce_w must hold C*25 and lce_b C elements")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", dt, dev)
    if out.shape != q.shape:
        raise ValueError("out has the wrong size")
    with torch.cuda.device(dev):
        _stream(dev)
        _call("bra_attention_dense", _ptr(q), _ptr(k), _ptr(v), _ptr(lce_w), _ptr(lce_b),
              N, H, W, C, heads, _dtype_code(q), _ptr(out))
    return out


def region_means(q, k, S: int):
    """bra_region_means: returns fp32 (N, S*S, C) region means of q and k."""
    _check(q, "q")
    _check(k, "k", q.dtype, q.device)
    N, H, W, C = q.shape
    qr = torch.empty((N, S * S, C), dtype=torch.float32, device=q.device)
    kr = torch.empty_like(qr)
    with torch.cuda.device(q.device):
        _stream(q.device)
        _call("bra_region_means", _ptr(q), _ptr(k), N, H, W, C, S, _dtype_code(q), _ptr(qr), _ptr(kr))
    return qr, kr


def route(qr, kr, topk: int):
    """bra_route: int32 (N, R, topk) routes from fp32 (N, R, C) region means."""
    _check(qr, "qr", torch.float32)
    _check(kr, "kr", torch.float32, qr.device)
    N, R, C = qr.shape
    if kr.shape != qr.shape:
        raise ValueError("qr and kr shapes differ")
    ri = torch.empty((N, R, max(topk, 0)), dtype=torch.int32, device=qr.device)
    with torch.cuda.device(qr.device):
        _stream(qr.device)
        _call("bra_route", _ptr(qr), _ptr(kr), N, R, C, topk, _ptr(ri))
    return ri


def attend(q, k, v, lce_w, lce_b, route_idx, heads: int, S: int, out=None):
    """bra_attend: attention over the given routes plus LCE."""
    _check(q, "q")
    dev, dt = q.device, q.dtype
    for name, t in (("k", k), ("v", v), ("lce_w", lce_w)):
        _check(t, name, dt, dev)
    if lce_b is not None:
        _check(lce_b, "lce_b", dt, dev)
    _check(route_idx, "route_idx", torch.int32, dev)
    N, H, W, C = q.shape
    topk = route_idx.shape[-1]
    if route_idx.numel() != N * S * S * topk:
        raise ValueError("route_idx must be (N, S*S, topk)")
    if out is None:
        out = torch.empty_like(q)
    _check(out, "out", dt, dev)
    with torch.cuda.device(dev):
        _stream(dev)
        _call("bra_attend", _ptr(q), _ptr(k), _ptr(v), _ptr(lce_w), _ptr(lce_b), _ptr(route_idx),
              N, H, W, C, heads, S, topk, _dtype_code(q), _ptr(out))
    return out


def lce(v, lce_w, lce_b):
    """bra_lce: fp32 LCE(v)."""
    _check(v, "v")
    _check(lce_w, "lce_w", v.dtype, v.device)
    if lce_b is not None:
        _check(lce_b, "lce_b", v.dtype, v.device)
    N, H, W, C = v.shape
    out = torch.empty((N, H, W, C), dtype=torch.float32, device=v.device)
    with torch.cuda.device(v.device):
        _stream(v.device)
        _call("bra_lce", _ptr(v), _ptr(lce_w), _ptr(lce_b), N, H, W, C, _dtype_code(v), _ptr(out))
    return out


def linear(x, w, b, split=None, outs=None):
    """bra_linear: y = x w^T + b over the last axis of x (float32 or
    bfloat16). w: (Nout, K); b: (Nout,) or None. The Nout features are
    returned as Nout // split tensors of shape x.shape[:-1] + (split,)
    (split defaults to Nout: one tensor)."""
    _check(x, "x")
    _check(w, "w", x.dtype, x.device)
    if b is not None:
        _check(b, "b", x.dtype, x.device)
    K = x.shape[-1]
    M = x.numel() // K if K else 0
    Nout = w.shape[0]
    if w.dim() != 2 or w.shape[1] != K or (b is not None and b.numel() != Nout):
        raise ValueError("w must be (Nout, K) and b (Nout,)")
    split = Nout if split is None else split
    if split <= 0 or Nout % split or not 1 <= Nout // split <= 3:
        raise ValueError("Nout must be 1, 2 or 3 times split")
    shape = tuple(x.shape[:-1]) + (split,)
    if outs is None:
        outs = [torch.empty(shape, dtype=x.dtype, device=x.device) for _ in range(Nout // split)]
    for i, o in enumerate(outs):
        _check(o, f"outs[{i}]", x.dtype, x.device)
        if tuple(o.shape) != shape:
            raise ValueError("an output has the wrong shape")
    ys = list(outs) + [None] * (3 - len(outs))
    with torch.cuda.device(x.device):
        _stream(x.device)
        _call("bra_linear", _ptr(x), _ptr(w), _ptr(b), M, K, Nout, split, _dtype_code(x),
              _ptr(ys[0]), _ptr(ys[1]), _ptr(ys[2]))
    return tuple(outs)


def block_forward(x, wqkv, bqkv, lce_w, lce_b, wo, bo, heads: int, S: int, topk: int,
                  out=None, route_idx=None):
    """bra_block_forward, the walk-through's BRA block: q, k, v =
    split(x wqkv^T + bqkv), o = the operator, y = o wo^T + bo (one library
    call; fused on the shapes bra_block_fused reports). x: (N, H, W, C);
    wqkv: (3C, C); bqkv: (3C,) or None; wo: (C, C); bo: (C,) or None.
    Returns (y, route_idx)."""
    _check(x, "x")
    dev, dt = x.device, x.dtype
    for name, t in (("wqkv", wqkv), ("lce_w", lce_w), ("wo", wo)):
        _check(t, name, dt, dev)
    for name, t in (("bqkv", bqkv), ("lce_b", lce_b), ("bo", bo)):
        if t is not None:
            _check(t, name, dt, dev)
    N, H, W, C = x.shape
    if tuple(wqkv.shape) != (3 * C, C) or tuple(wo.shape) != (C, C):
        raise ValueError("wqkv must be (3C, C) and wo (C, C)")
    if (bqkv is not None and bqkv.numel() != 3 * C) or (bo is not None and bo.numel() != C):
        raise ValueError("bqkv must hold 3C and bo C elements")
    if lce_w.numel() != C * 25 or (lce_b is not None and lce_b.numel() != C):
        raise ValueError("lce_w must hold C*25 and lce_b C elements")
    if out is None:
        out = torch.empty_like(x)
    if route_idx is None:
        route_idx = torch.empty((N, S * S, topk) if S > 0 and topk > 0 else (0,),
                                dtype=torch.int32, device=dev)
    _check(out, "out", dt, dev)
    _check(route_idx, "route_idx", torch.int32, dev)
    if out.shape != x.shape or route_idx.numel() != N * S * S * topk:
        raise ValueError("out / route_idx have the wrong size")
    with torch.cuda.device(dev):
        _stream(dev)
        _call("bra_block_forward", _ptr(x), _ptr(wqkv), _ptr(bqkv), _ptr(lce_w), _ptr(lce_b),
              _ptr(wo), _ptr(bo), N, H, W, C, heads, S, topk, _dtype_code(x), _ptr(out),
              _ptr(route_idx))
    return out, route_idx


def block_fused(N: int, H: int, W: int, C: int, heads: int, S: int, topk: int, dtype) -> bool:
    """Does bra_block_forward run these sizes fused? dtype: torch dtype."""
    code = BF16 if dtype == torch.bfloat16 else F32
    return bool(load().bra_block_fused(N, H, W, C, heads, S, topk, code))


def workspace_bytes(N: int, C: int, S: int) -> int:
    return int(load().bra_workspace_bytes(N, C, S))


def release() -> None:
    load().bra_release()


def version() -> int:
    return int(load().bra_version())


def profile_begin(kinds=KERNEL_NAMES) -> None:
    """Records HIP events around the named kernel kinds ("pool", "route",
    "attn", "lce"); an empty sequence (or False) stops recording."""
    if kinds is True:
        kinds = KERNEL_NAMES
    mask = 0
    for k in (kinds or ()):
        mask |= 1 << KERNEL_NAMES.index(k)
    _call("bra_profile_begin", mask)


def profile_set_mask(kinds=KERNEL_NAMES) -> None:
    """Changes which kernel kinds are recorded from the next launch on,
    keeping what was recorded so far."""
    mask = 0
    for k in (kinds or ()):
        mask |= 1 << KERNEL_NAMES.index(k)
    _call("bra_profile_set_mask", mask)


def profile_read() -> dict:
    """Summed event milliseconds and launch counts per kernel kind since the
    last profile_begin/profile_read (synchronises on the recorded events)."""
    n = len(KERNEL_NAMES)
    ms = (ctypes.c_double * n)()
    cnt = (ctypes.c_int * n)()
    _call("bra_profile_read", ms, cnt, n)
    return {KERNEL_NAMES[i]: (ms[i], cnt[i]) for i in range(n)}


def calib_copy(src: torch.Tensor, dst: torch.Tensor) -> None:
    _check(src, "src")
    _check(dst, "dst", device=src.device)
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() < nbytes:
        raise ValueError("dst too small")
    with torch.cuda.device(src.device):
        _stream(src.device)
        _call("bra_calib_copy", _ptr(src), _ptr(dst), nbytes)
