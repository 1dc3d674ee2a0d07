"""Planted mistakes in the oracle (CPU only): each plausible error -- a dropped
term, a wrong sign, index, axis or orientation, a transposed operand -- must
make at least one pin fail. This shows the pins constrain the oracle rather
than echo it."""
import numpy as np
import pytest

from oracle import bra_oracle as O
from tests import oracle_pins as P


def _partition_swapped(x, S):
    N, H, W, C = x.shape
    y = x.reshape(N, S, H // S, S, W // S, C).transpose(0, 3, 1, 2, 4, 5)  # region i-major
    return y.reshape(N, S * S, -1, C)


def _means_over_channels(xp):
    return np.repeat(xp.mean(axis=3, keepdims=True), xp.shape[3], axis=3).mean(axis=2)


def _means_wrong_count(xp):
    return xp.sum(axis=2) / (xp.shape[2] + 1)


def _affinity_no_scale(qr, kr):
    return qr @ np.swapaxes(kr, -1, -2)


def _affinity_transposed(qr, kr):
    C = qr.shape[-1]
    return (kr / np.sqrt(C)) @ np.swapaxes(qr, -1, -2)


def _topk_ascending(A, topk):
    return np.argsort(A, axis=-1, kind="stable")[..., :topk]


def _topk_ties_high(A, topk):
    R = A.shape[-1]
    rev = np.argsort(-A[..., ::-1], axis=-1, kind="stable")
    return (R - 1 - rev)[..., :topk]


def _attention_variant(scale_mode="hd", axis=-1, head_split="major"):
    def f(qp, kg, vg, heads, return_probs=False):
        N, R, T, C = qp.shape
        hd = C // heads
        scale = 1.0 / np.sqrt(C if scale_mode == "C" else hd)
        out = np.empty_like(qp)
        probs = []
        for m in range(heads):
            sl = slice(m * hd, (m + 1) * hd) if head_split == "major" else slice(m, C, heads)
            s = (qp[..., sl] * scale) @ np.swapaxes(kg[..., sl], -1, -2)
            s = s - s.max(axis=axis, keepdims=True)
            e = np.exp(s)
            p = e / e.sum(axis=axis, keepdims=True)
            out[..., sl] = p @ vg[..., sl]
            probs.append(p)
        return (out, probs) if return_probs else out
    return f


def _gather_shifted(xp, route):
    R = xp.shape[1]
    return O.__dict__["_orig_gather"]((xp), (route + 1) % R)


def _lce_flipped(v, w, b):
    return O.__dict__["_orig_lce"](v, w[:, ::-1, ::-1], b)


def _lce_no_bias(v, w, b):
    return O.__dict__["_orig_lce"](v, w, None)


def _lce_per_region_padding(v, w, b):
    # pads each half of the image separately, as if LCE ran per region
    H = v.shape[1]
    h = H // 2
    top = O.__dict__["_orig_lce"](v[:, :h], w, b)
    bot = O.__dict__["_orig_lce"](v[:, h:], w, b)
    return np.concatenate([top, bot], axis=1)


def _lce_dropped(v, w, b):
    return np.zeros_like(v)


def _linear_weight_not_transposed(x, w, b=None):
    y = np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64)
    return y if b is None else y + b


def _linear_bias_dropped(x, w, b=None):
    return np.asarray(x, dtype=np.float64) @ np.asarray(w, dtype=np.float64).T


def _round_bf16_truncates(x):
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    return (f.view(np.uint32) >> 16 << 16).view(np.float32).astype(np.float64)


def _round_bf16_ties_up(x):
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    return ((u + 0x8000) >> 16 << 16).astype(np.uint32).view(np.float32).astype(np.float64)


def _block_kv_swapped(x, wqkv, bqkv, lce_w, lce_b, wo, bo, heads, S, topk, store=None,
                      route_override=None):
    C = np.asarray(x).shape[-1]
    wqkv = np.asarray(wqkv, dtype=np.float64)
    wqkv = np.concatenate([wqkv[:C], wqkv[2 * C:], wqkv[C:2 * C]])
    if bqkv is not None:
        bqkv = np.concatenate([bqkv[:C], bqkv[2 * C:], bqkv[C:2 * C]])
    return O.__dict__["_orig_block"](x, wqkv, bqkv, lce_w, lce_b, wo, bo, heads, S, topk,
                                     store, route_override)


def _dense_variant(mode):
    def f(q, k, v, lce_w, lce_b, heads):
        q, k, v = (np.asarray(x, dtype=np.float64) for x in (q, k, v))
        N, H, W, C = q.shape
        hd = C // heads
        scale = 1.0 / np.sqrt(C if mode == "scale_C" else hd)
        axis = 0 if mode == "softmax_over_queries" else 1
        att = np.empty((N, H * W, C))
        for n in range(N):
            qn, kn, vn = (x[n].reshape(H * W, C) for x in (q, k, v))
            if mode == "k_v_swapped":
                kn, vn = vn, kn
            for m in range(heads):
                sl = slice(m * hd, (m + 1) * hd)
                s = (qn[:, sl] @ kn[:, sl].T) * scale
                e = np.exp(s - s.max(axis=axis, keepdims=True))
                att[n][:, sl] = (e / e.sum(axis=axis, keepdims=True)) @ vn[:, sl]
        att = att.reshape(N, H, W, C)
        if mode == "lepe_dropped":
            return att
        lw = np.asarray(lce_w, dtype=np.float64).reshape(C, 5, 5)
        if mode == "lepe_on_q":
            return att + O.lce(q, lw, lce_b)
        return att + O.lce(v, lw, lce_b)
    return f


def _head_routed_shared(q, k, v, lce_w, lce_b, heads, S, topk, route_override=None):
    # routes once over all channels and gives every head that choice
    base = O.bra_forward(q, k, v, lce_w, lce_b, heads, S, topk)
    r = np.repeat(base["route_idx"][:, None], heads, axis=1)
    lg = np.repeat(base["logits"][:, None], heads, axis=1)
    return {"out": base["out"], "route_idx": r, "route_oracle": r, "logits": lg}


def _head_routed_heads_swapped(q, k, v, lce_w, lce_b, heads, S, topk, route_override=None):
    res = O.__dict__["_orig_head_routed"](q, k, v, lce_w, lce_b, heads, S, topk)
    perm = np.roll(np.arange(heads), 1)
    again = O.__dict__["_orig_head_routed"](q, k, v, lce_w, lce_b, heads, S, topk,
                                            route_override=res["route_idx"][:, perm])
    again["logits"] = res["logits"][:, perm]
    again["route_oracle"] = res["route_idx"][:, perm]
    return again


def _head_routed_scale_C(q, k, v, lce_w, lce_b, heads, S, topk, route_override=None):
    res = O.__dict__["_orig_head_routed"](q, k, v, lce_w, lce_b, heads, S, topk, route_override)
    res["logits"] = res["logits"] / np.sqrt(heads)   # C^-1/2 instead of head_dim^-1/2
    return res


def _backward_variant(mode):
    """bra_backward with one planted mistake (the same steps otherwise)."""
    def f(q, k, v, lce_w, route, dout, heads, S):
        q, k, v, g = (np.asarray(x, dtype=np.float64) for x in (q, k, v, dout))
        N, H, W, C = q.shape
        route = np.asarray(route, dtype=np.int64)
        R, hd = S * S, C // heads
        scale = 1.0 / np.sqrt(hd)
        w = np.asarray(lce_w, dtype=np.float64).reshape(C, 5, 5)
        qp, kp, vp, gp = (O.partition(x, S) for x in (q, k, v, g))
        T = qp.shape[2]
        dqp, dkp, dvp = np.zeros_like(qp), np.zeros_like(kp), np.zeros_like(vp)
        for n in range(N):
            for m in range(heads):
                sl = slice(m * hd, (m + 1) * hd)
                for r in range(R):
                    Q, G = qp[n, r, :, sl], gp[n, r, :, sl]
                    rr = (route[n, r] + 1) % R if mode == "scatter_wrong_region" else route[n, r]
                    Kg = np.concatenate([kp[n, s, :, sl] for s in route[n, r]])
                    Vg = np.concatenate([vp[n, s, :, sl] for s in route[n, r]])
                    sc = (Q @ Kg.T) * scale
                    P = np.exp(sc - sc.max(axis=1, keepdims=True))
                    P /= P.sum(axis=1, keepdims=True)
                    dP = G @ Vg.T
                    D = 0.0 if mode == "no_D" else (P * dP).sum(axis=1, keepdims=True)
                    dS = P * (dP - D)
                    dqp[n, r, :, sl] += (1.0 if mode == "dq_unscaled" else scale) * (dS @ Kg)
                    dK, dV = scale * (dS.T @ Q), P.T @ G
                    for i, s in enumerate(rr):
                        dkp[n, s, :, sl] += dK[i * T:(i + 1) * T]
                        dvp[n, s, :, sl] += dV[i * T:(i + 1) * T]
        dq, dk, dv = (O.unpartition(x, S, H, W) for x in (dqp, dkp, dvp))
        gpad = np.zeros((N, H + 4, W + 4, C))
        gpad[:, 2:H + 2, 2:W + 2, :] = g
        vpad = np.zeros((N, H + 4, W + 4, C))
        vpad[:, 2:H + 2, 2:W + 2, :] = v
        dw = np.zeros((C, 5, 5))
        for a in range(5):
            for e in range(5):
                src = gpad[:, a:a + H, e:e + W, :] if mode == "lce_dv_unflipped" else \
                    gpad[:, 4 - a:4 - a + H, 4 - e:4 - e + W, :]
                dv += w[:, a, e] * src
                dw[:, a, e] = (g * vpad[:, a:a + H, e:e + W, :]).sum(axis=(0, 1, 2))
        if mode == "lce_dw_transposed":
            dw = np.swapaxes(dw, 1, 2)
        return {"dq": dq, "dk": dk, "dv": dv, "dlce_w": dw, "dlce_b": g.sum(axis=(0, 1, 2))}
    return f


MUTATIONS = {
    "backward_without_D": ("bra_backward", _backward_variant("no_D")),
    "backward_dq_unscaled": ("bra_backward", _backward_variant("dq_unscaled")),
    "backward_scatter_wrong_region": ("bra_backward", _backward_variant("scatter_wrong_region")),
    "backward_lce_dv_unflipped": ("bra_backward", _backward_variant("lce_dv_unflipped")),
    "backward_lce_dw_transposed": ("bra_backward", _backward_variant("lce_dw_transposed")),
    "head_routed_shares_routes": ("bra_forward_head_routed", _head_routed_shared),
    "head_routed_heads_swapped": ("bra_forward_head_routed", _head_routed_heads_swapped),
    "head_routed_scale_uses_C": ("bra_forward_head_routed", _head_routed_scale_C),
    "dense_scale_uses_C": ("dense_attention", _dense_variant("scale_C")),
    "dense_softmax_over_queries": ("dense_attention", _dense_variant("softmax_over_queries")),
    "dense_k_and_v_swapped": ("dense_attention", _dense_variant("k_v_swapped")),
    "dense_lepe_dropped": ("dense_attention", _dense_variant("lepe_dropped")),
    "dense_lepe_on_q": ("dense_attention", _dense_variant("lepe_on_q")),
    "linear_weight_not_transposed": ("linear", _linear_weight_not_transposed),
    "linear_bias_dropped": ("linear", _linear_bias_dropped),
    "round_bf16_truncates": ("round_bf16", _round_bf16_truncates),
    "round_bf16_ties_away": ("round_bf16", _round_bf16_ties_up),
    "block_k_and_v_swapped": ("bra_block_forward", _block_kv_swapped),
    "partition_region_order_swapped": ("partition", _partition_swapped),
    "means_over_channels": ("region_means", _means_over_channels),
    "means_wrong_count": ("region_means", _means_wrong_count),
    "affinity_scale_dropped": ("region_affinity", _affinity_no_scale),
    "affinity_operands_transposed": ("region_affinity", _affinity_transposed),
    "topk_ascending": ("topk_routes", _topk_ascending),
    "topk_ties_to_higher_index": ("topk_routes", _topk_ties_high),
    "attention_scale_uses_C": ("token_attention", _attention_variant(scale_mode="C")),
    "softmax_over_query_axis": ("token_attention", _attention_variant(axis=-2)),
    "head_split_interleaved": ("token_attention", _attention_variant(head_split="minor")),
    "gather_wrong_region": ("gather_regions", _gather_shifted),
    "lce_kernel_flipped": ("lce", _lce_flipped),
    "lce_bias_dropped": ("lce", _lce_no_bias),
    "lce_padded_per_region": ("lce", _lce_per_region_padding),
    "lce_term_dropped": ("lce", _lce_dropped),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_some_pin_catches(name, monkeypatch):
    attr, bad = MUTATIONS[name]
    monkeypatch.setitem(O.__dict__, "_orig_gather", O.gather_regions)
    monkeypatch.setitem(O.__dict__, "_orig_lce", O.lce)
    monkeypatch.setitem(O.__dict__, "_orig_block", O.bra_block_forward)
    monkeypatch.setitem(O.__dict__, "_orig_head_routed", O.bra_forward_head_routed)
    monkeypatch.setattr(O, attr, bad)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(O)
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin catches the planted mistake {name}"
