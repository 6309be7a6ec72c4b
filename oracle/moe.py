"""Expert SwiGLU MLPs on dequantized int4 weights and the weighted combine (oracle).

The pages run every selected expert in full with int4 routed-expert weights
(ExactMoE abstract; Fig. 1 caption). The expert MLP itself is not written on the pages;
the reading used is the SwiGLU expert of the OLMoE-shaped workload:
  g = W_gate x, u = W_up x, a = silu(g) * u, o = W_down a,   silu(z) = z / (1 + e^-z),
with W the dequantized weights q*s. Everything is fp64 (no bf16 rounding of a).
Combine: y[t] = sum over slots j = 0..k-1, in that order, of w[t, j] * o[t, j].

Two drivers compute the same thing: forward_per_token (loop over t, then j) and
forward_grouped (loop over experts ascending, rows of each segment in sorted order,
then combine); with rowwise=True their per-row arithmetic is identical.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from .quant import quantize_group128, dequantize_group128


@dataclass
class QuantExpert:
    qg: np.ndarray
    sg: np.ndarray
    qu: np.ndarray
    su: np.ndarray
    qd: np.ndarray
    sd: np.ndarray
    _deq: dict = field(default_factory=dict, repr=False)

    def deq(self):
        if not self._deq:
            self._deq["g"] = dequantize_group128(self.qg, self.sg)
            self._deq["u"] = dequantize_group128(self.qu, self.su)
            self._deq["d"] = dequantize_group128(self.qd, self.sd)
        return self._deq["g"], self._deq["u"], self._deq["d"]

    def drop_cache(self):
        self._deq.clear()


@dataclass
class DenseExpert:
    """An expert of the comparator layer: bf16 weights (bits), used as they are (abstract;
    Tab. 1 and Tab. 4: the same model with its experts in bf16). deq() gives the weights as
    fp64, so every driver below runs it unchanged."""
    g_bits: np.ndarray
    u_bits: np.ndarray
    d_bits: np.ndarray
    _w: dict = field(default_factory=dict, repr=False)

    def deq(self):
        from .quant import bf16_bits_to_f64
        if not self._w:
            self._w["g"] = bf16_bits_to_f64(self.g_bits)
            self._w["u"] = bf16_bits_to_f64(self.u_bits)
            self._w["d"] = bf16_bits_to_f64(self.d_bits)
        return self._w["g"], self._w["u"], self._w["d"]

    def drop_cache(self):
        self._w.clear()


def quantize_expert(w_gate, w_up, w_down) -> QuantExpert:
    qg, sg = quantize_group128(w_gate)
    qu, su = quantize_group128(w_up)
    qd, sd = quantize_group128(w_down)
    return QuantExpert(qg, sg, qu, su, qd, sd)


def expert_mlp(qe: QuantExpert, x: np.ndarray) -> np.ndarray:
    """x fp64 [n, H] -> o fp64 [n, H] for one expert."""
    wg, wu, wd = qe.deq()
    g = x @ wg.T
    u = x @ wu.T
    with np.errstate(over="ignore"):
        a = g / (1.0 + np.exp(-g)) * u
    return a @ wd.T


def combine(o_flat: np.ndarray, weights: np.ndarray, T: int, k: int) -> np.ndarray:
    """o_flat fp64 [T*k, H] in flat (t, j) order, weights fp32 [T, k] -> y fp64 [T, H]."""
    H = o_flat.shape[1] if o_flat.ndim == 2 else 0
    y = np.zeros((T, H), dtype=np.float64)
    w = np.asarray(weights, dtype=np.float32).astype(np.float64)
    for j in range(k):                      # fixed slot order
        y += w[:, j:j + 1] * o_flat.reshape(T, k, H)[:, j, :]
    return y


def forward_per_token(x_bits_f64: np.ndarray, ids: np.ndarray, weights: np.ndarray,
                      experts, tokens=None) -> np.ndarray:
    """Per-token sequential driver. x fp64 [T, H]; returns y fp64 [len(tokens), H]."""
    T, k = ids.shape
    tokens = range(T) if tokens is None else tokens
    rows = []
    for t in tokens:
        o = np.stack([expert_mlp(experts[int(ids[t, j])], x_bits_f64[t:t + 1])[0] for j in range(k)])
        rows.append(combine(o, weights[t:t + 1], 1, k)[0])
    return np.stack(rows) if rows else np.zeros((0, x_bits_f64.shape[1]))


def forward_grouped(x_bits_f64: np.ndarray, ids: np.ndarray, weights: np.ndarray, experts,
                    offsets: np.ndarray, sorted_flat: np.ndarray, rowwise: bool = False,
                    return_o: bool = False):
    """Grouped driver: experts ascending, each segment's rows in sorted order.

    rowwise=True runs one row at a time (the per-token driver's exact arithmetic);
    rowwise=False runs each segment as one batched product.
    """
    T, k = ids.shape
    H = x_bits_f64.shape[1]
    E = offsets.shape[0] - 1
    o_flat = np.zeros((T * k, H), dtype=np.float64)
    for e in range(E):
        seg = sorted_flat[offsets[e]:offsets[e + 1]]
        if seg.size == 0:
            continue
        toks = seg // k
        if rowwise:
            for f, t in zip(seg, toks):
                o_flat[f] = expert_mlp(experts[e], x_bits_f64[t:t + 1])[0]
        else:
            o_flat[seg] = expert_mlp(experts[e], x_bits_f64[toks])
    y = combine(o_flat, weights, T, k)
    return (y, o_flat) if return_o else y


def knockout_rows(ids: np.ndarray, e: int) -> np.ndarray:
    """Tokens whose output depends on expert e (those routed to it)."""
    return np.nonzero((np.asarray(ids) == e).any(axis=1))[0]


def moe_layer(x_bits: np.ndarray, wr_bits: np.ndarray, experts, k: int, bias=None,
              renormalize: bool = True, tokens=None):
    """Whole layer: logits -> top-k -> weights -> per-token expert MLPs -> combine.

    Returns dict with logits (bf16 bits), ids, weights, offsets, sorted_flat,
    flat_to_sorted and y (fp64, rows ``tokens`` or all).
    """
    from .router import router_logits, topk_ids, topk_weights
    from .group import group_tokens
    from .quant import bf16_bits_to_f64
    E = wr_bits.shape[0]
    logits = router_logits(x_bits, wr_bits, bias)
    ids = topk_ids(logits, k)
    w = topk_weights(logits, ids, renormalize)
    offsets, sorted_flat, flat_to_sorted = group_tokens(ids, E)
    x = bf16_bits_to_f64(x_bits)
    y = forward_per_token(x, ids, w, experts, tokens)
    return dict(logits=logits, ids=ids, weights=w, offsets=offsets, sorted_flat=sorted_flat,
                flat_to_sorted=flat_to_sorted, y=y)
