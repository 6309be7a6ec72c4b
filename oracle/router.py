"""BF16 router and unchanged top-k selection (oracle).

The pages keep the router in BF16 and the top-k routing procedure unchanged: the
original router picks the experts and every picked expert runs (ExactMoE abstract;
Fig. 1 caption). Readings where the pages are silent:
  * logits are a bf16 linear layer's output: exact bf16 x bf16 products summed in fp64,
    plus an optional fp32 per-expert bias, rounded once to bf16;
  * selection is on the bf16 logits, ordered by (logit descending, expert id ascending),
    slots 0..k-1 in that order (-0 and +0 compare equal);
  * weights: softmax over the selected logits (the full softmax renormalized over the
    top-k); with renormalize=False, the full-softmax probability of each selected expert.
"""
from __future__ import annotations

import numpy as np

from .quant import bf16_bits_to_f64, f64_to_bf16_bits


def router_logits(x_bits: np.ndarray, wr_bits: np.ndarray, bias=None) -> np.ndarray:
    """x bf16 bits [T, H], router bf16 bits [E, H], bias fp32 [E] or None -> bf16 bits [T, E]."""
    x = bf16_bits_to_f64(x_bits)
    w = bf16_bits_to_f64(wr_bits)
    acc = x @ w.T                                   # fp64 accumulation of exact products
    if bias is not None:
        acc = acc + np.asarray(bias, dtype=np.float32).astype(np.float64)[None, :]
    return f64_to_bf16_bits(acc)


def topk_ids(logit_bits: np.ndarray, k: int) -> np.ndarray:
    """bf16 bits [T, E] -> int32 [T, k]: first k of the stable order (logit desc, id asc)."""
    l = bf16_bits_to_f64(logit_bits)
    T, E = l.shape
    assert 1 <= k <= E
    # argsort of -l with a stable sort keeps equal logits in ascending expert order;
    # -0.0 == +0.0 compares equal, so signed zeros tie as the reading requires.
    order = np.argsort(-l, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def topk_weights(logit_bits: np.ndarray, ids: np.ndarray, renormalize: bool = True) -> np.ndarray:
    """Routing weights fp32 [T, k], computed in fp64."""
    l = bf16_bits_to_f64(logit_bits)
    T, E = l.shape
    sel = np.take_along_axis(l, ids.astype(np.int64), axis=1)          # [T, k]
    if renormalize:
        m = sel.max(axis=1, keepdims=True)
        p = np.exp(sel - m)
        w = p / p.sum(axis=1, keepdims=True)
    else:
        m = l.max(axis=1, keepdims=True)
        z = np.exp(l - m).sum(axis=1, keepdims=True)
        w = np.exp(sel - m) / z
    return w.astype(np.float32)
