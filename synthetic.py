"""Seeded synthetic inputs for the W4A16 MoE expert layer.

This module is shared by the CPU oracle and the HIP path and holds none of the
method's arithmetic: it only draws random tensors (and the random routing trace
of the slot-cache workload) with NumPy's PCG64, one child stream per tensor,
and converts fp32 draws to bf16 bit patterns (round to nearest even) the way any
bf16 input tensor would be stored.

Child-stream order for ``SeedSequence(seed).spawn``: 0 router, 1+3e gate,
2+3e up, 3+3e down of expert e, then x, the logit-bias permutation and the trace.
"""
from __future__ import annotations

import math
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass

import numpy as np

__all__ = [
    "f32_to_bf16_bits", "bf16_bits_to_f32", "LayerShape", "SyntheticLayer",
    "TINY", "OLMOE", "LARGE", "zipf_logit_bias", "slot_cache_trace",
]


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit pattern (uint16), round to nearest, ties to even."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


@dataclass(frozen=True)
class LayerShape:
    H: int          # hidden size
    I: int          # expert intermediate size
    E: int          # experts
    k: int          # experts per token
    w_sigma: float = 0.02      # expert weight std
    router_sigma: float = 0.02


TINY = LayerShape(H=256, I=256, E=8, k=2)                         # 16-token tiny layer
OLMOE = LayerShape(H=2048, I=1024, E=64, k=8)                      # OLMoE-shaped layer
LARGE = LayerShape(H=4096, I=14336, E=8, k=2, w_sigma=0.01)        # large-expert prefill layer


class SyntheticLayer:
    """One MoE layer's seeded inputs. Expert weights are drawn lazily per expert."""

    def __init__(self, shape: LayerShape, seed: int = 0, layer: int = 0):
        self.shape = shape
        self.seed = seed
        self.layer = layer
        ss = np.random.SeedSequence([seed, layer]) if layer else np.random.SeedSequence(seed)
        self._children = ss.spawn(3 * shape.E + 4)

    def _rng(self, i: int) -> np.random.Generator:
        return np.random.Generator(np.random.PCG64(self._children[i]))

    def router(self) -> np.ndarray:
        """Router weight, bf16 bits [E, H], ~N(0, router_sigma)."""
        s = self.shape
        w = self._rng(0).standard_normal((s.E, s.H), dtype=np.float32) * np.float32(s.router_sigma)
        return f32_to_bf16_bits(w)

    def expert(self, e: int):
        """fp32 (gate [I,H], up [I,H], down [H,I]) of expert e, ~N(0, w_sigma)."""
        s = self.shape
        sig = np.float32(s.w_sigma)
        g = self._rng(1 + 3 * e).standard_normal((s.I, s.H), dtype=np.float32) * sig
        u = self._rng(2 + 3 * e).standard_normal((s.I, s.H), dtype=np.float32) * sig
        d = self._rng(3 + 3 * e).standard_normal((s.H, s.I), dtype=np.float32) * sig
        return g, u, d

    def experts(self, which=None, threads: int = 8):
        which = range(self.shape.E) if which is None else which
        with ThreadPoolExecutor(threads) as ex:
            return list(ex.map(self.expert, which))

    def x(self, T: int, stream: int = 0) -> np.ndarray:
        """Activations, bf16 bits [T, H], ~N(0, 1). ``stream`` picks an independent draw."""
        s = self.shape
        ss = self._children[3 * s.E + 1]
        if stream:
            ss = np.random.SeedSequence(entropy=ss.entropy, spawn_key=ss.spawn_key + (stream,))
        r = np.random.Generator(np.random.PCG64(ss))
        return f32_to_bf16_bits(r.standard_normal((T, s.H), dtype=np.float32))

    def zipf_bias(self, s_exp: float = 1.1) -> np.ndarray:
        return zipf_logit_bias(self.shape.E, self._rng(3 * self.shape.E + 2), s_exp)

    def trace_rng(self) -> np.random.Generator:
        return self._rng(3 * self.shape.E + 3)


def zipf_logit_bias(E: int, rng: np.random.Generator, s_exp: float = 1.1) -> np.ndarray:
    """Per-expert fp32 logit bias: the expert at Zipf rank r gets -s*ln(r), ranks over a
    seeded random permutation, so exp(bias) follows Zipf(s) popularity."""
    perm = rng.permutation(E)
    b = np.empty(E, dtype=np.float32)
    for r in range(1, E + 1):
        b[perm[r - 1]] = np.float32(-s_exp * math.log(r))
    return b


def slot_cache_trace(E: int, k: int, layers: int, steps: int, seed: int,
                     s_exp: float = 1.1, reuse: float = 0.5) -> np.ndarray:
    """Routing trace int32 [steps, layers, k] of distinct expert ids per (step, layer).

    Per layer, popularity p[perm(r)] ~ r^-s over a seeded permutation. Step 0 draws k
    distinct experts from p. Each later pick is, with probability ``reuse``, uniform over
    the previous step's experts not yet picked, else drawn from p renormalized over the
    experts not yet picked.
    """
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0xC3])))
    out = np.empty((steps, layers, k), dtype=np.int32)
    ranks = np.arange(1, E + 1, dtype=np.float64) ** (-s_exp)
    for l in range(layers):
        perm = rng.permutation(E)
        p = np.empty(E)
        p[perm] = ranks
        p /= p.sum()
        prev: list[int] = []
        for st in range(steps):
            chosen: list[int] = []
            for _ in range(k):
                cand_prev = [e for e in prev if e not in chosen]
                if st > 0 and cand_prev and rng.random() < reuse:
                    e = cand_prev[int(rng.integers(len(cand_prev)))]
                else:
                    q = p.copy()
                    q[chosen] = 0.0
                    q /= q.sum()
                    e = int(rng.choice(E, p=q))
                chosen.append(e)
            out[st, l] = chosen
            prev = chosen
    return out


def batch_trace(E: int, k: int, layers: int, steps: int, batch: int, seed: int,
                s_exp: float = 1.1, reuse: float = 0.5) -> np.ndarray:
    """Routing trace int32 [steps, layers, batch, k] of a batch of sequences decoded together.

    The sequences share each layer's Zipf(s) popularity over a seeded permutation (one
    model); each sequence walks it on its own generator like slot_cache_trace: step 0 draws
    k distinct experts, each later pick is, with probability ``reuse``, uniform over that
    sequence's previous experts not yet picked, else drawn from the popularity renormalized
    over the experts not yet picked.
    """
    pop = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0xB7])))
    ranks = np.arange(1, E + 1, dtype=np.float64) ** (-s_exp)
    out = np.empty((steps, layers, batch, k), dtype=np.int32)
    for l in range(layers):
        perm = pop.permutation(E)
        p = np.empty(E)
        p[perm] = ranks
        p /= p.sum()
        for b in range(batch):
            rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0xB8, l, b])))
            prev: list[int] = []
            for st in range(steps):
                chosen: list[int] = []
                for _ in range(k):
                    cand_prev = [e for e in prev if e not in chosen]
                    if st > 0 and cand_prev and rng.random() < reuse:
                        e = cand_prev[int(rng.integers(len(cand_prev)))]
                    else:
                        q = p.copy()
                        q[chosen] = 0.0
                        q /= q.sum()
                        e = int(rng.choice(E, p=q))
                    chosen.append(e)
                out[st, l, b] = chosen
                prev = chosen
    return out

