"""Symmetric group-128 int4 weight quantization (oracle).

Follows the ExactMoE abstract: symmetric int4 with one scale per 128 inputs, applied to
the routed experts only. Readings where the pages are silent:
  * scale divisor: s = absmax / 7 (largest positive int4 code), computed as an IEEE
    fp32 division, then rounded to bf16 (nearest, ties to even);
  * code: q = clamp(round_half_even(w / s), -8, 7), the quotient formed in fp64
    (exact enough that no false .5 tie can arise for fp32 / bf16 operands);
  * an all-zero group has s = 0 and q = 0.
Dequantized weight: q * s (exact in fp32 and fp64).
"""
from __future__ import annotations

import numpy as np

GROUP = 128


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bits, round to nearest even (finite inputs)."""
    u = np.asarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    return ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    """fp64 -> bf16 bits with ONE rounding (nearest, ties to even), no detour via fp32.

    For a normal value with binary exponent e (2^e <= |v| < 2^(e+1)) bf16 keeps 8
    significant bits, so the quantum is 2^(e-7); the rounded value is rint(v/2^(e-7))*2^(e-7),
    exact in fp64. Subnormal bf16 values share the quantum 2^-133.
    """
    v = np.asarray(v, dtype=np.float64)
    m, e = np.frexp(v)                  # v = m * 2^e, 0.5 <= |m| < 1  ->  2^(e-1) <= |v|
    quantum_exp = np.maximum(e - 1 - 7, -133)
    r = np.ldexp(np.rint(np.ldexp(v, -quantum_exp)), quantum_exp)
    r32 = r.astype(np.float32)          # exact: r has <= 8 significant bits and is in range
    return (r32.view(np.uint32) >> 16).astype(np.uint16)


def quantize_group128(w: np.ndarray):
    """w fp32 [N, K] (K % 128 == 0) -> (q int8 [N, K], s bf16 bits [N, K/128])."""
    w = np.asarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % GROUP == 0
    G = K // GROUP
    wg = w.reshape(N, G, GROUP)
    absmax = np.max(np.abs(wg), axis=2)                       # fp32 [N, G]
    s_f32 = absmax / np.float32(7.0)                          # IEEE fp32 division
    s_bits = _f32_to_bf16_bits(s_f32)
    s = bf16_bits_to_f64(s_bits)                              # exact
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = wg.astype(np.float64) / s[:, :, None]
    q = np.where(s[:, :, None] == 0.0, 0.0, np.clip(np.rint(quot), -8, 7))
    return q.reshape(N, K).astype(np.int8), s_bits


def dequantize_group128(q: np.ndarray, s_bits: np.ndarray) -> np.ndarray:
    """(q int8 [N, K], s bf16 bits [N, K/128]) -> fp64 [N, K] = q * s."""
    N, K = q.shape
    s = bf16_bits_to_f64(s_bits)
    return (q.reshape(N, K // GROUP, GROUP).astype(np.float64) * s[:, :, None]).reshape(N, K)
