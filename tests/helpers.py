"""Shared helpers of the GPU parity tests: build a seeded layer for both sides (the
library packs it, the oracle quantizes it on its own), move bf16 bit patterns to the
device, and apply the layer-output tolerance."""
from __future__ import annotations

import sys
from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle
from synthetic import SyntheticLayer, bf16_bits_to_f32

# Layer output tolerance: max|dy| / max|y_ref| <= 1e-2 over the tensor, and per element
# |dy| <= 1e-2 |y_ref| + 1e-2 rms(y_ref[t, :]) (pure elementwise relative error is
# unbounded where outputs cross zero).
REL_TOL = 1e-2


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


class Layer:
    """Seeded layer: fp32 expert weights, library blobs (device bank) and oracle experts."""

    def __init__(self, shape, seed=0, experts=None, device="cuda", oracle_experts=True, layer=0):
        import torch
        import w4a16_mixture_experts_amd as exm
        self.shape = shape
        self.syn = SyntheticLayer(shape, seed=seed, layer=layer)
        which = list(range(shape.E)) if experts is None else experts
        self.wr_bits = self.syn.router()
        blobs = {}
        qexp = {}

        def one(e):
            g, u, d = self.syn.expert(e)
            b = exm.quantize_pack(g, u, d)
            q = oracle.quantize_expert(g, u, d) if oracle_experts else None
            return e, b, q

        with ThreadPoolExecutor(8) as ex:
            for e, b, q in ex.map(one, which):
                blobs[e] = b
                qexp[e] = q
        nb = exm.packed_expert_bytes(shape.H, shape.I)
        zero = np.zeros(nb, np.uint8)
        self.blobs = [blobs.get(e, zero) for e in range(shape.E)]
        self.experts = [qexp.get(e) for e in range(shape.E)]
        self.bank = exm.bank_from_blobs(self.blobs, device)
        self.wr = to_dev_bf16(self.wr_bits, device)
        self.device = device
        self.bf16_bank = None

    def add_bf16(self, oracle_experts=True):
        """The comparator's dense bf16 experts: the same fp32 weights rounded to bf16 (an
        input of both sides), packed by the library, read as they are by the oracle."""
        import w4a16_mixture_experts_amd as exm
        from synthetic import f32_to_bf16_bits

        def one(e):
            bits = [f32_to_bf16_bits(w) for w in self.syn.expert(e)]
            return exm.bf16_pack(*bits), (oracle.DenseExpert(*bits) if oracle_experts else None)

        with ThreadPoolExecutor(8) as ex:
            res = list(ex.map(one, range(self.shape.E)))
        self.bf16_blobs = [b for b, _ in res]
        self.dense = [d for _, d in res]
        self.bf16_bank = exm.bank_from_blobs(self.bf16_blobs, self.device)
        return self


def to_dev_bf16(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)


def bf16_dev_to_bits(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_dev_to_f64(t) -> np.ndarray:
    return bf16_bits_to_f32(bf16_dev_to_bits(t)).astype(np.float64)


def check_y(y_gpu: np.ndarray, y_ref: np.ndarray, label: str = "") -> float:
    assert y_gpu.shape == y_ref.shape, (y_gpu.shape, y_ref.shape)
    assert np.all(np.isfinite(y_gpu)), f"{label}: non-finite GPU output"
    d = np.abs(y_gpu - y_ref)
    scale = np.abs(y_ref).max()
    rel = d.max() / scale if scale > 0 else d.max()
    rms = np.sqrt(np.mean(y_ref ** 2, axis=1, keepdims=True))
    bound = REL_TOL * np.abs(y_ref) + REL_TOL * rms
    bad = d > bound
    log(f"  {label}: max|dy|/max|y| = {rel:.3e}, worst elem ratio = {(d / np.maximum(bound, 1e-300)).max():.3f}")
    assert rel <= REL_TOL, f"{label}: max|dy|/max|y| = {rel:.3e}"
    assert not bad.any(), f"{label}: {bad.sum()} elements outside the per-element bound"
    return rel


def check_routing(gpu: dict, ref: dict, label: str = ""):
    """Integer outputs bit-exact; weights within 1e-6 absolute."""
    if "logits" in gpu:
        lg, lr = gpu["logits"], ref["logits"]
        if not np.array_equal(lg, lr):
            bad = np.argwhere(lg != lr)
            raise AssertionError(f"{label}: {len(bad)} logits differ, first {bad[:5].tolist()}")
    assert np.array_equal(gpu["ids"], ref["ids"]), f"{label}: top-k ids differ"
    dw = np.abs(gpu["weights"].astype(np.float64) - ref["weights"].astype(np.float64)).max()
    assert dw <= 1e-6, f"{label}: routing weights differ by {dw:.2e}"
    for key in ("offsets", "sorted_flat", "flat_to_sorted"):
        if key in gpu:
            assert np.array_equal(gpu[key], ref[key]), f"{label}: {key} differs"
