"""Group routed (token, slot) pairs by expert (oracle).

Fig. 1 of ExactMoE groups tokens by selected expert before the expert kernels run.
Reading: flat index f = t*k + j; segment of expert e holds, in ascending f, every f with
ids.flat[f] == e (a stable grouping); offsets are the exclusive prefix sum of the
per-expert counts with offsets[E] = T*k, unpadded.
"""
from __future__ import annotations

import numpy as np


def group_tokens(ids: np.ndarray, E: int):
    """ids int32 [T, k] -> (offsets int32 [E+1], sorted_flat int32 [T*k], flat_to_sorted int32 [T*k])."""
    flat = np.asarray(ids, dtype=np.int64).reshape(-1)
    counts = np.bincount(flat, minlength=E)
    assert counts.shape[0] == E, "expert id out of range"
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(counts)
    sorted_flat = np.argsort(flat, kind="stable")
    flat_to_sorted = np.empty_like(sorted_flat)
    flat_to_sorted[sorted_flat] = np.arange(flat.size)
    return offsets.astype(np.int32), sorted_flat.astype(np.int32), flat_to_sorted.astype(np.int32)
