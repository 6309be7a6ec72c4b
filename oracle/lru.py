"""Slot-cache residency simulator (oracle).

ExactMoE keeps every packed expert in pinned host memory and serves the selected
experts from a configurable GPU slot cache; larger caches cut transfers (abstract;
Fig. 1 and Fig. 2 captions; Tab. 1 reports hit rate and H2D bytes). The pages do not
state the eviction policy. Reading (least-recently-used, per layer):
  * each layer-step looks up its distinct active experts in ascending id order;
  * a lookup stamps the expert with a global counter; a hit is an expert already resident;
  * a miss copies one packed expert (bytes += expert_bytes) into the lowest free slot,
    else evicts the resident expert with the smallest stamp that is not in the current
    active set;
  * more active experts than slots is an error for one lookup; a forward splits them into
    cache-sized waves (Fig. 1 caption: active experts run in waves that fit the cache).
    Reading (the order of the waves is not on the pages): the distinct active experts that
    are already resident come first, in ascending id, then the others in ascending id; an
    active set that fits is one wave, a larger one is cut into consecutive waves of
    slots // 2 (of 1 when slots == 1), and each wave is one layer-step of the policy above
    (acquire_waves). Taking the resident experts first means a repeated active set larger
    than the cache hits `slots` times instead of thrashing the LRU; half-size waves mean the
    misses of a wave never evict an expert of the wave before it, so its copies can run
    while that wave computes (Fig. 1: waves that fit the cache; the overlap is this
    reading's, not the pages');
  * slots == experts is full residency: everything is preloaded, lookups are bypassed and
    the counters stay at zero (Fig. 2 caption: accounting bypassed when resident).
"""
from __future__ import annotations

import numpy as np


class LRUSlotCacheSim:
    def __init__(self, layers: int, E: int, slots: int, expert_bytes: int):
        assert 1 <= slots <= E
        self.layers, self.E, self.S, self.expert_bytes = layers, E, slots, expert_bytes
        self.resident = slots == E
        self.slot_of = [dict() for _ in range(layers)]       # expert -> slot
        self.owner = [[-1] * slots for _ in range(layers)]   # slot -> expert
        self.stamp = [dict() for _ in range(layers)]
        self.clock = 0
        self.reset_stats()
        if self.resident:
            for l in range(layers):
                for e in range(E):
                    self.slot_of[l][e] = e
                    self.owner[l][e] = e

    def reset_stats(self):
        self.lookups = self.hits = self.misses = self.evictions = 0
        self.h2d_bytes = 0

    def acquire(self, layer: int, active) -> np.ndarray:
        """active: iterable of expert ids. Returns expert->slot int32 [E] (-1 = absent)."""
        A = sorted(set(int(e) for e in active))
        if len(A) > self.S:
            raise ValueError("more active experts than slots")
        if not self.resident:
            slot_of, owner, stamp = self.slot_of[layer], self.owner[layer], self.stamp[layer]
            Aset = set(A)
            for e in A:
                self.lookups += 1
                self.clock += 1
                if e in slot_of:
                    self.hits += 1
                else:
                    self.misses += 1
                    self.h2d_bytes += self.expert_bytes
                    free = [s for s in range(self.S) if owner[s] < 0]
                    if free:
                        s = free[0]
                    else:
                        victim = min((x for x in slot_of if x not in Aset), key=lambda x: stamp[x])
                        s = slot_of.pop(victim)
                        del stamp[victim]
                        self.evictions += 1
                    slot_of[e] = s
                    owner[s] = e
                stamp[e] = self.clock
        table = np.full(self.E, -1, dtype=np.int32)
        for e, s in self.slot_of[layer].items():
            table[e] = s
        return table

    def acquire_waves(self, layer: int, active):
        """The waves of one cached forward: [(wave expert ids, table after its acquire)]."""
        A = sorted(set(int(e) for e in active))
        resident = self.slot_of[layer]
        A = [e for e in A if e in resident] + [e for e in A if e not in resident]
        W = self.S // 2 if len(A) > self.S and self.S >= 2 else self.S
        out = []
        for w0 in range(0, len(A), W):
            wave = A[w0:w0 + W]
            out.append((wave, self.acquire(layer, wave)))
        return out

