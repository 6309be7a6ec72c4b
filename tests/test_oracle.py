"""Pins of the CPU oracle against closed forms, exact arithmetic, brute force and the
figures of ExactMoE's Table 1 -- none of them re-types the oracle's own formula."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import layout as L
from oracle.quant import bf16_bits_to_f64, f64_to_bf16_bits, quantize_group128
from synthetic import SyntheticLayer, TINY, LayerShape, f32_to_bf16_bits, bf16_bits_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- bf16 rounding
def _frac_to_bf16_bits(v: Fraction) -> int:
    """Exact rational -> bf16 bits, round to nearest even, by integer arithmetic."""
    if v == 0:
        return 0
    sign = 0x8000 if v < 0 else 0
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    qe = max(e - 7, -133)
    m = a / Fraction(2) ** qe            # want round-half-even(m)
    fl = m.numerator // m.denominator
    rem = m - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    val = Fraction(fl) * Fraction(2) ** qe
    bits = int(np.array(float(val), dtype=np.float32).view(np.uint32)) >> 16
    return sign | bits


def test_f64_to_bf16_ties_and_no_double_rounding():
    one = 0x3F80
    assert f64_to_bf16_bits(np.array([1.0 + 2.0 ** -8]))[0] == one           # tie -> even
    assert f64_to_bf16_bits(np.array([1.0 + 3 * 2.0 ** -8]))[0] == one + 2   # tie -> even (up)
    # fp32 would round 1 + 2^-8 + 2^-30 to the exact tie and then to 1.0; one rounding gives 1 + 2^-7
    assert f64_to_bf16_bits(np.array([1.0 + 2.0 ** -8 + 2.0 ** -30]))[0] == one + 1
    assert f64_to_bf16_bits(np.array([-2.5]))[0] == 0xC020
    rng = np.random.default_rng(5)
    v = rng.standard_normal(2000) * 10.0 ** rng.integers(-6, 6, 2000)
    got = f64_to_bf16_bits(v)
    exp = [_frac_to_bf16_bits(Fraction(float(x))) for x in v]
    assert np.array_equal(got, np.array(exp, dtype=np.uint16))


# ---------------------------------------------------------------- quantization
def _weights(seed, n=48, k=512, sigma=0.02):
    rng = np.random.default_rng(seed)
    w = (rng.standard_normal((n, k)) * sigma).astype(np.float32)
    w[3, 128:256] *= 50.0            # a group with a large absmax
    w[5, 0:128] = 0.0                # an all-zero group
    w[7, 256:384] = 1e-30            # tiny constant group (bf16 subnormal-free scale range)
    return w


def test_quant_hand_worked_group():
    # absmax 0.7 -> fp32 0.7/7 = 0x3DCCCCCD -> bf16 0x3DCD = 0.10009765625
    w = np.zeros((1, 128), np.float32)
    w[0, :4] = [0.7, -0.35, 0.1, -0.05]
    q, s = quantize_group128(w)
    assert s[0, 0] == 0x3DCD
    assert list(q[0, :4]) == [7, -3, 1, 0]          # 6.993 -> 7; -3.4966 -> -3; 0.999 -> 1; -0.4995 -> -0
    assert not q[0, 4:].any()


def test_quant_roundtrip_bound_and_range():
    w = _weights(0)
    q, s = quantize_group128(w)
    sv = np.repeat(bf16_bits_to_f64(s), 128, axis=1)
    deq = q.astype(np.float64) * sv
    assert q.min() >= -7 and q.max() <= 7               # -8 is never needed with absmax/7
    assert np.all(np.abs(w.astype(np.float64) - deq) <= sv / 2)


def test_quant_matches_bruteforce_argmin():
    w = _weights(1, n=16, k=256)
    q, s = quantize_group128(w)
    sv = np.repeat(bf16_bits_to_f64(s), 128, axis=1)
    for n in range(w.shape[0]):
        for kk in range(w.shape[1]):
            sc = sv[n, kk]
            if sc == 0.0:
                assert q[n, kk] == 0
                continue
            best, bestd = None, None
            for cand in range(-8, 8):
                d = abs(float(w[n, kk]) - cand * sc)
                if bestd is None or d < bestd or (d == bestd and cand % 2 == 0):
                    best, bestd = cand, d
            assert q[n, kk] == best, (n, kk)


def test_quant_scale_is_bf16_of_absmax_over_7():
    w = _weights(2)
    q, s = quantize_group128(w)
    absmax = np.abs(w.astype(np.float64)).reshape(w.shape[0], -1, 128).max(axis=2)
    sv = bf16_bits_to_f64(s)
    # bf16 keeps 8 significant bits: relative error of one rounding <= 2^-8 (plus fp32's 2^-24)
    nz = absmax > 0
    assert np.all(np.abs(sv[nz] - absmax[nz] / 7) <= (2.0 ** -8 + 2.0 ** -23) * absmax[nz] / 7)
    assert np.all(sv[~nz] == 0)
    # the absmax element of each group gets code +-7
    g = np.abs(w).reshape(w.shape[0], -1, 128).argmax(axis=2)
    qq = q.reshape(w.shape[0], -1, 128)
    for n in range(w.shape[0]):
        for gi in range(g.shape[1]):
            if nz[n, gi]:
                assert abs(int(qq[n, gi, g[n, gi]])) == 7


def test_quant_idempotent_and_zero_group():
    w = _weights(3)
    q, s = quantize_group128(w)
    deq = (q.astype(np.float64) * np.repeat(bf16_bits_to_f64(s), 128, axis=1)).astype(np.float32)
    q2, s2 = quantize_group128(deq)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)
    assert s[5, 0] == 0 and not q[5, :128].any()


# ---------------------------------------------------------------- packed layout
def test_packed_size_formula():
    for H, I in [(256, 256), (2048, 1024), (4096, 14336), (128, 384)]:
        assert L.packed_expert_bytes(H, I) == 3 * H * I // 2 + 3 * H * I // 64
    assert L.packed_expert_bytes(2048, 1024) == 3_244_032
    assert L.packed_expert_bytes(256, 256) == 101_376
    assert L.packed_expert_bytes(4096, 14336) == 90_832_896


def test_packed_size_matches_table1_transfer_volume():
    """Table 1: H2D GiB per 128-token request / implied misses ~= one packed OLMoE expert.
    int4 without scales, or with fp32 scales, would be >= 3% off."""
    with open(os.path.join(GOLDEN, "table1_slot_cache.json")) as f:
        t1 = json.load(f)
    size = L.packed_expert_bytes(2048, 1024)
    for row in t1["rows"]:
        if row["hit_rate_pct"] is None:
            assert row["h2d_gib"] == 0.0          # fully resident: no transfers
            continue
        for steps in (127, 128):
            misses = (1 - row["hit_rate_pct"] / 100) * steps * 16 * 8
            per_miss = row["h2d_gib"] * 2 ** 30 / misses
            assert abs(per_miss / size - 1) < 0.012, (row, steps, per_miss)
    assert abs((3 * 2048 * 1024 // 2) / (30.04 * 2 ** 30 / ((1 - 0.388) * 127 * 128)) - 1) > 0.025


def test_pack_hand_worked_nibble():
    H = I = 128
    qg = np.zeros((I, H), np.int8); qu = np.zeros((I, H), np.int8); qd = np.zeros((H, I), np.int8)
    sg = np.zeros((I, 1), np.uint16); su = np.zeros((I, 1), np.uint16); sd = np.zeros((H, 1), np.uint16)
    qu[17, 45] = 7
    su[17, 0] = 0x1234
    blob = L.pack_expert(qg, sg, qu, su, qd, sd, H, I)
    # row 17 -> block 1, tile row 1; up -> tile 2*1+1 = 3; input 45 -> word 1, lane 16+1, j = 5
    # j = 5 sits at bits 16 + 4*2 = 24.  All other nibbles hold u = 8.
    off = 1024 * 3 + 16 * 17 + 4 * 1
    assert int.from_bytes(blob[off:off + 4], "little") == 0x8F888888
    assert blob[:off].count(b"\x88") == off and set(blob[off + 4:1024 * 24]) == {0x88}
    n_tiles = 24
    so = 1024 * n_tiles + 32 * 3 + 2 * 1
    assert int.from_bytes(blob[so:so + 2], "little") == 0x1234


def test_pack_fast_equals_loop_and_roundtrip():
    rng = np.random.default_rng(7)
    H, I = 256, 384
    qg = rng.integers(-8, 8, (I, H)).astype(np.int8); qu = rng.integers(-8, 8, (I, H)).astype(np.int8)
    qd = rng.integers(-8, 8, (H, I)).astype(np.int8)
    sg = rng.integers(0, 65535, (I, H // 128)).astype(np.uint16); su = rng.integers(0, 65535, (I, H // 128)).astype(np.uint16)
    sd = rng.integers(0, 65535, (H, I // 128)).astype(np.uint16)
    a = L.pack_expert(qg, sg, qu, su, qd, sd, H, I, fast=True)
    b = L.pack_expert(qg, sg, qu, su, qd, sd, H, I, fast=False)
    assert a == b and len(a) == L.packed_expert_bytes(H, I)
    out = L.unpack_expert(a, H, I)
    for x, y in zip(out, (qg, sg, qu, su, qd, sd)):
        assert np.array_equal(x, y)


def test_int4_layout_positions():
    """Packed int4 blob: random elements of every matrix, in both the gate/up and the down
    region and over several input groups, land at the tile, lane, word and nibble that
    the layout statement gives, and their row scales at the tile's scale slot. The
    positions are computed here from the statement alone (not from the packer's tile
    list), so a swapped loop order, a transposed operand or a wrong nibble shift fails."""
    H, I = 256, 384
    G, GD = H // 128, I // 128
    rng = np.random.default_rng(11)
    qg = rng.integers(-8, 8, (I, H)).astype(np.int8); qu = rng.integers(-8, 8, (I, H)).astype(np.int8)
    qd = rng.integers(-8, 8, (H, I)).astype(np.int8)
    # scales all distinct, so a scale read from the wrong slot cannot match
    sv = rng.permutation(2 * I * G + H * GD).astype(np.uint16) + 1
    sg = sv[:I * G].reshape(I, G); su = sv[I * G:2 * I * G].reshape(I, G); sd = sv[2 * I * G:].reshape(H, GD)
    blob = L.pack_expert(qg, sg, qu, su, qd, sd, H, I)
    nt = 2 * (I // 16) * G + (H // 16) * GD
    assert len(blob) == nt * (1024 + 32)
    mats = ((qg, sg, I, H), (qu, su, I, H), (qd, sd, H, I))
    hit = {0: set(), 1: set(), 2: set()}
    for _ in range(4000):
        which = int(rng.integers(0, 3))
        Q, S, R, K = mats[which]
        r, c = int(rng.integers(0, R)), int(rng.integers(0, K))
        b, g = r // 16, c // 128
        if which < 2:   # row block b: H/128 gate tiles, then H/128 up tiles
            t = b * 2 * G + which * G + g
        else:           # after every gate/up tile: row block b of down, I/128 tiles
            t = 2 * (I // 16) * G + b * GD + g
        lane = (r % 16) + 16 * ((c % 32) // 8)
        word, j = (c % 128) // 32, c % 8
        off = 1024 * t + 16 * lane + 4 * word
        w = int.from_bytes(blob[off:off + 4], "little")
        shift = 4 * (j // 2) if j % 2 == 0 else 16 + 4 * (j // 2)
        assert (w >> shift) & 0xF == int(Q[r, c]) + 8, (which, r, c)
        so = 1024 * nt + 32 * t + 2 * (r % 16)
        assert int.from_bytes(blob[so:so + 2], "little") == int(S[r, g]), (which, r, g)
        hit[which].add(g)
    assert hit[0] == hit[1] == set(range(G)) and hit[2] == set(range(GD))


# ---------------------------------------------------------------- router
def test_logits_equal_exact_rational_sum_tiny_layer():
    lay = SyntheticLayer(TINY, seed=0)
    x = lay.x(16)
    wr = lay.router()
    bias = np.linspace(-1, 1, TINY.E).astype(np.float32)
    got = oracle.router_logits(x, wr, bias)
    xf = bf16_bits_to_f32(x); wf = bf16_bits_to_f32(wr)
    for t in range(16):
        for e in range(TINY.E):
            acc = Fraction(float(bias[e]))
            for h in range(TINY.H):
                acc += Fraction(float(xf[t, h])) * Fraction(float(wf[e, h]))
            assert got[t, e] == _frac_to_bf16_bits(acc), (t, e)


def test_topk_equals_full_stable_sort_bruteforce():
    rng = np.random.default_rng(3)
    logits = f32_to_bf16_bits(rng.standard_normal((200, 64)).astype(np.float32) * 0.9)
    logits[:, 10] = logits[:, 3]          # forced ties
    logits[0, :] = 0x8000                 # all -0
    logits[0, 5] = 0x0000                 # one +0: ties with -0
    for k in (1, 2, 8, 64):
        ids = oracle.topk_ids(logits, k)
        lf = bf16_bits_to_f32(logits)
        for t in range(logits.shape[0]):
            order = sorted(range(64), key=lambda e: (-float(lf[t, e]), e))
            assert list(ids[t]) == order[:k]
            assert len(set(ids[t])) == k
    assert list(oracle.topk_ids(logits, 3)[0]) == [0, 1, 2]


def test_weights_closed_forms():
    rng = np.random.default_rng(4)
    logits = f32_to_bf16_bits(rng.standard_normal((50, 16)).astype(np.float32))
    lf = bf16_bits_to_f32(logits).astype(np.float64)
    full = scipy.special.softmax(lf, axis=1)
    for k in (1, 4, 16):
        ids = oracle.topk_ids(logits, k)
        w = oracle.topk_weights(logits, ids, renormalize=True).astype(np.float64)
        p = np.take_along_axis(full, ids.astype(np.int64), axis=1)
        assert np.allclose(w, p / p.sum(axis=1, keepdims=True), rtol=1e-6, atol=1e-7)
        assert np.allclose(w.sum(axis=1), 1.0, atol=1e-6)
        wr = oracle.topk_weights(logits, ids, renormalize=False).astype(np.float64)
        assert np.allclose(wr, p, rtol=1e-6, atol=1e-8)
    ids = oracle.topk_ids(logits, 16)
    w = oracle.topk_weights(logits, ids)
    assert np.allclose(np.take_along_axis(full, ids.astype(np.int64), axis=1), w, rtol=1e-6)
    assert np.all(np.diff(w, axis=1) <= 0)     # slots ordered by logit


# ---------------------------------------------------------------- grouping
def test_group_is_stable_bucket_permutation():
    rng = np.random.default_rng(8)
    E, T, k = 16, 37, 3
    ids = np.stack([rng.choice(np.arange(1, E, 2), k, replace=False) for _ in range(T)]).astype(np.int32)
    off, sf, fs = oracle.group_tokens(ids, E)
    buckets = [[] for _ in range(E)]
    for f, e in enumerate(ids.reshape(-1)):
        buckets[e].append(f)
    assert off[0] == 0 and off[-1] == T * k
    for e in range(E):
        assert list(sf[off[e]:off[e + 1]]) == buckets[e]
        if e % 2 == 0:
            assert off[e] == off[e + 1]          # never-selected experts get empty segments
    assert sorted(sf) == list(range(T * k))
    assert np.array_equal(sf[fs], np.arange(T * k)) and np.array_equal(fs[sf], np.arange(T * k))


# ---------------------------------------------------------------- expert MLP + combine
def _tiny_layer(H=128, I=128, E=3, T=3, k=2, seed=11):
    shape = LayerShape(H=H, I=I, E=E, k=k)
    lay = SyntheticLayer(shape, seed=seed)
    experts = [oracle.quantize_expert(*lay.expert(e)) for e in range(E)]
    x = lay.x(T)
    wr = lay.router()
    return shape, lay, experts, x, wr


def test_mlp_bruteforce_python_loops():
    shape, lay, experts, x, wr = _tiny_layer()
    res = oracle.moe_layer(x, wr, experts, shape.k)
    xf = bf16_bits_to_f32(x)
    for t in range(x.shape[0]):
        y = [0.0] * shape.H
        for j in range(shape.k):
            e = int(res["ids"][t, j])
            qe = experts[e]
            sg = bf16_bits_to_f32(qe.sg); su = bf16_bits_to_f32(qe.su); sd = bf16_bits_to_f32(qe.sd)
            a = []
            for n in range(shape.I):
                gn = sum(float(xf[t, kk]) * int(qe.qg[n, kk]) * float(sg[n, kk // 128]) for kk in range(shape.H))
                un = sum(float(xf[t, kk]) * int(qe.qu[n, kk]) * float(su[n, kk // 128]) for kk in range(shape.H))
                a.append(gn / (1 + math.exp(-gn)) * un)
            wj = float(res["weights"][t, j])
            for m in range(shape.H):
                om = sum(a[n] * int(qe.qd[m, n]) * float(sd[m, n // 128]) for n in range(shape.I))
                y[m] += wj * om
        assert np.allclose(res["y"][t], y, rtol=1e-9, atol=1e-12)


def test_grouped_equals_per_token():
    shape, lay, experts, x, wr = _tiny_layer(H=256, I=256, E=8, T=16, k=2, seed=0)
    res = oracle.moe_layer(x, wr, experts, shape.k)
    xf = bf16_bits_to_f64(x)
    yg = oracle.forward_grouped(xf, res["ids"], res["weights"], experts, res["offsets"], res["sorted_flat"], rowwise=True)
    assert np.array_equal(yg, res["y"])                  # identical per-row arithmetic: bit-exact
    yb = oracle.forward_grouped(xf, res["ids"], res["weights"], experts, res["offsets"], res["sorted_flat"])
    assert np.allclose(yb, res["y"], rtol=1e-12, atol=1e-15)


def test_mlp_special_cases():
    shape, lay, experts, x, wr = _tiny_layer(E=4, T=5, k=2)
    res = oracle.moe_layer(x, wr, experts, shape.k)
    # x = 0 -> y = 0
    z = oracle.moe_layer(np.zeros_like(x), wr, experts, shape.k)
    assert not np.any(z["y"])
    # W_down = 0 -> y = 0
    import copy
    ex0 = [copy.copy(e) for e in experts]
    for e in ex0:
        e.qd = np.zeros_like(e.qd); e._deq = {}
    assert not np.any(oracle.moe_layer(x, wr, ex0, shape.k)["y"])
    # doubling every down scale (exact in bf16) doubles y exactly
    ex2 = [copy.copy(e) for e in experts]
    for e in ex2:
        e.sd = (e.sd.astype(np.uint32) + (1 << 7)).astype(np.uint16); e._deq = {}    # exponent + 1
    assert np.array_equal(oracle.moe_layer(x, wr, ex2, shape.k)["y"], 2 * res["y"])
    # relabelling experts consistently (router rows and expert list) leaves y unchanged
    perm = np.array([2, 0, 3, 1])
    exp_perm = [experts[perm[i]] for i in range(4)]
    wr_perm = wr[perm]
    r2 = oracle.moe_layer(x, wr_perm, exp_perm, shape.k)
    assert np.allclose(r2["y"], res["y"], rtol=1e-14, atol=1e-16)
    # k = 1 with weight 1: y equals the single routed expert's MLP
    r1 = oracle.moe_layer(x, wr, experts, 1)
    assert np.allclose(r1["weights"], 1.0)
    for t in range(x.shape[0]):
        o = oracle.expert_mlp(experts[int(r1["ids"][t, 0])], bf16_bits_to_f64(x[t:t + 1]))[0]
        assert np.array_equal(r1["y"][t], o)


def test_knockout_every_routed_expert_runs():
    shape, lay, experts, x, wr = _tiny_layer(E=4, T=12, k=2, seed=5)
    res = oracle.moe_layer(x, wr, experts, shape.k)
    other = SyntheticLayer(shape, seed=99)
    for e in range(4):
        ex = list(experts)
        ex[e] = oracle.quantize_expert(*other.expert(e))
        y2 = oracle.moe_layer(x, wr, ex, shape.k)["y"]
        changed = np.nonzero(np.any(y2 != res["y"], axis=1))[0]
        assert np.array_equal(changed, oracle.knockout_rows(res["ids"], e))


# ---------------------------------------------------------------- LRU slot cache
def _lru_reference(trace, E, S, nbytes):
    """Independent formulation: a recency list per layer, free slots taken lowest first."""
    layers = trace.shape[1]
    rec = [[] for _ in range(layers)]       # least recent first
    slots = [dict() for _ in range(layers)]
    c = dict(lookups=0, hits=0, misses=0, evictions=0, bytes=0)
    for step in trace:
        for l in range(layers):
            A = sorted(set(int(e) for e in step[l]))
            for e in A:
                c["lookups"] += 1
                if e in rec[l]:
                    c["hits"] += 1
                    rec[l].remove(e)
                else:
                    c["misses"] += 1; c["bytes"] += nbytes
                    used = set(slots[l].values())
                    if len(rec[l]) < S:
                        slots[l][e] = min(set(range(S)) - used)
                    else:
                        victim = next(x for x in rec[l] if x not in A)
                        rec[l].remove(victim)
                        slots[l][e] = slots[l].pop(victim)
                        c["evictions"] += 1
                rec[l].append(e)
    return c, slots


def test_lru_matches_independent_reference():
    from synthetic import slot_cache_trace
    for S in (1, 2, 3, 5, 8):
        k = min(S, 3)
        trace = slot_cache_trace(E=8, k=k, layers=2, steps=60, seed=S)
        sim = oracle.LRUSlotCacheSim(layers=2, E=8, slots=S, expert_bytes=10) if S < 8 else None
        if sim is None:
            continue
        for step in trace:
            for l in range(2):
                table = sim.acquire(l, step[l])
        ref, slots = _lru_reference(trace, 8, S, 10)
        assert (sim.lookups, sim.hits, sim.misses, sim.evictions, sim.h2d_bytes) == \
            (ref["lookups"], ref["hits"], ref["misses"], ref["evictions"], ref["bytes"])
        for l in range(2):
            assert sim.slot_of[l] == slots[l]


def test_lru_closed_forms():
    # enough slots: only compulsory misses
    tr = np.array([[[0, 1]], [[1, 2]], [[0, 2]], [[3, 1]]], dtype=np.int32)
    sim = oracle.LRUSlotCacheSim(layers=1, E=6, slots=4, expert_bytes=7)
    for st in tr:
        sim.acquire(0, st[0])
    assert sim.misses == 4 and sim.evictions == 0 and sim.h2d_bytes == 28 and sim.lookups == 8
    # one slot, k = 1: a miss on every change of expert
    seq = [0, 0, 1, 1, 1, 0, 2, 2, 0]
    sim = oracle.LRUSlotCacheSim(layers=1, E=3, slots=1, expert_bytes=1)
    for e in seq:
        sim.acquire(0, [e])
    assert sim.misses == 1 + sum(a != b for a, b in zip(seq, seq[1:]))
    # resident: counters bypassed
    sim = oracle.LRUSlotCacheSim(layers=1, E=3, slots=3, expert_bytes=1)
    assert list(sim.acquire(0, [2, 0])) == [0, 1, 2] and sim.lookups == 0
    with pytest.raises(ValueError):
        oracle.LRUSlotCacheSim(layers=1, E=4, slots=2, expert_bytes=1).acquire(0, [0, 1, 2])


def test_lru_waves_closed_forms_and_reference():
    """Cache-sized waves (Fig. 1 caption): resident active experts first, then the others,
    each in ascending id; one wave when the set fits, else waves of S // 2; each wave is
    one layer-step of the policy."""
    S, n = 4, 6
    sim = oracle.LRUSlotCacheSim(layers=1, E=12, slots=S, expert_bytes=3)
    waves = sim.acquire_waves(0, [5, 3, 1, 0, 2, 4, 3])         # duplicates and order ignored
    assert [w for w, _ in waves] == [[0, 1], [2, 3], [4, 5]]     # cold cache: plain ascending
    assert (sim.misses, sim.hits, sim.evictions, sim.h2d_bytes) == (n, 0, n - S, 3 * n)
    # every expert of a wave is resident right after its acquire
    for w, table in waves:
        assert all(table[e] >= 0 for e in w)
    # the last wave evicted the oldest (0, 1), so {2, 3, 4, 5} stay; the same forward again
    # takes them first (S hits) and then misses the other n - S
    sim.reset_stats()
    waves = sim.acquire_waves(0, range(n))
    assert [w for w, _ in waves] == [[2, 3], [4, 5], [0, 1]]
    assert (sim.misses, sim.hits, sim.evictions) == (n - S, S, n - S)
    # any repeated active set larger than the cache: exactly S hits per forward
    for rep in range(3):
        sim.reset_stats()
        sim.acquire_waves(0, range(n))
        assert (sim.hits, sim.misses) == (S, n - S)
    # a set that fits is one wave; S == 1 takes waves of one
    assert [w for w, _ in oracle.LRUSlotCacheSim(1, 12, 4, 1).acquire_waves(0, [7, 2, 9, 4])] == [[2, 4, 7, 9]]
    assert [w for w, _ in oracle.LRUSlotCacheSim(1, 12, 1, 1).acquire_waves(0, [7, 2])] == [[2], [7]]
    # no wave's misses evict an expert of the wave before it (its copies may overlap that
    # wave's kernels), over random active sets, slot counts and histories
    rng = np.random.default_rng(3)
    for S2 in (2, 3, 4, 5, 8):
        sim = oracle.LRUSlotCacheSim(layers=1, E=16, slots=S2, expert_bytes=1)
        for _ in range(40):
            A = rng.choice(16, size=int(rng.integers(1, 17)), replace=False)
            before = None
            waves = sim.acquire_waves(0, A)
            for w, table in waves:
                if before is not None and len(waves) > 1:
                    prev_w, prev_t = before
                    assert all(table[e] == prev_t[e] for e in prev_w), (S2, sorted(A))
                before = (w, table)
    # the waves as layer-steps of the independent reference, the wave split recomputed from
    # that reference's own residency before each forward
    forwards = ([3, 9, 1, 7, 11, 0], [2, 3, 4], list(range(12)), [11, 10], [0, 1, 2, 3, 4, 11], list(range(12)))
    trace = []

    def padded(ws):
        width = max(len(w) for w in ws)
        arr = np.full((len(ws), 1, width), -1, dtype=np.int64)
        for i, w in enumerate(ws):
            arr[i, 0, :len(w)] = w
            arr[i, 0, len(w):] = w[0]                            # padding repeats an id (deduplicated)
        return arr

    for active in forwards:
        A = sorted(set(active))
        res = set(_lru_reference(padded(trace), 12, S, 5)[1][0]) if trace else set()
        order = [e for e in A if e in res] + [e for e in A if e not in res]
        W = S if len(A) <= S else S // 2
        trace += [order[i:i + W] for i in range(0, len(order), W)]
    sim = oracle.LRUSlotCacheSim(layers=1, E=12, slots=S, expert_bytes=5)
    got = []
    for active in forwards:
        got += [w for w, _ in sim.acquire_waves(0, active)]
    assert got == trace
    ref, slots = _lru_reference(padded(trace), 12, S, 5)
    assert (sim.lookups, sim.hits, sim.misses, sim.evictions, sim.h2d_bytes) == \
        (ref["lookups"], ref["hits"], ref["misses"], ref["evictions"], ref["bytes"])
    assert sim.slot_of[0] == slots[0]


# ---------------------------------------------------------------------------- bf16 comparator
def test_bf16_layout_positions():
    """Dense bf16 blob: every element lands where the layout statement puts it (tile order
    gate/up per row block, then down; lane l holds row l % 16, inputs 8 (l // 16) + j)."""
    H, I = 128, 96 + 32
    vals = np.random.default_rng(0).permutation(3 * H * I).astype(np.uint16)   # all distinct
    g = vals[:I * H].reshape(I, H)
    u = vals[I * H:2 * I * H].reshape(I, H)
    d = vals[2 * I * H:].reshape(H, I)
    blob = np.frombuffer(oracle.pack_expert_bf16(g, u, d), dtype="<u2")
    CH, CI = H // 32, I // 32
    rng = np.random.default_rng(1)
    for _ in range(3000):
        which = int(rng.integers(0, 3))
        W, R, K = ((g, I, H), (u, I, H), (d, H, I))[which]
        r, c = int(rng.integers(0, R)), int(rng.integers(0, K))
        b, cc = r // 16, c // 32
        if which < 2:
            t = b * 2 * CH + which * CH + cc
        else:
            t = 2 * (I // 16) * CH + b * CI + cc
        lane = (r % 16) + 16 * ((c % 32) // 8)
        assert blob[512 * t + 8 * lane + c % 8] == W[r, c]


def test_dense_expert_equals_quant_expert_on_exact_weights():
    """Weights q * 2^-6 with every (row, group) reaching |q| = 7 are exact in bf16 and are
    quantized back to the same codes and scales, so the bf16 expert and the int4 expert
    have identical weights and identical outputs."""
    H, I = 256, 128
    rng = np.random.default_rng(5)

    def exact(R, K):
        q = rng.integers(-7, 8, size=(R, K)).astype(np.float32)
        for gi in range(K // 128):
            cols = rng.integers(0, 128, size=R) + 128 * gi
            q[np.arange(R), cols] = rng.choice([-7.0, 7.0], size=R)
        return q * np.float32(2.0 ** -6)

    wg, wu, wd = exact(I, H), exact(I, H), exact(H, I)
    bits = [(w.view(np.uint32) >> 16).astype(np.uint16) for w in (wg, wu, wd)]
    assert all(np.array_equal(oracle.bf16_bits_to_f64(b), w.astype(np.float64)) for b, w in zip(bits, (wg, wu, wd)))
    de = oracle.DenseExpert(*bits)
    qe = oracle.quantize_expert(wg, wu, wd)
    for a, b in zip(de.deq(), qe.deq()):
        assert np.array_equal(a, b)
    x = rng.standard_normal((3, H))
    assert np.array_equal(oracle.expert_mlp(de, x), oracle.expert_mlp(qe, x))
    # and a transposed or misread matrix would not pass: the bits are the weights
    assert not np.array_equal(oracle.DenseExpert(bits[1], bits[0], bits[2]).deq()[0], de.deq()[0])

