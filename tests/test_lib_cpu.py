"""Host-side checks of libexmoe that need no GPU: exported symbols, the offline packer
against the oracle's independent packer, argument validation, and the slot-cache policy
(dry-run mode) against the oracle's LRU simulator."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle
from oracle import layout as OL
from synthetic import SyntheticLayer, TINY, OLMOE, LayerShape, slot_cache_trace, batch_trace

exm = pytest.importorskip("w4a16_mixture_experts_amd")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_exports_every_declared_symbol():
    hdr = open(os.path.join(ROOT, "include", "exmoe.h")).read()
    declared = set(re.findall(r"\b(exmoe_[a-z0-9_]+)\s*\(", hdr))
    assert declared, "no declarations parsed"
    lib = ctypes.CDLL(exm.LIB_PATH)
    for name in sorted(declared):
        assert hasattr(lib, name), name
    assert declared == set(exm.EXPORTED)
    assert exm.abi_version() == 1


@pytest.mark.parametrize("H,I,seed", [(256, 256, 0), (128, 384, 1), (384, 128, 2)])
def test_packer_bit_exact_vs_oracle(H, I, seed):
    lay = SyntheticLayer(LayerShape(H=H, I=I, E=2, k=1), seed=seed)
    for e in range(2):
        g, u, d = lay.expert(e)
        if e == 1:
            g[3, :128] = 0.0          # all-zero group
            u[5, 7] = 1.0             # large outlier
        blob = exm.quantize_pack(g, u, d)
        qe = oracle.quantize_expert(g, u, d)
        ref = OL.pack_expert(qe.qg, qe.sg, qe.qu, qe.su, qe.qd, qe.sd, H, I)
        assert blob.tobytes() == ref
        out = exm.unpack_expert(blob, H, I)
        for a, b in zip(out, (qe.qg, qe.sg, qe.qu, qe.su, qe.qd, qe.sd)):
            assert np.array_equal(a, b)


def test_packer_bit_exact_olmoe_expert():
    lay = SyntheticLayer(OLMOE, seed=0)
    g, u, d = lay.expert(5)
    blob = exm.quantize_pack(g, u, d)
    assert blob.nbytes == 3_244_032 == exm.packed_expert_bytes(2048, 1024)
    qe = oracle.quantize_expert(g, u, d)
    assert blob.tobytes() == OL.pack_expert(qe.qg, qe.sg, qe.qu, qe.su, qe.qd, qe.sd, 2048, 1024)


@pytest.mark.parametrize("H,I,seed", [(256, 128, 0), (128, 384, 1)])
def test_bf16_packer_bit_exact_vs_oracle(H, I, seed):
    rng = np.random.default_rng(seed)
    g = rng.integers(0, 1 << 16, size=(I, H), dtype=np.uint16)
    u = rng.integers(0, 1 << 16, size=(I, H), dtype=np.uint16)
    d = rng.integers(0, 1 << 16, size=(H, I), dtype=np.uint16)
    blob = exm.bf16_pack(g, u, d)
    assert blob.nbytes == exm.bf16_expert_bytes(H, I) == OL.bf16_expert_bytes(H, I) == 6 * H * I
    assert blob.tobytes() == OL.pack_expert_bf16(g, u, d)


def test_bf16_pack_rejects_bad_input():
    g = np.zeros((128, 128), np.uint16)
    lib = exm._lib
    buf = np.zeros(exm.bf16_expert_bytes(128, 128), np.uint8)
    assert lib.exmoe_bf16_pack(g.ctypes.data, g.ctypes.data, g.ctypes.data, 128, 128, buf.ctypes.data, buf.nbytes - 1) == exm.ERR_INVALID_ARGUMENT
    assert lib.exmoe_bf16_pack(g.ctypes.data, g.ctypes.data, g.ctypes.data, 96, 128, buf.ctypes.data, buf.nbytes) == exm.ERR_INVALID_ARGUMENT
    assert lib.exmoe_bf16_pack(None, g.ctypes.data, g.ctypes.data, 128, 128, buf.ctypes.data, buf.nbytes) == exm.ERR_INVALID_ARGUMENT
    assert exm.bf16_expert_bytes(100, 128) == 0


def test_packer_rejects_bad_input():
    g = np.zeros((128, 128), np.float32)
    with pytest.raises(exm.ExmoeError) as ei:
        exm.quantize_pack(g, g, np.full((128, 128), np.nan, np.float32))
    assert ei.value.status == exm.ERR_INVALID_ARGUMENT and "finite" in str(ei.value)
    lib = exm._lib
    buf = np.zeros(exm.packed_expert_bytes(128, 128), np.uint8)
    assert lib.exmoe_quantize_pack(g.ctypes.data, g.ctypes.data, g.ctypes.data, 128, 128, 64, buf.ctypes.data, buf.nbytes) == exm.ERR_UNSUPPORTED
    assert lib.exmoe_quantize_pack(g.ctypes.data, g.ctypes.data, g.ctypes.data, 128, 128, 128, buf.ctypes.data, buf.nbytes - 1) == exm.ERR_INVALID_ARGUMENT
    assert lib.exmoe_quantize_pack(g.ctypes.data, g.ctypes.data, g.ctypes.data, 100, 128, 128, buf.ctypes.data, buf.nbytes) == exm.ERR_INVALID_ARGUMENT
    assert exm.packed_expert_bytes(100, 128) == 0


FAKE = 0x10000   # aligned, never dereferenced: validation fails before any enqueue


def _bank(stride=None, base=FAKE):
    return exm.ExpertBankC(base, exm.packed_expert_bytes(256, 256) if stride is None else stride, None)


def _fwd(T=4, H=256, I=256, E=8, k=2, flags=0, ws=1 << 30, bank=None, x=FAKE, y=FAKE, ws_ptr=FAKE):
    b = bank or _bank()
    return exm._lib.exmoe_moe_forward(x, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.byref(b), T, H, I, E, k, flags, y,
                                      ws_ptr, ws, None)


def test_forward_validation_errors():
    E_INV, E_WS, E_UNS = exm.ERR_INVALID_ARGUMENT, exm.ERR_WORKSPACE, exm.ERR_UNSUPPORTED
    assert _fwd(H=200) == E_INV
    assert _fwd(I=100) == E_INV
    assert _fwd(k=9) == E_INV
    assert _fwd(E=0) == E_INV
    assert _fwd(E=300, k=2) == E_INV
    assert _fwd(T=-1) == E_INV
    assert _fwd(x=None) == E_INV and "x" in exm.last_error()
    assert _fwd(x=FAKE + 2) == E_INV and "aligned" in exm.last_error()
    assert _fwd(flags=7) == E_INV
    assert _fwd(flags=1 << 10) == E_INV      # 0x100 and 0x200 are flags; 0x400 is not
    assert _fwd(bank=_bank(stride=100)) == E_INV
    assert _fwd(bank=_bank(base=None)) == E_INV
    need = exm.moe_workspace_bytes(4, 256, 256, 8, 2)
    assert need > 0
    assert _fwd(ws=need - 1) == E_WS and str(need) in exm.last_error()
    assert _fwd(ws_ptr=None) == E_WS
    assert _fwd(T=0) == exm.OK            # no-op, nothing touched
    assert _fwd(E=128, k=65) == E_UNS


def test_route_and_group_validation_errors():
    lib = exm._lib
    assert lib.exmoe_route_topk(FAKE, FAKE, None, 4, 100, 8, 2, 1, FAKE, FAKE, FAKE, None) == exm.ERR_INVALID_ARGUMENT
    assert lib.exmoe_route_topk(FAKE, FAKE, None, 4, 256, 8, 9, 1, FAKE, FAKE, FAKE, None) == exm.ERR_INVALID_ARGUMENT
    assert lib.exmoe_route_topk(None, FAKE, None, 4, 256, 8, 2, 1, FAKE, FAKE, FAKE, None) == exm.ERR_INVALID_ARGUMENT
    assert lib.exmoe_route_topk(FAKE, FAKE, None, 0, 256, 8, 2, 1, None, None, None, None) == exm.OK
    assert lib.exmoe_group_tokens(FAKE, 4, 2, 8, None, FAKE, FAKE, None, 0, None) == exm.ERR_INVALID_ARGUMENT
    assert lib.exmoe_group_tokens(FAKE, 4, 2, 8, FAKE + 1, FAKE, FAKE, None, 0, None) == exm.ERR_INVALID_ARGUMENT
    assert lib.exmoe_topk_from_logits(FAKE, 4, 8, 0, 1, FAKE, FAKE, None) == exm.ERR_INVALID_ARGUMENT
    assert lib.exmoe_active_experts(FAKE, 0, FAKE, FAKE, None) == exm.ERR_INVALID_ARGUMENT
    assert exm.last_error() != ""


def test_last_error_is_thread_local():
    import threading
    assert _fwd(H=200) == exm.ERR_INVALID_ARGUMENT
    main_msg = exm.last_error()
    seen = {}

    def worker():
        seen["before"] = exm.last_error()
        _fwd(k=9)
        seen["after"] = exm.last_error()

    th = threading.Thread(target=worker)
    th.start(); th.join()
    assert seen["before"] == "" and "k must be" in seen["after"]
    assert exm.last_error() == main_msg


@pytest.mark.parametrize("S", [1, 2, 5, 8, 16, 32])
def test_slot_cache_policy_matches_oracle(S):
    E, layers, k = 64, 3, min(S, 8)
    trace = slot_cache_trace(E=E, k=k, layers=layers, steps=64, seed=S)
    c = exm.SlotCache(layers, E, S, expert_bytes=3_244_032, dry_run=True)
    sim = oracle.LRUSlotCacheSim(layers, E, S, 3_244_032)
    for step in trace:
        for l in range(layers):
            c.acquire(l, list(step[l]))
            table = sim.acquire(l, step[l])
            assert np.array_equal(c.table(l), table)
    st = c.stats()
    assert (st["lookups"], st["hits"], st["misses"], st["evictions"], st["h2d_bytes"]) == \
        (sim.lookups, sim.hits, sim.misses, sim.evictions, sim.h2d_bytes)
    assert st["h2d_copies"] == sim.misses and st["resident"] == 0
    c.reset_stats()
    assert c.stats()["lookups"] == 0
    c.close()


def _same_stats(c, sim):
    st = c.stats()
    assert (st["lookups"], st["hits"], st["misses"], st["evictions"], st["h2d_bytes"]) == \
        (sim.lookups, sim.hits, sim.misses, sim.evictions, sim.h2d_bytes)
    return st


@pytest.mark.parametrize("S", [8, 16, 32, 64])
def test_slot_cache_benchmark_trace_matches_oracle(S):
    """The slot-cache decode workload as timed: 16 OLMoE-shaped layers, one 256-step trace
    (seed 0), the first 128 steps warm the cache, counters reset, the next 128 are the
    reported ones. The library's policy (dry run, the same host code as the cached forward,
    one wave per layer-step since 8 experts fit every S) and the oracle's simulator agree
    on every counter at both points, and the reported hit rates are those counters."""
    E, k, layers, steps = 64, 8, 16, 128
    nb = 3_244_032
    trace = slot_cache_trace(E, k, layers, 2 * steps, seed=0)
    c = exm.SlotCache(layers, E, S, nb, dry_run=True)
    sim = oracle.LRUSlotCacheSim(layers, E, S, nb)
    rates = []
    for half in range(2):
        for st in range(half * steps, (half + 1) * steps):
            for l in range(layers):
                active = sorted(set(int(e) for e in trace[st, l]))
                waves = c.waves(l, active, run=True)
                ref = sim.acquire_waves(l, active)
                assert waves == [w for w, _ in ref]
                assert np.array_equal(c.table(l), ref[-1][1])
        got = _same_stats(c, sim)
        rates.append(got["hits"] / max(got["lookups"], 1))
        c.reset_stats(); sim.reset_stats()
    if S == E:
        assert got["resident"] == 1 and got["lookups"] == 0
    else:
        # every layer-step looks up its 8 distinct experts
        assert got["lookups"] == steps * layers * k
    print(f"S={S}: cold hit rate {rates[0]:.4f}, warm {rates[1]:.4f}")
    c.close()


def test_batched_trace_waves_match_oracle():
    """Batched decode through 16 slots per layer as timed: batch 1, 2, 4, 8 in turn on one
    cache, each 64 warm-up steps then 64 counted ones (counters reset in between), the
    batch's distinct experts per layer in cache-sized waves. The library's wave plan and
    policy (dry run) equal the oracle's wave simulation at every layer-step, and the
    counters agree at every reset."""
    E, k, layers, steps, S = 64, 8, 16, 64, 16
    nb = 3_244_032
    trace = batch_trace(E, k, layers, 2 * steps, 8, seed=0)
    c = exm.SlotCache(layers, E, S, nb, dry_run=True)
    sim = oracle.LRUSlotCacheSim(layers, E, S, nb)
    multi = 0
    for B in (1, 2, 4, 8):
        for half in range(2):
            for st in range(half * steps, (half + 1) * steps):
                for l in range(layers):
                    active = np.unique(trace[st, l, :B]).tolist()
                    waves = c.waves(l, active, run=True)
                    ref = sim.acquire_waves(l, active)
                    assert waves == [w for w, _ in ref], (B, st, l)
                    multi += len(waves) > 1
            _same_stats(c, sim)
            c.reset_stats(); sim.reset_stats()
    assert multi > 0          # batch 2 and above route some layer-steps past 16 experts
    c.close()


def test_slot_cache_waves_plan_only():
    c = exm.SlotCache(1, 8, 4, 100, dry_run=True)
    assert c.waves(0, [5, 1, 1, 7, 3, 2]) == [[1, 2], [3, 5], [7]]     # 5 > 4: waves of 2
    assert c.stats()["lookups"] == 0                                     # plan only
    c.acquire(0, [5, 7])
    assert c.waves(0, [1, 5, 7]) == [[5, 7, 1]]                          # fits: residents first
    assert c.waves(0, [1, 2, 3, 5, 7]) == [[5, 7], [1, 2], [3]]
    with pytest.raises(exm.ExmoeError) as ei:
        c.waves(1, [0])
    assert ei.value.status == exm.ERR_CACHE
    with pytest.raises(exm.ExmoeError):
        c.waves(0, [8])
    assert c.waves(0, []) == []
    c.close()


def test_slot_cache_errors_and_resident():
    with pytest.raises(exm.ExmoeError):
        exm.SlotCache(1, 8, 9, 100, dry_run=True)
    c = exm.SlotCache(2, 8, 4, 100, dry_run=True)
    with pytest.raises(exm.ExmoeError) as ei:
        c.acquire(0, [0, 1, 2, 3, 4])
    assert ei.value.status == exm.ERR_CACHE
    with pytest.raises(exm.ExmoeError) as ei:
        c.acquire(2, [0])
    assert ei.value.status == exm.ERR_CACHE
    with pytest.raises(exm.ExmoeError) as ei:
        c.acquire(0, [8])
    assert ei.value.status == exm.ERR_INVALID_ARGUMENT
    c.acquire(0, [1, 1, 2])               # duplicates count once
    assert c.stats()["lookups"] == 2
    r = exm.SlotCache(1, 8, 8, 100, dry_run=True)
    r.acquire(0, [3, 4])
    st = r.stats()
    assert st["resident"] == 1 and st["lookups"] == 0 and st["h2d_bytes"] == 0
    assert list(r.table(0)) == list(range(8))


def test_workspace_flags_rejects_bad_input():
    lib = exm._lib
    v = ctypes.c_uint32(7)
    assert lib.exmoe_workspace_flags(None, 4096, 1, ctypes.byref(v), None) == exm.ERR_INVALID_ARGUMENT
    assert lib.exmoe_workspace_flags(FAKE, 4096, 1, None, None) == exm.ERR_INVALID_ARGUMENT
    assert lib.exmoe_workspace_flags(FAKE, 4095, 1, ctypes.byref(v), None) == exm.ERR_WORKSPACE
    assert v.value == 7


def test_group_workspace_size_and_check():
    assert exm._lib.exmoe_group_workspace_bytes(512, 8, 64) == 0                    # 4096 rows: one workgroup
    assert exm._lib.exmoe_group_workspace_bytes(513, 8, 64) == 5 * 64 * 4           # 4104 rows: 5 chunks
    assert exm._lib.exmoe_group_workspace_bytes(2048, 8, 64) == 16 * 64 * 4
    lib = exm._lib
    assert lib.exmoe_group_tokens(FAKE, 513, 8, 64, FAKE, FAKE, FAKE, None, 0, None) == exm.ERR_WORKSPACE
    assert lib.exmoe_group_tokens(FAKE, 513, 8, 64, FAKE, FAKE, FAKE, FAKE, 5 * 64 * 4 - 1, None) == exm.ERR_WORKSPACE

