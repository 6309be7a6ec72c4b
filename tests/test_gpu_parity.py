"""GPU parity: the HIP path through the C ABI against the CPU oracle on the same seeded
inputs. Integer outputs (logits bits, top-k ids, offsets, permutation) bit-exact; routing
weights within 1e-6; the layer output within the 1e-2 relative tolerance."""
import numpy as np
import pytest

import oracle
from synthetic import TINY, OLMOE, LARGE, LayerShape
from tests.helpers import (Layer, to_dev_bf16, bf16_dev_to_bits, bf16_dev_to_f64, check_y, check_routing, log)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def exm():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w4a16_mixture_experts_amd as m
    return m


def run_layer(exm, lay: Layer, x_bits, bias=None, flags=0, renormalize=True):
    import torch
    x = to_dev_bf16(x_bits, lay.device)
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(lay.device)
    out = exm.moe_layer(x, lay.wr, lay.bank, lay.shape.I, lay.shape.k, bias=b, renormalize=renormalize, flags=flags)
    torch.cuda.synchronize()
    return dict(logits=bf16_dev_to_bits(out.logits), ids=out.ids.cpu().numpy(), weights=out.weights.cpu().numpy(),
                offsets=out.offsets.cpu().numpy(), sorted_flat=out.sorted_flat.cpu().numpy()[: x_bits.shape[0] * lay.shape.k],
                flat_to_sorted=out.flat_to_sorted.cpu().numpy()[: x_bits.shape[0] * lay.shape.k],
                y=bf16_dev_to_f64(out.y), y_bits=bf16_dev_to_bits(out.y))


def oracle_layer(lay: Layer, x_bits, bias=None, renormalize=True, grouped=False, tokens=None, experts=None):
    from oracle.quant import bf16_bits_to_f64
    experts = lay.experts if experts is None else experts
    if not grouped:
        return oracle.moe_layer(x_bits, lay.wr_bits, experts, lay.shape.k, bias=bias, renormalize=renormalize,
                                tokens=tokens)
    logits = oracle.router_logits(x_bits, lay.wr_bits, bias)
    ids = oracle.topk_ids(logits, lay.shape.k)
    w = oracle.topk_weights(logits, ids, renormalize)
    off, sf, fs = oracle.group_tokens(ids, lay.shape.E)
    y = oracle.forward_grouped(bf16_bits_to_f64(x_bits), ids, w, experts, off, sf)
    return dict(logits=logits, ids=ids, weights=w, offsets=off, sorted_flat=sf, flat_to_sorted=fs, y=y)


# ------------------------------------------------------------------ tiny layer, every path
@pytest.fixture(scope="module")
def tiny(exm):
    return Layer(TINY, seed=0)


@pytest.mark.parametrize("path", [0, 1, 2, 3])
def test_tiny_layer_all_paths(exm, tiny, path):
    log(f"tiny layer T=16 path={path}")
    x = tiny.syn.x(16)
    ref = oracle_layer(tiny, x)
    got = run_layer(exm, tiny, x, flags=path)
    check_routing(got, ref, f"tiny/path{path}")
    check_y(got["y"], ref["y"], f"tiny/path{path}")
    again = run_layer(exm, tiny, x, flags=path)
    assert np.array_equal(again["y_bits"], got["y_bits"]), "not bitwise reproducible"


def test_tiny_paths_agree_and_separate_calls_match(exm, tiny):
    import torch
    x_bits = tiny.syn.x(37)      # ragged: 74 routed rows, 2.3 tiles of 32
    ref = oracle_layer(tiny, x_bits)
    outs = {p: run_layer(exm, tiny, x_bits, flags=p) for p in (1, 2, 3)}
    for p, o in outs.items():
        check_routing(o, ref, f"ragged/path{p}")
        check_y(o["y"], ref["y"], f"ragged/path{p}")
    # separate entry points give the same bits as the fused layer call
    x = to_dev_bf16(x_bits)
    logits, ids, w = exm.route_topk(x, tiny.wr, TINY.k)
    off, sf, fs = exm.group_tokens(ids, TINY.E)
    y = exm.moe_forward(x, ids, w, off, sf, fs, tiny.bank, TINY.I, flags=1)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_dev_to_bits(y), outs[1]["y_bits"])
    ids2, w2 = exm.topk_from_logits(logits, TINY.k)
    assert torch.equal(ids2, ids) and torch.equal(w2, w)
    w3 = exm.route_weights(logits, ids)
    assert torch.equal(w3, w)


def test_tiny_renormalize_off_and_bias(exm, tiny):
    x = tiny.syn.x(16)
    bias = np.linspace(-2, 2, TINY.E).astype(np.float32)
    ref = oracle_layer(tiny, x, bias=bias, renormalize=False)
    got = run_layer(exm, tiny, x, bias=bias, renormalize=False)
    check_routing(got, ref, "renorm0")
    check_y(got["y"], ref["y"], "renorm0")


def test_all_tokens_one_expert_and_empty_experts(exm, tiny):
    x = tiny.syn.x(40)
    bias = np.zeros(TINY.E, np.float32)
    bias[5] = 1000.0                       # every token picks expert 5 first
    for path in (1, 2):
        ref = oracle_layer(tiny, x, bias=bias)
        got = run_layer(exm, tiny, x, bias=bias, flags=path)
        assert (got["ids"][:, 0] == 5).all()
        check_routing(got, ref, f"one-expert/path{path}")
        check_y(got["y"], ref["y"], f"one-expert/path{path}")


def test_k_equals_E_and_single_expert(exm):
    for shape in (LayerShape(H=128, I=256, E=4, k=4), LayerShape(H=256, I=128, E=1, k=1)):
        lay = Layer(shape, seed=3)
        x = lay.syn.x(9)
        ref = oracle_layer(lay, x)
        for path in (1, 2, 3):
            got = run_layer(exm, lay, x, flags=path)
            check_routing(got, ref, f"{shape}/path{path}")
            check_y(got["y"], ref["y"], f"E{shape.E}k{shape.k}/path{path}")


@pytest.mark.parametrize("shape,Ts", [
    (LayerShape(H=128, I=128, E=256, k=64), (1, 3, 40)),      # most experts and the largest k
    (LayerShape(H=16384, I=128, E=2, k=1), (1, 5, 20)),       # largest hidden size: staged in 8 chunks
    (LayerShape(H=128, I=16384, E=2, k=2), (1, 5, 20)),       # largest intermediate size
])
def test_shape_limits(exm, shape, Ts):
    """The largest E, k, H and I the boundary accepts, on the decode, prefill and
    sequential paths and the automatic choice, at a ragged token count."""
    log(f"shape limits {shape}")
    lay = Layer(shape, seed=4)
    for T in Ts:
        x = lay.syn.x(T, stream=T)
        ref = oracle_layer(lay, x)
        for path in (0, 1, 2, 3):
            got = run_layer(exm, lay, x, flags=path)
            check_routing(got, ref, f"{shape} T={T} path={path}")
            check_y(got["y"], ref["y"], f"{shape} T={T} path={path}")


@pytest.mark.parametrize("T", [4, 5, 13, 16])
def test_table_routed_every_expert_repeated(exm, T):
    """Decode sizes with the routing kernel's table and every expert launched (8-wave fused
    kernel, 16 experts, intermediate 2048), ragged token counts: all outputs against the
    oracle, and three calls in a row equal bit for bit (the routing kernel leaves its
    arrival counters at zero for the next call)."""
    log(f"table routing, every expert launched, T={T}")
    lay = Layer(LayerShape(H=256, I=2048, E=16, k=8), seed=5)
    x = lay.syn.x(T, stream=70 + T)
    ref = oracle_layer(lay, x)
    first = None
    for rep in range(3):
        got = run_layer(exm, lay, x)
        check_routing(got, ref, f"T={T} call {rep}")
        if first is None:
            check_y(got["y"], ref["y"], f"T={T}")
            first = got["y_bits"]
        else:
            assert np.array_equal(got["y_bits"], first), f"call {rep} differs"


def test_zero_tokens_is_noop(exm, tiny):
    import torch
    x = torch.empty((0, TINY.H), dtype=torch.bfloat16, device="cuda")
    out = exm.moe_layer(x, tiny.wr, tiny.bank, TINY.I, TINY.k)
    torch.cuda.synchronize()
    assert out.offsets.cpu().numpy().tolist() == [0] * (TINY.E + 1)


def test_slot_indirection_and_knockout(exm, tiny):
    """A permuted bank with an expert->slot table gives identical bits; replacing one
    expert's blob changes exactly the tokens routed to it (every routed expert runs)."""
    import torch
    x = tiny.syn.x(16)
    base = run_layer(exm, tiny, x, flags=1)
    perm = np.array([3, 7, 0, 5, 1, 6, 2, 4])             # expert e lives in slot perm[e]
    blobs = [None] * TINY.E
    for e in range(TINY.E):
        blobs[perm[e]] = tiny.blobs[e]
    bank = exm.bank_from_blobs(blobs)
    bank.expert_to_slot = torch.from_numpy(perm.astype(np.int32)).cuda()
    for path in (1, 2, 3):
        xx = to_dev_bf16(x)
        out = exm.moe_layer(xx, tiny.wr, bank, TINY.I, TINY.k, flags=path)
        torch.cuda.synchronize()
        ref_path = run_layer(exm, tiny, x, flags=path)
        assert np.array_equal(bf16_dev_to_bits(out.y), ref_path["y_bits"]), f"path {path}"
    other = Layer(TINY, seed=77, experts=[2], oracle_experts=False)
    for e in (2,):
        blobs = list(tiny.blobs)
        blobs[e] = other.blobs[e]
        lay2 = exm.bank_from_blobs(blobs)
        xx = to_dev_bf16(x)
        out = exm.moe_layer(xx, tiny.wr, lay2, TINY.I, TINY.k, flags=1)
        torch.cuda.synchronize()
        changed = np.nonzero(np.any(bf16_dev_to_bits(out.y) != base["y_bits"], axis=1))[0]
        assert np.array_equal(changed, oracle.knockout_rows(base["ids"], e))


@pytest.mark.parametrize("path", [1, 2, 3])
def test_expert_without_slot_is_flagged(exm, tiny, path):
    """A routed expert mapped to slot -1 is a caller error: the kernels skip its rows and
    record it in the workspace, which exmoe_workspace_flags reports (and clears); a call
    with every routed expert mapped records nothing."""
    import torch
    x = to_dev_bf16(tiny.syn.x(16))
    bank = exm.bank_from_blobs(tiny.blobs)
    out = exm.moe_layer(x, tiny.wr, bank, TINY.I, TINY.k, flags=path)
    assert exm.workspace_flags(out.workspace) == 0
    routed = sorted(set(out.ids.cpu().numpy().ravel().tolist()))
    table = np.arange(TINY.E, dtype=np.int32)
    table[routed[0]] = -1
    bank.expert_to_slot = torch.from_numpy(table).cuda()
    exm.moe_layer(x, tiny.wr, bank, TINY.I, TINY.k, flags=path, buffers=out)
    assert exm.workspace_flags(out.workspace) & exm.FLAG_EXPERT_WITHOUT_SLOT
    assert exm.workspace_flags(out.workspace) == 0          # cleared by the previous read


@pytest.mark.parametrize("T,k,E", [(4096, 1, 8), (4097, 1, 64), (2049, 8, 64), (300, 64, 256), (5000, 2, 3),
                                   (8192, 8, 256), (9000, 8, 64)])
def test_grouping_many_rows_chunked(exm, T, k, E):
    """The grouping of more than 4096 routed rows (chunk counts of 1024 rows, then up to 64
    chunks scatters that scan the counts themselves, beyond that one scan launch and the
    scatters) against the oracle, bit for bit, including a ragged last chunk, empty
    experts, exactly 64 chunks (8192 x 8) and 71 chunks (9000 x 8)."""
    import torch
    rng = np.random.default_rng(T + E)
    if E >= k:
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    else:
        ids = rng.integers(0, E, size=(T, k)).astype(np.int32)
    ids[:, 0] = np.where(rng.random(T) < 0.5, 0, ids[:, 0]) if k == 1 else ids[:, 0]   # skew toward expert 0
    off, sf, fs = exm.group_tokens(torch.from_numpy(ids).cuda(), E)
    torch.cuda.synchronize()
    r_off, r_sf, r_fs = oracle.group_tokens(ids, E)
    assert np.array_equal(off.cpu().numpy(), r_off)
    assert np.array_equal(sf.cpu().numpy(), r_sf)
    assert np.array_equal(fs.cpu().numpy(), r_fs)


@pytest.mark.parametrize("T", [40, 128, 300])
def test_pass_parallel_decode_hot_experts(exm, T):
    """More than 16 tokens with every token on the same k experts (a +30 logit bias on
    them): the pass-parallel decode kernel gives each expert T / 16 passes of its own
    workgroups. T k <= 1024 groups in the kernel (ids), above that the grouping comes in
    (offsets and permutation); against the oracle, with the automatic path as well."""
    log(f"hot experts, T={T}")
    shape = LayerShape(H=256, I=1024, E=32, k=4)
    lay = Layer(shape, seed=8)
    bias = np.zeros(shape.E, np.float32)
    bias[[3, 11, 20, 29]] = 30.0
    x = lay.syn.x(T, stream=T)
    ref = oracle_layer(lay, x, bias=bias)
    assert set(np.unique(ref["ids"])) == {3, 11, 20, 29}
    for path in (0, 1):
        got = run_layer(exm, lay, x, bias=bias, flags=path)
        check_routing(got, ref, f"T={T} path={path}")
        check_y(got["y"], ref["y"], f"T={T} path={path}")


# ------------------------------------------------------------------ OLMoE-shaped layers
@pytest.fixture(scope="module")
def olmoe(exm):
    log("building OLMoE-shaped layer (64 experts)")
    return Layer(OLMOE, seed=0)


@pytest.mark.parametrize("T,path", [(1, 0), (3, 0), (5, 0), (1, 1), (3, 1)])
def test_tiny_few_tokens_narrow_kernel(exm, tiny, T, path):
    """A few routed rows (the narrow fused kernel: 32-row slices, quarters of the input
    groups, one 32-input step of each down tile): here H = 256 leaves two of the four
    quarters and most down row blocks empty."""
    log(f"tiny layer T={T} path={path}")
    x = tiny.syn.x(T, stream=60 + T)
    ref = oracle_layer(tiny, x)
    got = run_layer(exm, tiny, x, flags=path)
    check_routing(got, ref, f"T={T} path={path}")
    check_y(got["y"], ref["y"], f"T={T} path={path}")


@pytest.mark.parametrize("T", [1, 2, 4, 16])
def test_olmoe_decode(exm, olmoe, T):
    log(f"olmoe decode T={T}")
    x = olmoe.syn.x(T)
    ref = oracle_layer(olmoe, x)
    for path in (0, 3):
        got = run_layer(exm, olmoe, x, flags=path)
        check_routing(got, ref, f"decode T={T} path={path}")
        check_y(got["y"], ref["y"], f"decode T={T} path={path}")
    # the sequential path's split launches add their partial sums in a fixed order
    again = run_layer(exm, olmoe, x, flags=3)
    assert np.array_equal(again["y_bits"], got["y_bits"]), "sequential path not bitwise reproducible"


@pytest.mark.parametrize("T,k,renormalize,biased", [(1, 8, True, False), (2, 8, False, True), (5, 1, True, False),
                                                    (7, 16, True, False), (9, 8, True, False), (16, 4, True, True),
                                                    (16, 8, False, True), (3, 64, True, False)])
def test_olmoe_logit_routed_decode(exm, olmoe, T, k, renormalize, biased):
    """Decode with E <= 64 and table-sized batches: the routing kernel writes only the
    logits and every expert workgroup makes the top-k selection itself (the narrow kernel,
    the 8-wave launch of the active experts with one or two tokens per wave, and the
    16-wave launch of every expert); the publisher writes ids and weights. Other k than the
    layer's own (1 to E), full-softmax weights and a logit bias; the same experts."""
    import copy
    import dataclasses
    lay = copy.copy(olmoe)
    lay.shape = dataclasses.replace(OLMOE, k=k)
    x = olmoe.syn.x(T, stream=70 + T)
    bias = olmoe.syn.zipf_bias() if biased else None
    log(f"olmoe logit-routed decode T={T} k={k} renormalize={renormalize} bias={biased}")
    ref = oracle_layer(lay, x, bias=bias, renormalize=renormalize)
    got = run_layer(exm, lay, x, bias=bias, renormalize=renormalize)
    check_routing(got, ref, f"T={T} k={k}")
    check_y(got["y"], ref["y"], f"T={T} k={k}")


@pytest.mark.parametrize("T", [128, 512, 2048])
def test_olmoe_prefill_zipf(exm, olmoe, T):
    log(f"olmoe prefill T={T} (Zipf-biased routing)")
    x = olmoe.syn.x(T)
    bias = olmoe.syn.zipf_bias()
    ref = oracle_layer(olmoe, x, bias=bias, grouped=True)
    counts = np.diff(ref["offsets"])
    log(f"  rows per expert: min {counts.min()} max {counts.max()} zero-count experts {(counts == 0).sum()}")
    # at 128 tokens the sequential path mixes both of its launch pairs: split launches for
    # experts with up to 16 rows, the decode kernel pair for the hot ones
    paths = (0, 1, 2, 3) if T <= 128 else (0, 1, 2) if T <= 512 else (0, 2)
    for path in paths:
        got = run_layer(exm, olmoe, x, bias=bias, flags=path)
        check_routing(got, ref, f"prefill T={T} path={path}")
        check_y(got["y"], ref["y"], f"prefill T={T} path={path}")


# ------------------------------------------------------------------ slot cache
def test_slot_cache_outputs_equal_resident(exm):
    """A 3-layer stack through a 3-slot cache: outputs bitwise equal to the fully resident
    bank, counters equal to the oracle's LRU simulator."""
    import torch
    from synthetic import slot_cache_trace
    shape = LayerShape(H=256, I=256, E=8, k=2)
    layers = [Layer(shape, seed=10 + l, oracle_experts=False) for l in range(3)]
    nb = exm.packed_expert_bytes(shape.H, shape.I)
    cache = exm.SlotCache(3, shape.E, 3, nb)
    for l, lay in enumerate(layers):
        for e in range(shape.E):
            cache.fill(l, e, lay.blobs[e])
    sim = oracle.LRUSlotCacheSim(3, shape.E, 3, nb)
    trace = slot_cache_trace(E=shape.E, k=2, layers=3, steps=20, seed=4)
    x_bits = layers[0].syn.x(1)
    x = to_dev_bf16(x_bits)
    for step in trace:
        for l, lay in enumerate(layers):
            ids = torch.from_numpy(step[l][None, :].astype(np.int32)).cuda()
            logits, _, _ = exm.route_topk(x, lay.wr, shape.k)
            w = exm.route_weights(logits, ids)
            off, sf, fs = exm.group_tokens(ids, shape.E)
            active = exm.active_experts(off)
            bank = cache.acquire(l, active)
            sim.acquire(l, active)
            y_c = exm.moe_forward(x, ids, w, off, sf, fs, bank, shape.I)
            y_r = exm.moe_forward(x, ids, w, off, sf, fs, lay.bank, shape.I)
            torch.cuda.synchronize()
            assert torch.equal(y_c.view(torch.int16), y_r.view(torch.int16))
    st = cache.stats()
    assert (st["lookups"], st["hits"], st["misses"], st["evictions"], st["h2d_bytes"]) == \
        (sim.lookups, sim.hits, sim.misses, sim.evictions, sim.h2d_bytes)
    cache.close()


# ------------------------------------------------------------------ cache-sized waves
def _cached_vs_resident(exm, lay, cache, sim, x, path, bias=None):
    import torch
    shape = lay.shape
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).cuda()
    logits, ids, w = exm.route_topk(x, lay.wr, shape.k, bias=b)
    off, sf, fs = exm.group_tokens(ids, shape.E)
    active = exm.active_experts(off)
    y_c = exm.moe_forward_cached(x, ids, w, off, sf, fs, cache, 0, active, shape.I, flags=path)
    waves = sim.acquire_waves(0, active)
    y_r = exm.moe_forward(x, ids, w, off, sf, fs, lay.bank, shape.I, flags=path)
    torch.cuda.synchronize()
    assert torch.equal(y_c.view(torch.int16), y_r.view(torch.int16)), f"cached output differs (path {path})"
    return len(active), len(waves)


def _same_counters(cache, sim):
    st = cache.stats()
    assert (st["lookups"], st["hits"], st["misses"], st["evictions"], st["h2d_bytes"]) == \
        (sim.lookups, sim.hits, sim.misses, sim.evictions, sim.h2d_bytes)


@pytest.mark.parametrize("path", [1, 2])
def test_forward_cached_waves_equal_resident(exm, path):
    """Calls routed to more experts than a 5-slot cache holds run in waves; the output is
    bitwise the resident bank's on the same path and the counters are the oracle's wave
    simulation (ragged T included)."""
    log(f"cached waves, 16 experts, 5 slots, path {path}")
    shape = LayerShape(H=256, I=256, E=16, k=4)
    lay = Layer(shape, seed=21, oracle_experts=False)
    nb = exm.packed_expert_bytes(shape.H, shape.I)
    S = 5
    cache = exm.SlotCache(1, shape.E, S, nb)
    for e in range(shape.E):
        cache.fill(0, e, lay.blobs[e])
    sim = oracle.LRUSlotCacheSim(1, shape.E, S, nb)
    for T, stream in ((16, 1), (37, 2), (5, 3), (16, 1)):
        n_act, n_waves = _cached_vs_resident(exm, lay, cache, sim, to_dev_bf16(lay.syn.x(T, stream=stream)), path)
        W = S if n_act <= S else S // 2
        assert n_waves == -(-n_act // W)
    _same_counters(cache, sim)
    cache.close()


@pytest.mark.parametrize("path", [1, 2])
def test_forward_cached_most_experts(exm, path):
    """256 experts (the largest E, so every per-wave table is the full 1 KiB of kernel
    arguments) behind 24 slots, top-8 of 40 tokens: several waves per call, bitwise equal
    to the resident bank; the counters are the oracle's wave simulation."""
    log(f"cached waves, 256 experts, 24 slots, path {path}")
    shape = LayerShape(H=128, I=128, E=256, k=8)
    lay = Layer(shape, seed=23, oracle_experts=False)
    nb = exm.packed_expert_bytes(shape.H, shape.I)
    cache = exm.SlotCache(1, shape.E, 24, nb)
    for e in range(shape.E):
        cache.fill(0, e, lay.blobs[e])
    sim = oracle.LRUSlotCacheSim(1, shape.E, 24, nb)
    for T, stream in ((40, 1), (7, 2), (40, 3)):
        n_act, n_waves = _cached_vs_resident(exm, lay, cache, sim, to_dev_bf16(lay.syn.x(T, stream=stream)), path)
        assert n_waves == -(-n_act // (24 if n_act <= 24 else 12))
    assert n_waves > 1
    _same_counters(cache, sim)
    cache.close()


def test_olmoe_cached_waves(exm, olmoe):
    """OLMoE-shaped decode (16 tokens, fused expert kernel) and Zipf-biased prefill (128
    tokens) through a 16-slot cache: bitwise equal to the resident bank."""
    log("olmoe through a 16-slot cache in waves")
    nb = exm.packed_expert_bytes(OLMOE.H, OLMOE.I)
    cache = exm.SlotCache(1, OLMOE.E, 16, nb)
    for e in range(OLMOE.E):
        cache.fill(0, e, olmoe.blobs[e])
    sim = oracle.LRUSlotCacheSim(1, OLMOE.E, 16, nb)
    n_act, n_waves = _cached_vs_resident(exm, olmoe, cache, sim, to_dev_bf16(olmoe.syn.x(16, stream=5)), 0)
    log(f"  decode: {n_act} active experts in {n_waves} waves")
    assert n_waves > 1
    n_act, n_waves = _cached_vs_resident(exm, olmoe, cache, sim, to_dev_bf16(olmoe.syn.x(128, stream=6)), 0,
                                         bias=olmoe.syn.zipf_bias())
    log(f"  prefill: {n_act} active experts in {n_waves} waves")
    assert n_waves > 1
    _same_counters(cache, sim)
    cache.close()


def test_cached_forward_layer_stack_without_sync(exm):
    """Three layers behind 4 slots each, 24 steps of 3-token cached forwards enqueued with
    no synchronization in between, so the copies of one layer run while the kernels of
    others are in flight (several waves when a step routes to more than 4 experts); every
    fifth step layer 1 goes through the public acquire and a plain forward instead. Every
    output equals the resident bank's bit for bit and the counters are the oracle's."""
    import torch
    from synthetic import slot_cache_trace
    log("3-layer stack through 4-slot caches, no synchronization between layers")
    shape = LayerShape(H=256, I=256, E=8, k=2)
    layers = [Layer(shape, seed=40 + l, oracle_experts=False) for l in range(3)]
    nb = exm.packed_expert_bytes(shape.H, shape.I)
    S, steps = 4, 24
    cache = exm.SlotCache(3, shape.E, S, nb)
    for l, lay in enumerate(layers):
        for e in range(shape.E):
            cache.fill(l, e, lay.blobs[e])
    sim = oracle.LRUSlotCacheSim(3, shape.E, S, nb)
    trace = slot_cache_trace(E=shape.E, k=2, layers=3, steps=steps, seed=7)
    outs, n_multi = [], 0
    for st in range(steps):
        x_all = to_dev_bf16(layers[0].syn.x(3, stream=100 + st))
        for l, lay in enumerate(layers):
            public = l == 1 and st % 5 == 2
            rows = [trace[(st + j) % steps][l] for j in range(1 if public else 3)]
            ids = torch.from_numpy(np.stack(rows).astype(np.int32)).cuda()
            x = x_all[: len(rows)]
            logits, _, _ = exm.route_topk(x, lay.wr, shape.k)
            w = exm.route_weights(logits, ids)
            off, sf, fs = exm.group_tokens(ids, shape.E)
            active = sorted(set(int(e) for r in rows for e in r))
            if public:
                sim.acquire(l, active)
                y = exm.moe_forward(x, ids, w, off, sf, fs, cache.acquire(l, active), shape.I)
            else:
                n_multi += len(sim.acquire_waves(l, active)) > 1
                y = exm.moe_forward_cached(x, ids, w, off, sf, fs, cache, l, active, shape.I)
            outs.append((st, l, y, exm.moe_forward(x, ids, w, off, sf, fs, lay.bank, shape.I)))
    torch.cuda.synchronize()
    for st, l, y, y_ref in outs:
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"step {st} layer {l}"
    log(f"  {n_multi} calls ran in several waves")
    assert n_multi > 0
    _same_counters(cache, sim)
    cache.close()


# ------------------------------------------------------------------ bf16 comparator
def run_layer_bf16(exm, lay: Layer, x_bits, bias=None, flags=0):
    import torch
    x = to_dev_bf16(x_bits, lay.device)
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(lay.device)
    out = exm.moe_layer(x, lay.wr, lay.bf16_bank, lay.shape.I, lay.shape.k, bias=b, flags=flags | exm.WEIGHTS_BF16)
    torch.cuda.synchronize()
    T = x_bits.shape[0]
    return dict(logits=bf16_dev_to_bits(out.logits), ids=out.ids.cpu().numpy(), weights=out.weights.cpu().numpy(),
                offsets=out.offsets.cpu().numpy(), sorted_flat=out.sorted_flat.cpu().numpy()[: T * lay.shape.k],
                flat_to_sorted=out.flat_to_sorted.cpu().numpy()[: T * lay.shape.k], y=bf16_dev_to_f64(out.y),
                y_bits=bf16_dev_to_bits(out.y))


def oracle_layer_bf16(lay: Layer, x_bits, bias=None):
    return oracle_layer(lay, x_bits, bias=bias, grouped=x_bits.shape[0] > 64, experts=lay.dense)


@pytest.mark.parametrize("path", [0, 1, 2])
def test_tiny_bf16_layer_paths(exm, path):
    """The comparator layer (dense bf16 experts) against the oracle on the same routing,
    every path, with a ragged token count."""
    log(f"tiny bf16 layer, path {path}")
    lay = Layer(TINY, seed=3, oracle_experts=False).add_bf16()
    for T in (16, 37):
        x = lay.syn.x(T, stream=T)
        ref = oracle_layer_bf16(lay, x)
        got = run_layer_bf16(exm, lay, x, flags=path)
        check_routing(got, ref, f"bf16 T={T} path={path}")
        check_y(got["y"], ref["y"], f"bf16 T={T} path={path}")


def test_bf16_sequential_path_unsupported(exm):
    lay = Layer(TINY, seed=3, oracle_experts=False).add_bf16(oracle_experts=False)
    with pytest.raises(exm.ExmoeError) as ei:
        run_layer_bf16(exm, lay, lay.syn.x(4), flags=exm.PATH_SEQUENTIAL)
    assert ei.value.status == exm.ERR_UNSUPPORTED


def test_olmoe_bf16_decode_and_prefill(exm, olmoe):
    """OLMoE-shaped comparator layer: decode at 1 and 16 tokens, Zipf-biased prefill at
    512 tokens, against the oracle's bf16 experts."""
    log("olmoe bf16 comparator: packing 64 dense experts")
    olmoe.add_bf16()
    for T, bias in ((1, None), (16, None), (512, olmoe.syn.zipf_bias())):
        x = olmoe.syn.x(T, stream=40 + T)
        ref = oracle_layer_bf16(olmoe, x, bias)
        got = run_layer_bf16(exm, olmoe, x, bias)
        check_routing(got, ref, f"olmoe bf16 T={T}")
        check_y(got["y"], ref["y"], f"olmoe bf16 T={T}")
    for d in olmoe.dense:
        d.drop_cache()


def test_bf16_cached_waves_equal_resident(exm):
    """Dense bf16 experts through a slot cache in waves: bitwise equal to the resident bf16
    bank on the decode and prefill paths."""
    import torch
    log("bf16 experts through a 5-slot cache")
    shape = LayerShape(H=256, I=256, E=16, k=4)
    lay = Layer(shape, seed=22, oracle_experts=False).add_bf16(oracle_experts=False)
    nb = exm.bf16_expert_bytes(shape.H, shape.I)
    cache = exm.SlotCache(1, shape.E, 5, nb)
    for e in range(shape.E):
        cache.fill(0, e, lay.bf16_blobs[e])
    for T, path in ((16, 1), (37, 2), (16, 1)):
        x = to_dev_bf16(lay.syn.x(T, stream=T))
        logits, ids, w = exm.route_topk(x, lay.wr, shape.k)
        off, sf, fs = exm.group_tokens(ids, shape.E)
        active = exm.active_experts(off)
        fl = path | exm.WEIGHTS_BF16
        y_c = exm.moe_forward_cached(x, ids, w, off, sf, fs, cache, 0, active, shape.I, flags=fl)
        y_r = exm.moe_forward(x, ids, w, off, sf, fs, lay.bf16_bank, shape.I, flags=fl)
        torch.cuda.synchronize()
        assert torch.equal(y_c.view(torch.int16), y_r.view(torch.int16)), f"T={T} path={path}"
    cache.close()

