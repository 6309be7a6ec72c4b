"""GPU parity, wider coverage: the large-expert layer on rows of every expert's segment
(first, last and the start of the ragged last 128-row tile), routing weights of a routing
trace (ids that are not the top-k), batched decode through a small slot-cache stack
against the oracle element by element, constructed top-k ties, and the exactness
counters and flags (every routed row runs once on its own expert; a skipped expert or an
incomplete grouping is reported). Everything goes through the C ABI; the oracle computes
every expected value."""
import numpy as np
import pytest

import oracle
from oracle.quant import bf16_bits_to_f64
from synthetic import LARGE, LayerShape, batch_trace
from tests.helpers import Layer, to_dev_bf16, bf16_dev_to_bits, bf16_dev_to_f64, check_y, check_routing, log

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def exm():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import w4a16_mixture_experts_amd as m
    return m


# ------------------------------------------------------------------ large-expert prefill, every expert
def _segment_rows(sf, off, e, k, tile=64):
    """Tokens of expert e's first row, of the first row of its last `tile`-row tile (the
    ragged one the kernel masks), of the row before it and of its last row."""
    seg = sf[off[e]:off[e + 1]]
    n = len(seg)
    if n == 0:
        return set()
    last_tile = (n - 1) // tile * tile
    picks = {0, n - 1, last_tile, max(last_tile - 1, 0)}
    return {int(seg[i]) // k for i in picks}


def test_large_prefill_every_expert_segment(exm):
    """Hidden 4096, 8 experts, top-2, intermediate 14336, 4096 tokens, in the benchmark's
    launch configuration. Routing is compared on every token; the output on the first and
    last rows of every expert's segment, the rows around the start of its ragged last
    tile, and 16 random tokens. The oracle computes one expert at a time on the rows
    routed to it and drops that expert before the next, so memory stays bounded."""
    log("large prefill, every expert: building the layer (hidden 4096, intermediate 14336)")
    lay = Layer(LARGE, seed=0, oracle_experts=False)
    T, k, E = 4096, LARGE.k, LARGE.E
    x = lay.syn.x(T)
    got = run_layer(exm, lay, x)
    logits = oracle.router_logits(x, lay.wr_bits)
    ids = oracle.topk_ids(logits, k)
    w = oracle.topk_weights(logits, ids)
    off, sf, fs = oracle.group_tokens(ids, E)
    check_routing(got, dict(logits=logits, ids=ids, weights=w, offsets=off, sorted_flat=sf, flat_to_sorted=fs),
                  "large")
    tokens = set()
    for e in range(E):
        tokens |= _segment_rows(sf, off, e, k)
    tokens |= {int(t) for t in np.random.default_rng(3).choice(T, 16, replace=False)}
    tokens = sorted(tokens)
    xf = bf16_bits_to_f64(x)
    o = {}
    for e in range(E):
        need = [(t, j) for t in tokens for j in range(k) if ids[t, j] == e]
        log(f"  expert {e}: segment of {off[e + 1] - off[e]} rows, {len(need)} rows checked")
        assert need, f"expert {e} has no checked row"
        qe = oracle.quantize_expert(*lay.syn.expert(e))
        out = oracle.expert_mlp(qe, xf[[t for t, _ in need]])
        for tj, v in zip(need, out):
            o[tj] = v
        del qe
    y_ref = np.stack([oracle.combine(np.stack([o[(t, j)] for j in range(k)]), w[t:t + 1], 1, k)[0]
                      for t in tokens])
    check_y(got["y"][tokens], y_ref, f"large, {len(tokens)} tokens over all {E} experts")


def run_layer(exm, lay, x_bits):
    import torch
    out = exm.moe_layer(to_dev_bf16(x_bits, lay.device), lay.wr, lay.bank, lay.shape.I, lay.shape.k)
    torch.cuda.synchronize()
    T = x_bits.shape[0]
    return dict(logits=bf16_dev_to_bits(out.logits), ids=out.ids.cpu().numpy(), weights=out.weights.cpu().numpy(),
                offsets=out.offsets.cpu().numpy(), sorted_flat=out.sorted_flat.cpu().numpy()[:T * lay.shape.k],
                flat_to_sorted=out.flat_to_sorted.cpu().numpy()[:T * lay.shape.k], y=bf16_dev_to_f64(out.y))


# ------------------------------------------------------------------ routing trace, batched decode through a cache
@pytest.mark.parametrize("renormalize", [True, False])
def test_route_weights_on_trace_ids(exm, renormalize):
    """Weights of externally chosen experts (a routing trace, not the top-k) from the GPU's
    own logits, against the oracle's weights over the same ids within 1e-6."""
    import torch
    shape = LayerShape(H=512, I=128, E=64, k=8)
    lay = Layer(shape, seed=31, oracle_experts=False)
    trace = batch_trace(shape.E, shape.k, 1, 4, 16, seed=5)          # [steps, 1, 16, k]
    for st in range(trace.shape[0]):
        ids_np = trace[st, 0]
        x_bits = lay.syn.x(16, stream=50 + st)
        logits, topk, _ = exm.route_topk(to_dev_bf16(x_bits), lay.wr, shape.k)
        ids = torch.from_numpy(ids_np.astype(np.int32)).cuda()
        w = exm.route_weights(logits, ids, renormalize=renormalize)
        torch.cuda.synchronize()
        lg = bf16_dev_to_bits(logits)
        ref_lg = oracle.router_logits(x_bits, lay.wr_bits)
        assert np.array_equal(lg, ref_lg)
        assert not np.array_equal(np.sort(ids_np, axis=1), np.sort(topk.cpu().numpy(), axis=1))
        ref = oracle.topk_weights(ref_lg, ids_np, renormalize)
        dw = np.abs(w.cpu().numpy().astype(np.float64) - ref).max()
        assert dw <= 1e-6, f"step {st}: weights differ by {dw:.2e}"


@pytest.mark.parametrize("B", [1, 2, 4, 8])
def test_batched_decode_through_cache_vs_oracle(exm, B):
    """Batched decode as the benchmark runs it, at a size the oracle finishes quickly:
    3 layers of 16 experts (top-4) behind 4 slots each, B sequences per call, routed by a
    per-sequence trace over each layer's shared Zipf popularity. Per (step, layer): logits
    on the GPU, weights of the trace's ids, grouping, the active set read back, then the
    expert layer in cache-sized waves. Logits bit-exact, weights within 1e-6, the output
    against the oracle's per-token layer (Q16 tolerance) and the counters against the
    oracle's wave simulation."""
    import torch
    shape = LayerShape(H=256, I=256, E=16, k=4)
    L, S, steps = 3, 4, 6
    layers = [Layer(shape, seed=60 + l) for l in range(L)]
    nb = exm.packed_expert_bytes(shape.H, shape.I)
    cache = exm.SlotCache(L, shape.E, S, nb)
    for l, lay in enumerate(layers):
        for e in range(shape.E):
            cache.fill(l, e, lay.blobs[e])
    sim = oracle.LRUSlotCacheSim(L, shape.E, S, nb)
    trace = batch_trace(shape.E, shape.k, L, steps, B, seed=9)
    multi = 0
    for st in range(steps):
        x_bits = layers[0].syn.x(B, stream=200 + st)
        x = to_dev_bf16(x_bits)
        xf = bf16_bits_to_f64(x_bits)
        for l, lay in enumerate(layers):
            ids_np = trace[st, l]
            ids = torch.from_numpy(ids_np.astype(np.int32)).cuda()
            logits, _, _ = exm.route_topk(x, lay.wr, shape.k)
            w = exm.route_weights(logits, ids)
            off, sf, fs = exm.group_tokens(ids, shape.E)
            active = exm.active_experts(off)
            waves = sim.acquire_waves(l, active)
            multi += len(waves) > 1
            y = exm.moe_forward_cached(x, ids, w, off, sf, fs, cache, l, active, shape.I)
            torch.cuda.synchronize()
            ref_lg = oracle.router_logits(x_bits, lay.wr_bits)
            ref_w = oracle.topk_weights(ref_lg, ids_np)
            ref_off, ref_sf, ref_fs = oracle.group_tokens(ids_np, shape.E)
            got = dict(logits=bf16_dev_to_bits(logits), ids=ids_np, weights=w.cpu().numpy(),
                       offsets=off.cpu().numpy(), sorted_flat=sf.cpu().numpy(), flat_to_sorted=fs.cpu().numpy())
            check_routing(got, dict(logits=ref_lg, ids=ids_np, weights=ref_w, offsets=ref_off, sorted_flat=ref_sf,
                                    flat_to_sorted=ref_fs), f"B={B} step {st} layer {l}")
            assert active == sorted(set(int(e) for e in ids_np.reshape(-1)))
            y_ref = oracle.forward_per_token(xf, ids_np, ref_w, lay.experts)
            check_y(bf16_dev_to_f64(y), y_ref, f"B={B} step {st} layer {l} ({len(waves)} waves)")
    st_ = cache.stats()
    assert (st_["lookups"], st_["hits"], st_["misses"], st_["evictions"], st_["h2d_bytes"]) == \
        (sim.lookups, sim.hits, sim.misses, sim.evictions, sim.h2d_bytes)
    if B >= 2:
        assert multi > 0, "no call ran in several waves"
    cache.close()


# ------------------------------------------------------------------ constructed ties
def _bits(vals):
    from synthetic import f32_to_bf16_bits
    return f32_to_bf16_bits(np.asarray(vals, np.float32))


@pytest.mark.parametrize("E,k", [(64, 8), (8, 2), (256, 8), (16, 16)])
def test_topk_constructed_ties(exm, E, k):
    """Top-k from given bf16 logits with ties built in: equal logits straddling the k-th
    place (the lower expert id wins), +0 against -0 at the k-th place (they are equal), a
    row of all-equal logits, a row whose k-th and (k+1)-th are the same negative value,
    and random rows with heavy duplication. Ids bit-exact against the oracle's stable
    sort; weights within 1e-6."""
    import torch
    rng = np.random.default_rng(E * 100 + k)
    rows = []
    r = rng.standard_normal(E).astype(np.float32)
    if k < E:
        order = np.argsort(-r, kind="stable")
        r[order[k]] = r[order[k - 1]]                 # tie across the k-th place
    rows.append(r)
    z = rng.uniform(0.5, 2.0, E).astype(np.float32)   # positive
    if k < E:
        sel = rng.choice(E, k - 1, replace=False)
        rest = np.setdiff1d(np.arange(E), sel)
        z[rest] = -rng.uniform(0.5, 2.0, rest.size)
        pz, nz = rng.choice(rest, 2, replace=False)
        z[pz], z[nz] = 0.0, -0.0                        # +0 and -0 compete for the k-th place
    rows.append(z)
    rows.append(np.full(E, 0.75, np.float32))           # all equal
    rows.append(np.full(E, -3.0, np.float32))
    for _ in range(5):
        rows.append(rng.integers(-3, 3, E).astype(np.float32) * np.float32(0.5))   # heavy duplication
    bits = np.stack([_bits(rw) for rw in rows])
    if k < E:
        bits[1][pz], bits[1][nz] = 0x0000, 0x8000
    lg = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
    for renorm in (True, False):
        ids, w = exm.topk_from_logits(lg, k, renormalize=renorm)
        torch.cuda.synchronize()
        ref_ids = oracle.topk_ids(bits, k)
        ref_w = oracle.topk_weights(bits, ref_ids, renorm)
        assert np.array_equal(ids.cpu().numpy(), ref_ids), (ids.cpu().numpy(), ref_ids)
        dw = np.abs(w.cpu().numpy().astype(np.float64) - ref_w).max()
        assert dw <= 1e-6, dw
    if k < E:
        # the ties really are at the k-th place
        l1 = bf16_bits_to_f64(bits[1])
        kth = np.sort(-l1, kind="stable")[k - 1]
        assert np.count_nonzero(-l1 == kth) >= 2


# ------------------------------------------------------------------ exactness counters and flags
def _forward_counted(exm, lay, x_bits, flags, bias=None):
    """One layer call with the exactness counters on; returns (rows per expert, offsets)."""
    import torch
    x = to_dev_bf16(x_bits, lay.device)
    b = None if bias is None else torch.from_numpy(np.asarray(bias, np.float32)).to(lay.device)
    bank = lay.bf16_bank if flags & exm.WEIGHTS_BF16 else lay.bank
    out = exm.moe_layer(x, lay.wr, bank, lay.shape.I, lay.shape.k, bias=b, flags=flags | exm.DEBUG_COUNTERS)
    rows = exm.workspace_rows(out.workspace, lay.shape.E)
    assert exm.workspace_flags(out.workspace) == 0
    return rows, out.offsets.cpu().numpy()


@pytest.fixture(scope="module")
def tiny_bf16(exm):
    from synthetic import TINY
    return Layer(TINY, seed=0, oracle_experts=False).add_bf16(oracle_experts=False)


@pytest.fixture(scope="module")
def olmoe_packed(exm):
    from synthetic import OLMOE
    return Layer(OLMOE, seed=0, oracle_experts=False)


@pytest.mark.parametrize("T,path,bf16", [
    (16, 0, False), (16, 1, False), (16, 2, False), (16, 3, False),   # two-kernel decode, grouped GEMM, sequential
    (3, 0, False), (1, 1, False), (37, 1, False), (37, 2, False),      # narrow kernel, more passes, ragged T
    (16, 1, True), (37, 2, True)])                                      # the bf16 comparator's kernels
def test_debug_counters_tiny_paths(exm, tiny_bf16, T, path, bf16):
    """Every routed row runs exactly once, on its own expert: the per-expert counters the
    expert kernels keep under EXMOE_FLAG_DEBUG_COUNTERS equal the segment sizes of the
    grouping, and the oracle's histogram of the same ids."""
    x = tiny_bf16.syn.x(T, stream=T + 7 * path)
    rows, off = _forward_counted(exm, tiny_bf16, x, path | (exm.WEIGHTS_BF16 if bf16 else 0))
    ids = oracle.topk_ids(oracle.router_logits(x, tiny_bf16.wr_bits), tiny_bf16.shape.k)
    assert np.array_equal(rows, np.diff(off)), (rows, np.diff(off))
    assert np.array_equal(rows, np.bincount(ids.reshape(-1), minlength=tiny_bf16.shape.E))


@pytest.mark.parametrize("T,bias", [(1, False), (4, False), (16, False), (64, True), (512, True)])
def test_debug_counters_olmoe_paths(exm, olmoe_packed, T, bias):
    """The OLMoE-shaped layer on the paths its sizes choose: narrow kernel (1 token), fused
    decode (4 and 16 tokens, table-routed), pass-parallel fused decode (64 tokens, Zipf
    skew) and the grouped GEMM (512 tokens, Zipf skew)."""
    x = olmoe_packed.syn.x(T, stream=900 + T)
    b = olmoe_packed.syn.zipf_bias() if bias else None
    rows, off = _forward_counted(exm, olmoe_packed, x, 0, bias=b)
    ids = oracle.topk_ids(oracle.router_logits(x, olmoe_packed.wr_bits, b), olmoe_packed.shape.k)
    assert np.array_equal(rows, np.bincount(ids.reshape(-1), minlength=olmoe_packed.shape.E))
    assert np.array_equal(rows, np.diff(off))


@pytest.mark.parametrize("T,bias", [(16, False), (128, True)])
def test_debug_counters_olmoe_sequential(exm, olmoe_packed, T, bias):
    """The sequential path on the OLMoE shape: experts with up to 16 rows run through the
    launch pair whose reductions are split over workgroups, hotter experts (Zipf skew at
    128 tokens) through the decode kernel pair; every routed row is counted once."""
    x = olmoe_packed.syn.x(T, stream=950 + T)
    b = olmoe_packed.syn.zipf_bias() if bias else None
    rows, off = _forward_counted(exm, olmoe_packed, x, 3, bias=b)
    ids = oracle.topk_ids(oracle.router_logits(x, olmoe_packed.wr_bits, b), olmoe_packed.shape.k)
    counts = np.bincount(ids.reshape(-1), minlength=olmoe_packed.shape.E)
    if bias:
        assert counts.max() > 16 and 0 < counts[counts > 0].min() <= 16   # both launch pairs ran
    assert np.array_equal(rows, counts)
    assert np.array_equal(rows, np.diff(off))


@pytest.mark.parametrize("path", [1, 2])
def test_debug_counters_cached_waves_and_missing_expert(exm, path):
    """A cached forward in several waves counts every routed row once; leaving a routed
    expert out of the active list of a multi-wave call leaves its counter short and sets
    EXMOE_FLAG_EXPERT_WITHOUT_SLOT (checked after the last wave)."""
    import torch
    shape = LayerShape(H=256, I=256, E=16, k=4)
    lay = Layer(shape, seed=21, oracle_experts=False)
    nb = exm.packed_expert_bytes(shape.H, shape.I)
    cache = exm.SlotCache(1, shape.E, 5, nb)
    for e in range(shape.E):
        cache.fill(0, e, lay.blobs[e])
    x = to_dev_bf16(lay.syn.x(16, stream=3))
    logits, ids, w = exm.route_topk(x, lay.wr, shape.k)
    off, sf, fs = exm.group_tokens(ids, shape.E)
    active = exm.active_experts(off)
    assert len(active) > 5
    ws = exm.alloc_workspace(exm.moe_workspace_bytes(16, shape.H, shape.I, shape.E, shape.k, path))
    exm.moe_forward_cached(x, ids, w, off, sf, fs, cache, 0, active, shape.I, flags=path | exm.DEBUG_COUNTERS,
                           workspace=ws)
    counts = np.diff(off.cpu().numpy())
    assert np.array_equal(exm.workspace_rows(ws, shape.E), counts)
    assert exm.workspace_flags(ws) == 0
    dropped = active[len(active) // 2]
    partial = [e for e in active if e != dropped]
    assert len(cache.waves(0, partial)) > 1
    exm.moe_forward_cached(x, ids, w, off, sf, fs, cache, 0, partial, shape.I, flags=path | exm.DEBUG_COUNTERS,
                           workspace=ws)
    rows = exm.workspace_rows(ws, shape.E)
    torch.cuda.synchronize()
    expect = counts.copy()
    expect[dropped] = 0
    assert np.array_equal(rows, expect)
    assert exm.workspace_flags(ws) & exm.FLAG_EXPERT_WITHOUT_SLOT
    cache.close()


@pytest.mark.parametrize("path", [1, 2, 3])
def test_slotless_expert_not_counted(exm, tiny_bf16, path):
    """Knockout through the bank: a routed expert mapped to slot -1 is skipped, flagged,
    and absent from the counters; every other expert's rows are still counted once."""
    import torch
    lay = tiny_bf16
    x = to_dev_bf16(lay.syn.x(16))
    logits, ids, w = exm.route_topk(x, lay.wr, lay.shape.k)
    off, sf, fs = exm.group_tokens(ids, lay.shape.E)
    counts = np.diff(off.cpu().numpy())
    gone = int(np.argmax(counts))
    table = torch.arange(lay.shape.E, dtype=torch.int32, device="cuda")
    table[gone] = -1
    bank = exm.ExpertBank(base=lay.bank.base, stride=lay.bank.stride, expert_to_slot=table)
    ws = exm.alloc_workspace(exm.moe_workspace_bytes(16, lay.shape.H, lay.shape.I, lay.shape.E, lay.shape.k, path))
    exm.moe_forward(x, ids, w, off, sf, fs, bank, lay.shape.I, flags=path | exm.DEBUG_COUNTERS, workspace=ws)
    expect = counts.copy()
    expect[gone] = 0
    assert np.array_equal(exm.workspace_rows(ws, lay.shape.E), expect)
    assert exm.workspace_flags(ws) == exm.FLAG_EXPERT_WITHOUT_SLOT


@pytest.mark.parametrize("path", [1, 2, 3])
def test_ungrouped_rows_flagged(exm, tiny_bf16, path):
    """An id outside [0, E) in the grouping input: the row is in no segment (offsets[E] =
    T k - 1, flat_to_sorted = -1 there), the other rows group as the oracle groups them,
    and the expert layer flags the incomplete grouping (EXMOE_FLAG_ROWS_UNGROUPED)."""
    import torch
    lay = tiny_bf16
    E, k = lay.shape.E, lay.shape.k
    x = to_dev_bf16(lay.syn.x(16))
    logits, ids, w = exm.route_topk(x, lay.wr, k)
    ids_np = ids.cpu().numpy()
    bad = ids_np.copy()
    bad[5, 1] = E
    off, sf, fs = exm.group_tokens(torch.from_numpy(bad).cuda(), E)
    off_np, fs_np = off.cpu().numpy(), fs.cpu().numpy()
    keep = np.ones(16 * k, bool)
    keep[5 * k + 1] = False
    assert off_np[E] == 16 * k - 1 and fs_np[5 * k + 1] == -1
    ref_counts = np.bincount(bad.reshape(-1)[keep], minlength=E)
    assert np.array_equal(np.diff(off_np), ref_counts)
    ref_sf = np.argsort(np.where(keep, bad.reshape(-1), E + 1), kind="stable")[:16 * k - 1]
    assert np.array_equal(sf.cpu().numpy()[:16 * k - 1], ref_sf)
    ws = exm.alloc_workspace(exm.moe_workspace_bytes(16, lay.shape.H, lay.shape.I, E, k, path))
    exm.moe_forward(x, ids, w, off, sf, fs, lay.bank, lay.shape.I, flags=path | exm.DEBUG_COUNTERS, workspace=ws)
    assert exm.workspace_flags(ws) == exm.FLAG_ROWS_UNGROUPED
    assert np.array_equal(exm.workspace_rows(ws, E), ref_counts)


# ------------------------------------------------------------------ whole-layer call against the separate calls
@pytest.mark.parametrize("T", [4, 5, 16])
def test_table_routed_layer_equals_separate_calls(exm, olmoe_packed, T):
    """The whole-layer call at decode sizes routes through the routing kernel's expert table
    (its fused expert kernel stages every token row, the 16-token case by direct copies
    into LDS); the same routing through the separate calls groups first and runs the
    fused kernel on the given grouping. Both outputs are equal bit for bit, and a second
    whole-layer call on the same workspace repeats them."""
    import torch
    lay = olmoe_packed
    s = lay.shape
    x_bits = lay.syn.x(T, stream=300 + T)
    x = to_dev_bf16(x_bits)
    out = exm.moe_layer(x, lay.wr, lay.bank, s.I, s.k)
    y_sep = exm.moe_forward(x, out.ids, out.weights, out.offsets, out.sorted_flat, out.flat_to_sorted, lay.bank, s.I)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_dev_to_bits(out.y), bf16_dev_to_bits(y_sep))
    again = exm.moe_layer(x, lay.wr, lay.bank, s.I, s.k, buffers=out)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_dev_to_bits(again.y), bf16_dev_to_bits(y_sep)), "second call on the same workspace differs"


@pytest.mark.parametrize("T", [1, 3])
def test_narrow_publisher_outputs_with_slot_table(exm, olmoe_packed, T):
    """A few tokens on the OLMoE shape (the narrow kernel, whose last slice workgroup also
    publishes ids, weights and the grouping): through a permuting expert->slot table the
    output equals the resident bank's bit for bit; with every expert unmapped (slot -1,
    so every workgroup returns before its weights, the publisher included) the call is
    flagged and the published routing and grouping still equal the oracle's."""
    import torch
    lay = olmoe_packed
    s = lay.shape
    x_bits = lay.syn.x(T, stream=500 + T)
    x = to_dev_bf16(x_bits)
    base = exm.moe_layer(x, lay.wr, lay.bank, s.I, s.k)
    torch.cuda.synchronize()
    logits = oracle.router_logits(x_bits, lay.wr_bits)
    ids = oracle.topk_ids(logits, s.k)
    w = oracle.topk_weights(logits, ids)
    off, sf, fs = oracle.group_tokens(ids, s.E)
    perm = np.random.default_rng(5).permutation(s.E).astype(np.int32)   # expert e in slot perm[e]
    blobs = [None] * s.E
    for e in range(s.E):
        blobs[perm[e]] = lay.blobs[e]
    bank = exm.bank_from_blobs(blobs)
    bank.expert_to_slot = torch.from_numpy(perm).cuda()
    out = exm.moe_layer(x, lay.wr, bank, s.I, s.k)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_dev_to_bits(out.y), bf16_dev_to_bits(base.y))
    assert exm.workspace_flags(out.workspace) == 0
    bank.expert_to_slot = torch.full((s.E,), -1, dtype=torch.int32, device="cuda")
    gone = exm.moe_layer(x, lay.wr, bank, s.I, s.k)
    torch.cuda.synchronize()
    assert exm.workspace_flags(gone.workspace) & exm.FLAG_EXPERT_WITHOUT_SLOT
    for got in (out, gone):
        assert np.array_equal(got.ids.cpu().numpy(), ids)
        np.testing.assert_allclose(got.weights.cpu().numpy(), w, rtol=0, atol=1e-6)
        assert np.array_equal(got.offsets.cpu().numpy(), off)
        assert np.array_equal(got.sorted_flat.cpu().numpy()[:T * s.k], sf)
        assert np.array_equal(got.flat_to_sorted.cpu().numpy()[:T * s.k], fs)


@pytest.mark.parametrize("shape,T", [("olmoe", 100), ("olmoe", 300), ("wide", 100), ("wide", 200)])
def test_prefill_layer_seeds_equal_separate_calls(exm, olmoe_packed, shape, T):
    """At prefill sizes the whole-layer call takes the grouped GEMM's correction seeds from
    the routing kernel (the vector kernel up to 128 tokens, in one pass of loads at hidden
    2048 and in several at 4096; the fp64 matrix-core kernel above), the separate forward
    call from a kernel of its own; both sum in one order, so the outputs are equal bit for
    bit, and the layer call meets the oracle."""
    import torch
    if shape == "olmoe":
        lay = olmoe_packed
    else:
        lay = Layer(LayerShape(H=4096, I=256, E=8, k=2), seed=31)
    s = lay.shape
    assert T * s.k > 10 * min(s.E, T * s.k), "a grouped-GEMM size"
    x_bits = lay.syn.x(T, stream=400 + T)
    x = to_dev_bf16(x_bits)
    out = exm.moe_layer(x, lay.wr, lay.bank, s.I, s.k)
    y_sep = exm.moe_forward(x, out.ids, out.weights, out.offsets, out.sorted_flat, out.flat_to_sorted, lay.bank, s.I)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_dev_to_bits(out.y), bf16_dev_to_bits(y_sep))
    ids = oracle.topk_ids(oracle.router_logits(x_bits, lay.wr_bits), s.k)
    assert np.array_equal(out.ids.cpu().numpy(), ids)
    if shape == "wide":   # small enough for the oracle on every token
        ref = oracle.moe_layer(x_bits, lay.wr_bits, lay.experts, s.k)
        check_y(bf16_dev_to_f64(out.y), ref["y"], f"wide T={T}")


def test_slotless_expert_leaves_workspace_clean(exm, olmoe_packed):
    """A routed expert without a slot in a whole-layer call: flagged, its tokens' outputs
    are undefined, and the workspace's persistent state (arrival counters, flag word once
    read) is left clean: the next call on the same workspace equals a call on a fresh one
    bit for bit."""
    import torch
    lay = olmoe_packed
    s = lay.shape
    x = to_dev_bf16(lay.syn.x(16, stream=400))
    ref = exm.moe_layer(x, lay.wr, lay.bank, s.I, s.k)
    torch.cuda.synchronize()
    gone = int(ref.ids[3, 0])
    table = torch.arange(s.E, dtype=torch.int32, device="cuda")
    table[gone] = -1
    holed = exm.ExpertBank(base=lay.bank.base, stride=lay.bank.stride, expert_to_slot=table)
    b = exm.LayerBuffers(16, s.H, s.I, s.E, s.k)
    exm.moe_layer(x, lay.wr, holed, s.I, s.k, buffers=b)
    assert exm.workspace_flags(b.workspace) == exm.FLAG_EXPERT_WITHOUT_SLOT
    exm.moe_layer(x, lay.wr, lay.bank, s.I, s.k, buffers=b)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_dev_to_bits(b.y), bf16_dev_to_bits(ref.y))
    assert exm.workspace_flags(b.workspace) == 0


def test_sequential_path_row_counts_at_the_crossover(exm):
    """The sequential path on constructed routing whose segments sit at the boundary between
    its two launch pairs: an expert with exactly 16 rows (the last size the short-chain
    pair takes), one with 17 (the decode kernel pair), one with a single row and one with
    none, on a shape whose short-chain launches put several waves on every row block
    (H = 1024: 8 input groups for gate/up; I = 512: 4 for down). The output against the
    oracle's per-token layer with the same ids and weights, the exactness counters against
    the segment sizes, and a repeated call bit for bit."""
    import torch
    shape = LayerShape(H=1024, I=512, E=8, k=4)
    lay = Layer(shape, seed=41)
    T, k, E = 20, shape.k, shape.E
    ids_np = np.zeros((T, k), np.int64)
    fill = [3, 4, 5, 6]
    for t in range(T):
        row = []
        if t < 16:
            row.append(0)
        if t < 17:
            row.append(1)
        if t == 19:
            row.append(2)
        j = t
        while len(row) < k:
            e = fill[j % len(fill)]
            if e not in row:
                row.append(e)
            j += 1
        ids_np[t] = row
    counts = np.bincount(ids_np.reshape(-1), minlength=E)
    assert counts[0] == 16 and counts[1] == 17 and counts[2] == 1 and counts[7] == 0
    rng = np.random.default_rng(7)
    w_np = rng.random((T, k)).astype(np.float32) + 0.1
    w_np /= w_np.sum(axis=1, keepdims=True)
    x_bits = lay.syn.x(T, stream=77)
    x = to_dev_bf16(x_bits)
    ids = torch.from_numpy(ids_np.astype(np.int32)).cuda()
    w = torch.from_numpy(w_np).cuda()
    off, sf, fs = exm.group_tokens(ids, E)
    ws = exm.alloc_workspace(exm.moe_workspace_bytes(T, shape.H, shape.I, E, k, 3))
    y = exm.moe_forward(x, ids, w, off, sf, fs, lay.bank, shape.I, flags=3 | exm.DEBUG_COUNTERS, workspace=ws)
    torch.cuda.synchronize()
    y_bits = bf16_dev_to_bits(y)
    assert np.array_equal(exm.workspace_rows(ws, E), counts)
    assert exm.workspace_flags(ws) == 0
    xf = bf16_bits_to_f64(x_bits)
    y_ref = oracle.forward_per_token(xf, ids_np, w_np.astype(np.float64), lay.experts)
    check_y(bf16_dev_to_f64(y), y_ref, "sequential at the 16/17-row crossover")
    again = exm.moe_forward(x, ids, w, off, sf, fs, lay.bank, shape.I, flags=3, workspace=ws)
    torch.cuda.synchronize()
    assert np.array_equal(bf16_dev_to_bits(again), y_bits)
