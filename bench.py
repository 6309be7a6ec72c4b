#!/usr/bin/env python3
"""Benchmark of the fused grouped W4A16 MoE expert layer on one MI355X.

One step = one whole MoE layer call through the C ABI (router logits, top-k, grouping,
gate/up + SiLU*up, down + routing weight, combine) on one batch of synthetic tokens,
with the packed experts resident in HBM. Default workload: the OLMoE-shaped decode layer
(hidden 2048, 64 experts, top-8, intermediate 1024, int4 group-128) at 16 tokens per
call; 8 copies of the layer's expert bank at distinct addresses (1.66 GB) and 64 token
batches are rotated so consecutive calls neither hit the 256 MB Infinity Cache nor reuse
a routing. Steps are captured in one HIP graph and replayed.

Prints one JSON line: tokens/s, the dominant kernel's roofline figure (algorithmic bytes
per launch over its average launch time, timed with HIP events around each launch on
its stream) and the CPU oracle's rate on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import statistics
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
METRIC = "MoE-layer tokens/s on 1 MI355X; % HBM BW (decode) / % bf16 MFMA (prefill)"
# The expert kernel each OLMoE-shaped decode size launches (kernel-trace name and grid).
DECODE_KERNEL = {1: ("decode_narrow_kernel<3>", "257x1x1 wg1024"),
                 4: ("decode_fused_kernel<3, false, 8>", "257x1x1 wg512"),
                 16: ("decode_fused_kernel<3, true, 16>", "257x1x1 wg1024")}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def to_dev_bf16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--tokens", type=int, default=16, choices=[1, 4, 16], help="tokens per decode call")
    ap.add_argument("--rotate", type=int, default=8, help="expert-bank copies rotated across calls")
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-secondary", action="store_true", help="skip the other decode sizes and the prefill lines")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--only", choices=["decode", "prefill", "large", "cache", "prefill_cache", "bf16", "batched", "blas"],
                    default=None,
                    help="run a single workload (for profiling)")
    ap.add_argument("--prefill-tokens", type=int, nargs="+", default=[128, 512, 2048],
                    help="token counts of the Zipf-biased OLMoE-shaped prefill lines")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="first run a plain device copy of this many MiB three times (traffic-counter calibration)")
    return ap.parse_args()


# ----------------------------------------------------------------------------- workloads
class Workload:
    def __init__(self, name, shape, T, layer, banks, xs, bias=None):
        self.name, self.shape, self.T, self.layer, self.banks, self.xs, self.bias = name, shape, T, layer, banks, xs, bias


def build_olmoe(exm, torch, rotate):
    from synthetic import SyntheticLayer, OLMOE
    lay = SyntheticLayer(OLMOE, seed=0)
    t0 = time.time()
    blobs = [None] * OLMOE.E
    from concurrent.futures import ThreadPoolExecutor

    def one(e):
        return e, exm.quantize_pack(*lay.expert(e))

    with ThreadPoolExecutor(8) as ex:
        for e, b in ex.map(one, range(OLMOE.E)):
            blobs[e] = b
    bank0 = exm.bank_from_blobs(blobs)
    banks = [bank0] + [exm.ExpertBank(base=bank0.base.clone(), stride=bank0.stride) for _ in range(rotate - 1)]
    torch.cuda.synchronize()
    log(f"built OLMoE-shaped layer: {rotate} bank copies of {bank0.base.numel() / 1e6:.1f} MB in {time.time() - t0:.1f}s")
    return lay, banks, blobs


def bytes_per_call(exm, torch, lay_syn, shape, wr, xs_dev, T, bias=None):
    """Distinct experts of each x batch (from a routing pass) -> algorithmic HBM bytes."""
    D = []
    for x in xs_dev:
        _, ids, _ = exm.route_topk(x, wr, shape.k, bias=bias)
        D.append(len(np.unique(ids.cpu().numpy())))
    return np.array(D)


SPAN_KERNELS = ("decode_gateup", "decode_down", "decode_fused", "combine", "prefill_gateup", "prefill_down",
                "bf16_decode_gateup", "bf16_decode_down", "bf16_prefill_gateup", "bf16_prefill_down")


def time_layer(exm, torch, wl, steps, warmup, use_graph, flags=0, spans=None, replays=1, per_replay=None):
    """Milliseconds per layer call over `steps` calls (one graph replay, or eager calls);
    with replays > 1 the graph is replayed that many times and the median per-call time is
    returned (per_replay, a list, receives every replay's figure). With a dict in `spans`,
    the expert-layer kernels of the first timed replay stamp their launch spans in-kernel,
    and spans[name] = (average microseconds, launches)."""
    shape = wl.shape
    bufs = exm.LayerBuffers(wl.T, shape.H, shape.I, shape.E, shape.k, flags)
    wr = wl.layer["wr"]

    def step(i):
        exm.moe_layer(wl.xs[i % len(wl.xs)], wr, wl.banks[i % len(wl.banks)], shape.I, shape.k, bias=wl.bias,
                      flags=flags, buffers=bufs)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    if spans is not None:
        exm.span_enable(steps * 8)   # slots for the launches below (captured or eager)
    graph = None
    if use_graph:
        graph = torch.cuda.CUDAGraph()
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            with torch.cuda.graph(graph, stream=s):
                for i in range(steps):
                    step(i)
        torch.cuda.current_stream().wait_stream(s)
        graph.replay()          # warm replay
        torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    if spans is not None:
        exm.span_clear()
    times = []
    for r in range(replays if graph is not None else 1):
        e0.record()
        if graph is not None:
            graph.replay()
        else:
            for i in range(steps):
                step(i)
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1))
        if r == 0 and spans is not None:
            # the first timed pass's spans (later replays keep stamping the same slots, so
            # the slots stay allocated until the last replay has finished)
            for n in SPAN_KERNELS:
                us, cnt = exm.span_read(n)
                if cnt:
                    spans[n] = (us / cnt, cnt)
    if spans is not None:
        torch.cuda.synchronize()
        exm.span_enable(0)
    ms = float(np.median(times))
    if per_replay is not None:
        per_replay.extend(t / steps for t in times)
    return ms / steps


def kernel_times(exm, torch, wl, steps, names, warm=None):
    """Average launch time of each named kernel: HIP events around every launch. The GPU
    first spins for a while on the same stream, so that the host has queued the launches
    before they run and they execute back to back, as in the timed graph replay (a start
    event recorded while the GPU waits for the host would count that wait); `warm`
    unrecorded calls run first in the same back-to-back stream (the first launches after
    an idle GPU run slower, at clocks still ramping up)."""
    shape = wl.shape
    bufs = exm.LayerBuffers(wl.T, shape.H, shape.I, shape.E, shape.k)
    wr = wl.layer["wr"]
    exm.moe_layer(wl.xs[0], wr, wl.banks[0], shape.I, shape.k, bias=wl.bias, buffers=bufs)   # warm
    torch.cuda.synchronize()
    exm.profile_reset()
    torch.cuda._sleep(int(2.0e9 * 0.05))   # ~50 ms of spinning at ~2 GHz
    for i in range(steps // 4 if warm is None else warm):
        exm.moe_layer(wl.xs[i % len(wl.xs)], wr, wl.banks[i % len(wl.banks)], shape.I, shape.k, bias=wl.bias,
                      buffers=bufs)
    exm.profile_enable(True)
    for i in range(steps):
        exm.moe_layer(wl.xs[i % len(wl.xs)], wr, wl.banks[i % len(wl.banks)], shape.I, shape.k, bias=wl.bias,
                      buffers=bufs)
    torch.cuda.synchronize()
    out = {}
    for n in names:
        ms, cnt = exm.profile_read(n)
        if cnt:
            out[n] = (ms / cnt, cnt)
    exm.profile_enable(False)
    exm.profile_reset()
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(lay_syn, shape, T, seconds, n_batches=64, extra=True):
    """The CPU oracle as it stands, on successive fresh batches of the same workload, until
    `seconds` of CPU work have run (dequantization of the used experts included). With
    `extra`, two single-thread samples extrapolated to the prefill workloads: the first 64
    tokens of the Zipf-biased 2048-token OLMoE batch through the whole oracle layer, and
    8 routed rows through one large expert (hidden 4096, intermediate 14336) with that
    expert's dequantization timed separately."""
    import oracle
    from threadpoolctl import threadpool_info, threadpool_limits
    wr = lay_syn.router()
    t0 = time.time()
    qexp = [oracle.quantize_expert(*lay_syn.expert(e)) for e in range(shape.E)]
    tq = time.time() - t0
    tokens = 0
    batches = 0
    t0 = time.time()
    while True:
        for q in qexp:
            q.drop_cache()
        x = lay_syn.x(T, stream=1000 + batches)
        oracle.moe_layer(x, wr, qexp, shape.k)
        tokens += T
        batches += 1
        el = time.time() - t0
        if el >= seconds or batches >= n_batches:
            break
    threads = max([d.get("num_threads", 1) for d in threadpool_info() if d.get("user_api") == "blas"] + [1])
    out = {"value": tokens / el, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
           "sample": f"{batches} fresh {T}-token batches of the OLMoE-shaped decode layer through the fp64 "
                     f"oracle (per-token expert MLPs, dequantization of the routed experts included; "
                     f"{el:.1f}s; quantization {tq:.1f}s not counted)",
           "host_cpus": len(os.sched_getaffinity(0)), "cpu_model": cpu_model(),
           "threads_note": "cores = the BLAS thread pool the oracle's matrix products ran on"}
    if not extra:
        return out
    from synthetic import LARGE, SyntheticLayer
    per = {}
    with threadpool_limits(1):
        for q in qexp:
            q.drop_cache()
        x = lay_syn.x(2048)[:64]
        t0 = time.time()
        oracle.moe_layer(x, wr, qexp, shape.k, bias=lay_syn.zipf_bias())
        t64 = time.time() - t0
        per["olmoe_prefill_zipf_T2048"] = {
            "tokens_per_s": 64 / t64, "threads": 1, "extrapolated": True,
            "layer_s_extrapolated": t64 * 2048 / 64,
            "sample": f"first 64 of the 2048 Zipf-biased tokens through the oracle layer in {t64:.2f}s "
                      "(routed experts dequantized inside; linear in tokens, so an upper bound on the time)"}
        for q in qexp:
            q.drop_cache()
        syn = SyntheticLayer(LARGE, seed=0)
        qe = oracle.quantize_expert(*syn.expert(0))
        t0 = time.time()
        qe.deq()
        tdeq = time.time() - t0
        xl = oracle.bf16_bits_to_f64(syn.x(8))
        t0 = time.time()
        oracle.expert_mlp(qe, xl)
        trow = (time.time() - t0) / 8
        qe.drop_cache()
        rows = 4096 * LARGE.k
        layer_s = LARGE.E * tdeq + rows * trow
        per["large_prefill_T4096"] = {
            "tokens_per_s": 4096 / layer_s, "threads": 1, "extrapolated": True, "layer_s_extrapolated": layer_s,
            "sample": f"expert 0: dequantization {tdeq:.2f}s, 8 routed rows {8 * trow:.2f}s; layer = 8 experts' "
                      f"dequantization + {rows} rows"}
    out["per_config"] = per
    return out


def run_blas_reference(torch, reps=20):
    """Context for the MFMA fractions: the installed BLAS (torch.matmul on bf16, i.e.
    hipBLASLt) on dense bf16 GEMMs of the per-expert shapes of the large-expert prefill
    layer (1024 tokens per expert: gate and up together, then down) and of a large square
    GEMM. Not part of the layer: it shows what a dense bf16 GEMM reaches on this GPU."""
    from synthetic import LARGE
    shapes = {"large_expert_gateup_1024x28672x4096": (1024, 2 * LARGE.I, LARGE.H),
              "large_expert_down_1024x4096x14336": (1024, LARGE.H, LARGE.I),
              "square_8192x8192x8192": (8192, 8192, 8192)}
    out = {}
    g = torch.Generator(device="cuda").manual_seed(0)
    for name, (M, N, K) in shapes.items():
        a = torch.randn(M, K, device="cuda", dtype=torch.bfloat16, generator=g)
        b = torch.randn(K, N, device="cuda", dtype=torch.bfloat16, generator=g)
        for _ in range(3):
            torch.matmul(a, b)
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(reps):
            ev0.record()
            torch.matmul(a, b)
            ev1.record()
            ev1.synchronize()
            ts.append(ev0.elapsed_time(ev1) * 1e-3)
        t = statistics.median(ts)
        tf = 2.0 * M * N * K / t / 1e12
        out[name] = {"us": t * 1e6, "tflops": tf, "mfma_frac": tf / BF16_PEAK_TFLOPS}
        log(f"blas dense bf16 {name}: {t * 1e6:.1f} us, {tf:.0f} TFLOP/s ({100 * tf / BF16_PEAK_TFLOPS:.1f}% of bf16 MFMA)")
        del a, b
    return out


def prefill_roofline(rec, read_kernel_avg):
    """The large-expert prefill layer (hidden 4096, intermediate 14336, 8 experts, top-2,
    4096 tokens) against the dense bf16 MFMA peak: expert FLOPs 6 T k H I per layer call
    over the median graph-replayed layer time; the two grouped GEMM kernels also by their
    event-timed launches and by the committed rocprofv3 trace of the same workload."""
    if not rec:
        return None
    T, k, H, I = 4096, 2, 4096, 14336
    flops = 6.0 * T * k * H * I
    out = {"bound": "mfma", "achieved": rec["layer_tflops"], "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
           "frac": rec["layer_mfma_frac"], "traffic": None, "workload": "large_prefill_T4096",
           "flops_per_layer": flops, "ms_per_layer": rec["ms_per_layer"],
           "ms_per_layer_is": f"median of {rec['layer_ms_median_of']} graph replays of 10 layer calls",
           "gemm_pair_ms_events": rec.get("gemm_pair_ms"), "gemm_pair_frac_events": rec.get("gemm_pair_mfma_frac"),
           "gateup_frac_events": rec.get("gateup_mfma_frac"), "down_frac_events": rec.get("down_mfma_frac")}
    path = os.path.join(ROOT, "profiles", "kernel_trace_large_prefill_T4096.txt")
    gu = read_kernel_avg(path, "prefill_kernel<true, 4, 64, true>", "15232x1x1 wg256")
    dn = read_kernel_avg(path, "prefill_kernel<false, 4, 64, true>", "2176x1x1 wg256")
    if gu and dn:
        out["gemm_pair_ms_rocprof_median"] = (gu[1] + dn[1]) * 1e-3
        out["gemm_pair_frac_rocprof_median"] = flops / ((gu[1] + dn[1]) * 1e-6) / 1e12 / BF16_PEAK_TFLOPS
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the layer is not sharded across GPUs "
                                   "(sharded, each GPU would hold E/G experts and trade token rows all-to-all)",
                          "n_gpus": args.gpus}))
        sys.exit(2)
    import torch
    import w4a16_mixture_experts_amd as exm
    from rocprof_summary import read_traffic, read_kernel_avg
    from synthetic import OLMOE, LARGE, SyntheticLayer
    assert torch.cuda.is_available(), "bench.py needs a GPU"

    H, I, E, k = OLMOE.H, OLMOE.I, OLMOE.E, OLMOE.k
    expert_bytes = exm.packed_expert_bytes(H, I)
    gu_bytes = 2 * (I // 16) * (H // 128) * 1056
    down_bytes = (H // 16) * (I // 128) * 1056
    result = {}
    secondary = {}
    use_graph = not args.no_graph

    olmoe_syn = banks = None
    if args.calib_copy_mib:
        nb = args.calib_copy_mib << 20
        src = torch.empty(nb, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        src.fill_(1)
        for _ in range(3):
            exm.device_copy(dst, src)
        torch.cuda.synchronize()
        log(f"calibration copy: 3 x {nb} bytes")
        del src, dst

    if args.only in (None, "decode", "prefill", "cache", "prefill_cache", "bf16", "batched"):
        olmoe_syn, banks, olmoe_blobs = build_olmoe(exm, torch, args.rotate)
        wr = to_dev_bf16(olmoe_syn.router())

    # ------------------------------------------------------------------ decode (headline)
    def run_decode(T, steps, warmup, want_kernels):
        xs = [to_dev_bf16(olmoe_syn.x(T, stream=s)) for s in range(64)]
        wl = Workload(f"olmoe_decode_T{T}", OLMOE, T, {"wr": wr}, banks, xs)
        D = bytes_per_call(exm, torch, olmoe_syn, OLMOE, wr, xs, T)
        spans = {}
        ms = time_layer(exm, torch, wl, steps, warmup, use_graph, spans=spans)
        layer_bytes = D.mean() * expert_bytes + E * H * 2 + 2 * T * H * 2 + T * k * 8
        rec = {"T": T, "tokens_per_s": T / (ms * 1e-3), "us_per_layer": ms * 1e3,
               "distinct_experts_mean": float(D.mean()),
               "layer_hbm_gbs": layer_bytes / (ms * 1e-3) / 1e9,
               "layer_hbm_frac": layer_bytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBS}
        if want_kernels:
            kt = kernel_times(exm, torch, wl, max(steps, 128),
                              ["route_logits", "route_token", "route_sel", "topk", "group", "topk_group", "decode_gateup", "decode_down",
                               "decode_fused", "combine"])
            rec["kernel_us"] = {n: v[0] * 1e3 for n, v in kt.items()}
            rec["kernel_span_us"] = {n: v[0] for n, v in spans.items()}
            # The dominant kernel and its bytes per launch as the work unit defines them: the
            # packed weights and scales of every distinct routed expert once, the tokens' x
            # in, their y out, and the ids and routing weights (what the layer must move,
            # less the router matrix, which the routing kernel reads). Its duration: HIP
            # events around each of its launches on its stream (the dispatch-to-completion
            # interval a rocprofv3 kernel trace reports), over back-to-back calls of the
            # same rotated workload as the timed replay.
            kname, grid = DECODE_KERNEL[T] if T in DECODE_KERNEL else (None, None)
            alg = D.mean() * expert_bytes + 2 * T * H * 2 + T * k * 8
            if "decode_fused" in kt:
                ev_us, span = kt["decode_fused"][0] * 1e3, spans.get("decode_fused")
            else:
                kname, grid = "decode_expert_kernel", None
                ev_us, span = kt["decode_gateup"][0] * 1e3 + kt["decode_down"][0] * 1e3, None
            base = kname.split("<")[0]
            tr = read_traffic(os.path.join(ROOT, "profiles", f"traffic_{base.replace('_kernel', '')}_olmoe_decode_T{T}.txt"),
                              base)
            prof = read_kernel_avg(os.path.join(ROOT, "profiles", "kernel_trace_olmoe_decode.txt"), kname, grid) \
                if grid else None
            rec["roofline"] = {"bound": "hbm", "achieved": alg / (ev_us * 1e-6) / 1e9, "peak": HBM_PEAK_GBS,
                               "unit": "GB/s", "frac": alg / (ev_us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                               "traffic": None if tr is None else tr["bytes"], "kernel": kname,
                               "algorithmic_bytes_per_launch": alg, "avg_launch_us": ev_us,
                               "duration_source": "HIP events around each launch (hipExtLaunchKernelGGL), "
                                                  f"{kt.get('decode_fused', (0, 0))[1]} back-to-back launches",
                               "span_avg_launch_us": None if span is None else span[0]}
            if prof is not None:
                # the same kernel in the committed rocprofv3 trace of this workload: its
                # median launch (warm-up launches aside) and the fraction it gives
                rec["roofline"]["rocprof_avg_launch_us"] = prof[0]
                rec["roofline"]["rocprof_median_launch_us"] = prof[1]
                rec["roofline"]["frac_at_rocprof_median"] = alg / (prof[1] * 1e-6) / 1e9 / HBM_PEAK_GBS
            if tr is not None:
                rec["roofline"]["traffic_over_algorithmic"] = tr["bytes"] / alg
        log(f"decode T={T}: {rec['tokens_per_s']:.0f} tok/s, {rec['us_per_layer']:.2f} us/layer, "
            f"layer {rec['layer_hbm_gbs']:.0f} GB/s ({rec['layer_hbm_frac'] * 100:.1f}% of HBM)")
        return rec

    def run_sequential(T, steps, warmup):
        """Fused layer vs the per-expert sequential W4 path, both launched eagerly (the
        sequential path reads the segment offsets back to the host, so it cannot be captured)."""
        xs = [to_dev_bf16(olmoe_syn.x(T, stream=s)) for s in range(64)]
        wl = Workload(f"olmoe_decode_T{T}", OLMOE, T, {"wr": wr}, banks, xs)
        fused = time_layer(exm, torch, wl, steps, warmup, False)
        seq = time_layer(exm, torch, wl, steps, warmup, False, flags=exm.PATH_SEQUENTIAL)
        log(f"decode T={T} eager: fused {fused * 1e3:.1f} us, sequential {seq * 1e3:.1f} us, ratio {seq / fused:.2f}")
        return {"T": T, "fused_eager_us": fused * 1e3, "sequential_eager_us": seq * 1e3,
                "fused_over_sequential_speedup": seq / fused}

    if args.only in (None, "decode"):
        head = run_decode(args.tokens, args.steps, args.warmup, True)
        result["head"] = head
        if not args.no_secondary:
            secondary["olmoe_decode_T16_fused_vs_sequential"] = run_sequential(16, 64, 8)
        if not args.no_secondary:
            for T in (1, 4, 16):
                if T != args.tokens:
                    secondary[f"olmoe_decode_T{T}"] = run_decode(T, args.steps, args.warmup, True)

    # ------------------------------------------------------------------ slot cache (decode through 16 layers)
    def run_slot_cache(slots_list, layers=16, steps=128):
        """Batch-1 decode through a stack of `layers` OLMoE-shaped layers whose experts sit in a
        pinned host pool behind `slots` GPU slots per layer (LRU). The routing of each
        (step, layer) comes from a Zipf(1.1) popularity trace with temporal reuse 0.5; the
        first `steps` steps of the trace warm the cache, the next `steps` are timed. Every
        layer shares one set of expert values (values do not change bytes moved or time);
        the routing differs per layer."""
        from synthetic import slot_cache_trace
        trace = slot_cache_trace(E, k, layers, 2 * steps, seed=0)
        ids_dev = torch.from_numpy(trace.reshape(2 * steps, layers, 1, k)).cuda()
        xs = [to_dev_bf16(olmoe_syn.x(1, stream=5000 + st)) for st in range(2 * steps)]
        # pinned-host -> device copy rate of one packed expert, for reference
        pin = torch.empty(expert_bytes, dtype=torch.uint8).pin_memory()
        dev = torch.empty(expert_bytes, dtype=torch.uint8, device="cuda")
        for _ in range(4):
            dev.copy_(pin, non_blocking=True)
        torch.cuda.synchronize()
        t0 = time.time()
        for _ in range(64):
            dev.copy_(pin, non_blocking=True)
        torch.cuda.synchronize()
        h2d_gbs = 64 * expert_bytes / (time.time() - t0) / 1e9
        del pin, dev
        out = {}
        for S in slots_list:
            cache = exm.SlotCache(layers, E, S, expert_bytes)
            for l in range(layers):
                for e in range(E):
                    cache.fill(l, e, olmoe_blobs[e])
            if S == E:
                cache.preload()

            b = exm.LayerBuffers(1, H, I, E, k)
            ws = exm.alloc_workspace(exm.moe_workspace_bytes(1, H, I, E, k))

            def run(lo, hi):
                # preallocated buffers; per layer: logits, weights of the trace's ids,
                # grouping, the active set read back from the GPU's grouping (the
                # reactive cache's one host synchronization per layer), then acquire +
                # experts + combine in one library call
                for st in range(lo, hi):
                    x = xs[st]
                    for l in range(layers):
                        ids = ids_dev[st, l]
                        exm.route_topk(x, wr, k, logits=b.logits, ids=b.ids, weights=b.weights)
                        exm.route_weights(b.logits, ids, weights=b.weights)
                        exm.group_tokens(ids, E, b.offsets, b.sorted_flat, b.flat_to_sorted)
                        active = exm.active_experts(b.offsets)
                        exm.moe_forward_cached(x, ids, b.weights, b.offsets, b.sorted_flat, b.flat_to_sorted, cache,
                                               l, active, I, y=b.y, workspace=ws)

            cache.reset_stats()
            torch.cuda.synchronize()
            t0 = time.time()
            run(0, steps)
            torch.cuda.synchronize()
            cold_s = time.time() - t0
            cold = cache.stats()
            cache.reset_stats()
            t0 = time.time()
            run(steps, 2 * steps)
            torch.cuda.synchronize()
            warm_s = time.time() - t0
            st = cache.stats()
            cache.close()
            rec = {"slots": S, "layers": layers, "steps": steps, "tokens_per_s": steps / warm_s,
                   "ms_per_token": warm_s / steps * 1e3, "resident": bool(st["resident"]),
                   "lookups": st["lookups"], "hits": st["hits"], "misses": st["misses"],
                   "evictions": st["evictions"], "hit_rate": st["hits"] / max(st["lookups"], 1),
                   "h2d_bytes": st["h2d_bytes"], "h2d_gb_per_token": st["h2d_bytes"] / steps / 1e9,
                   "h2d_gbs_achieved": st["h2d_bytes"] / warm_s / 1e9, "h2d_gbs_pinned_copy": h2d_gbs,
                   "device_bytes": st["device_bytes"], "pinned_host_bytes": st["pinned_host_bytes"],
                   "cold": {"tokens_per_s": steps / cold_s, "hit_rate": cold["hits"] / max(cold["lookups"], 1),
                            "misses": cold["misses"], "h2d_bytes": cold["h2d_bytes"]}}
            log(f"slot cache S={S}: {rec['tokens_per_s']:.1f} tok/s through {layers} layers, hit rate "
                f"{rec['hit_rate'] * 100:.1f}%, H2D {st['h2d_bytes'] / 1e9:.2f} GB over {steps} steps")
            out[f"slot_cache_S{S}"] = rec
        return out

    if not args.no_secondary and args.only in (None, "cache"):
        secondary.update(run_slot_cache([8, 16, 32, 64]))

    # ------------------------------------------------------------------ bf16 comparator
    bf16_banks = []

    def build_bf16_banks(copies=2):
        """The same 64 experts with bf16 weights (the comparator), 805 MB per copy."""
        if bf16_banks:
            return bf16_banks
        from synthetic import f32_to_bf16_bits
        from concurrent.futures import ThreadPoolExecutor
        t0 = time.time()

        def one(e):
            return exm.bf16_pack(*[f32_to_bf16_bits(w) for w in olmoe_syn.expert(e)])

        with ThreadPoolExecutor(8) as ex:
            blobs = list(ex.map(one, range(E)))
        b0 = exm.bank_from_blobs(blobs)
        del blobs
        bf16_banks.append(b0)
        for _ in range(copies - 1):
            bf16_banks.append(exm.ExpertBank(base=b0.base.clone(), stride=b0.stride))
        torch.cuda.synchronize()
        log(f"built the bf16 comparator bank: {copies} copies of {b0.base.numel() / 1e6:.1f} MB in {time.time() - t0:.1f}s")
        return bf16_banks

    def run_bf16_comparator(decode_T=(1, 4, 16), prefill_T=(512, 2048), steps=200, warmup=20):
        """The layer with dense bf16 experts (same routing, grouping and combine) against the
        int4 layer, timed the same way, back to back: the layer-level W4A16 / BF16 ratio."""
        bb = build_bf16_banks()
        bf16_bytes = exm.bf16_expert_bytes(H, I)
        out = {}
        for T in decode_T:
            xs = [to_dev_bf16(olmoe_syn.x(T, stream=s)) for s in range(64)]
            D = bytes_per_call(exm, torch, olmoe_syn, OLMOE, wr, xs, T).mean()
            w4 = time_layer(exm, torch, Workload(f"olmoe_decode_T{T}", OLMOE, T, {"wr": wr}, banks, xs), steps, warmup,
                            use_graph)
            spans = {}
            bf = time_layer(exm, torch, Workload(f"olmoe_decode_T{T}_bf16", OLMOE, T, {"wr": wr}, bb, xs), steps,
                            warmup, use_graph, flags=exm.WEIGHTS_BF16, spans=spans)
            rec = {"T": T, "w4a16_us_per_layer": w4 * 1e3, "bf16_us_per_layer": bf * 1e3,
                   "w4a16_over_bf16_speedup": bf / w4, "distinct_experts_mean": float(D),
                   "bf16_kernel_span_us": {n: v[0] for n, v in spans.items()}}
            if "bf16_decode_gateup" in spans and "bf16_decode_down" in spans:
                us = spans["bf16_decode_gateup"][0] + spans["bf16_decode_down"][0]
                alg = D * bf16_bytes + T * H * 2 + T * k * H * 4
                rec["bf16_expert_kernels_gbs"] = alg / (us * 1e-6) / 1e9
                rec["bf16_expert_kernels_hbm_frac"] = rec["bf16_expert_kernels_gbs"] / HBM_PEAK_GBS
            log(f"bf16 comparator decode T={T}: bf16 {bf * 1e3:.1f} us vs w4a16 {w4 * 1e3:.1f} us per layer "
                f"({bf / w4:.2f}x)" + (f", bf16 expert kernels {rec['bf16_expert_kernels_gbs']:.0f} GB/s"
                                        if "bf16_expert_kernels_gbs" in rec else ""))
            out[f"bf16_vs_w4a16_decode_T{T}"] = rec
        bias = torch.from_numpy(olmoe_syn.zipf_bias()).cuda()
        for T in prefill_T:
            xs = [to_dev_bf16(olmoe_syn.x(T, stream=s)) for s in range(4)]
            w4 = time_layer(exm, torch, Workload(f"olmoe_prefill_T{T}", OLMOE, T, {"wr": wr}, banks[:2], xs, bias),
                            20, 3, use_graph)
            spans = {}
            bf = time_layer(exm, torch, Workload(f"olmoe_prefill_T{T}_bf16", OLMOE, T, {"wr": wr}, bb, xs, bias),
                            20, 3, use_graph, flags=exm.WEIGHTS_BF16, spans=spans)
            flops = 6.0 * T * k * H * I
            rec = {"T": T, "w4a16_ms_per_layer": w4, "bf16_ms_per_layer": bf, "w4a16_over_bf16_speedup": bf / w4,
                   "bf16_layer_tflops": flops / (bf * 1e-3) / 1e12,
                   "bf16_kernel_span_us": {n: v[0] for n, v in spans.items()}}
            log(f"bf16 comparator prefill T={T}: bf16 {bf:.3f} ms vs w4a16 {w4:.3f} ms per layer ({bf / w4:.2f}x)")
            out[f"bf16_vs_w4a16_prefill_zipf_T{T}"] = rec
        return out

    if not args.no_secondary and args.only in (None, "bf16"):
        secondary.update(run_bf16_comparator())

    # ------------------------------------------------------------------ batched decode through the cache
    def run_batched_cache(batches=(1, 2, 4, 8), S=16, layers=16, steps=64):
        """Batched generation analogue: B sequences decoded together (T = B tokens per call)
        through `layers` OLMoE-shaped expert layers. The experts sit behind S slots per layer
        (the batch's distinct experts per layer run in cache-sized waves; the host drives
        every layer, since each needs its active set), or are resident (int4, and the bf16
        comparator; those steps are captured in one graph and replayed). Routing comes from a
        per-sequence trace over each layer's shared Zipf(1.1) popularity (reuse 0.5); every
        layer shares one set of expert values. The first `steps` steps warm up, the next
        `steps` are timed; tokens/s = B * steps / wall clock."""
        from synthetic import batch_trace
        Bmax = max(batches)
        trace = batch_trace(E, k, layers, 2 * steps, Bmax, seed=0)
        ids_all = torch.from_numpy(np.ascontiguousarray(trace)).cuda()          # [steps, layers, B, k]
        xs = [to_dev_bf16(olmoe_syn.x(Bmax, stream=9000 + st)) for st in range(2 * steps)]
        bank_bf = build_bf16_banks()[0]
        cache = exm.SlotCache(layers, E, S, expert_bytes)
        for l in range(layers):
            for e in range(E):
                cache.fill(l, e, olmoe_blobs[e])
        out = {}
        for B in batches:
            ws = exm.alloc_workspace(exm.moe_workspace_bytes(B, H, I, E, k))
            y = torch.empty((B, H), dtype=torch.bfloat16, device="cuda")
            lb = exm.LayerBuffers(B, H, I, E, k)
            rec = {"batch": B, "slots": S, "layers": layers, "steps": steps}
            for name in ("w4a16_S%d" % S, "w4a16_resident", "bf16_resident"):
                n_act = 0

                def run(lo, hi):
                    nonlocal n_act
                    for st in range(lo, hi):
                        x = xs[st][:B]
                        for l in range(layers):
                            ids = ids_all[st, l, :B]
                            exm.route_topk(x, wr, k, logits=lb.logits, ids=lb.ids, weights=lb.weights)
                            w = exm.route_weights(lb.logits, ids, weights=lb.weights)
                            off, sf, fs = exm.group_tokens(ids, E, lb.offsets, lb.sorted_flat, lb.flat_to_sorted)
                            if name == "bf16_resident":
                                exm.moe_forward(x, ids, w, off, sf, fs, bank_bf, I, flags=exm.WEIGHTS_BF16, y=y,
                                                workspace=ws)
                            elif name == "w4a16_resident":
                                exm.moe_forward(x, ids, w, off, sf, fs, banks[0], I, y=y, workspace=ws)
                            else:
                                active = exm.active_experts(off)   # read back from the GPU's grouping
                                n_act += len(active)
                                exm.moe_forward_cached(x, ids, w, off, sf, fs, cache, l, active, I, y=y,
                                                       workspace=ws)

                run(0, steps)
                torch.cuda.synchronize()
                graph = None
                if name != "w4a16_S%d" % S:
                    graph = torch.cuda.CUDAGraph()
                    s_ = torch.cuda.Stream()
                    s_.wait_stream(torch.cuda.current_stream())
                    with torch.cuda.stream(s_):
                        with torch.cuda.graph(graph, stream=s_):
                            run(steps, 2 * steps)
                    torch.cuda.current_stream().wait_stream(s_)
                    graph.replay()
                    torch.cuda.synchronize()
                else:
                    cache.reset_stats()
                    n_act = 0
                t0 = time.time()
                if graph is not None:
                    graph.replay()
                else:
                    run(steps, 2 * steps)
                torch.cuda.synchronize()
                dt = time.time() - t0
                del graph
                r = {"tokens_per_s": B * steps / dt, "ms_per_step": dt / steps * 1e3}
                if name == "w4a16_S%d" % S:
                    st_ = cache.stats()
                    r.update({"distinct_experts_per_layer": n_act / steps / layers,
                              "hit_rate": st_["hits"] / max(st_["lookups"], 1), "misses": st_["misses"],
                              "h2d_bytes_per_step": st_["h2d_bytes"] / steps})
                rec[name] = r
            rec["w4a16_S%d_over_bf16" % S] = rec["w4a16_S%d" % S]["tokens_per_s"] / rec["bf16_resident"]["tokens_per_s"]
            rec["w4a16_resident_over_bf16"] = rec["w4a16_resident"]["tokens_per_s"] / rec["bf16_resident"]["tokens_per_s"]
            c16 = rec["w4a16_S%d" % S]
            log(f"batched decode B={B}: S={S} {c16['tokens_per_s']:.0f} tok/s (hit {c16['hit_rate'] * 100:.1f}%, "
                f"{c16['h2d_bytes_per_step'] / 1e6:.0f} MB H2D/step, {c16['distinct_experts_per_layer']:.1f} experts/layer), "
                f"resident {rec['w4a16_resident']['tokens_per_s']:.0f}, bf16 {rec['bf16_resident']['tokens_per_s']:.0f} tok/s")
            out[f"batched_decode_B{B}"] = rec
        cache.close()
        torch.cuda.empty_cache()
        return out

    if not args.no_secondary and args.only in (None, "batched"):
        secondary.update(run_batched_cache())

    # ------------------------------------------------------------------ prefill through the slot cache
    def run_prefill_cache(slots_list, T=512, layers=16, warm=2, timed=5):
        """Time-to-first-token analogue: a T-token prompt through the expert layers of a
        `layers`-deep OLMoE-shaped stack whose experts sit in the pinned host pool behind
        `slots` GPU slots per layer. Each layer has its own seeded router and Zipf(1.1)
        logit bias (so each layer routes the prompt to its own active set); the prompt's x
        is shared by all layers; the cache is persistent-warm (the first `warm` prompts
        are untimed). Per layer: routing, grouping, the active set read back to the host,
        then the expert layer in cache-sized waves. Wall clock per prompt, median."""
        per_layer = [SyntheticLayer(OLMOE, seed=0, layer=l) for l in range(layers)]
        wrs = [to_dev_bf16(sl.router()) for sl in per_layer]
        biases = [torch.from_numpy(sl.zipf_bias()).cuda() for sl in per_layer]
        xs = [to_dev_bf16(olmoe_syn.x(T, stream=7000 + p)) for p in range(warm + timed)]
        ws = exm.alloc_workspace(exm.moe_workspace_bytes(T, H, I, E, k))
        y = torch.empty((T, H), dtype=torch.bfloat16, device="cuda")
        pin = torch.empty(expert_bytes, dtype=torch.uint8).pin_memory()
        dev = torch.empty(expert_bytes, dtype=torch.uint8, device="cuda")
        for _ in range(4):
            dev.copy_(pin, non_blocking=True)
        torch.cuda.synchronize()
        t0 = time.time()
        for _ in range(64):
            dev.copy_(pin, non_blocking=True)
        torch.cuda.synchronize()
        h2d_gbs = 64 * expert_bytes / (time.time() - t0) / 1e9
        del pin, dev
        out = {}
        for S in slots_list:
            if S == "bf16":
                # the comparator: every layer's experts resident in bf16 (one shared bank)
                bank_bf = build_bf16_banks()[0]
                n_waves = n_active = 0

                def prompt(x):
                    nonlocal n_active
                    for l in range(layers):
                        logits, ids, w = exm.route_topk(x, wrs[l], k, bias=biases[l])
                        off, sf, fs = exm.group_tokens(ids, E)
                        n_active += len(exm.active_experts(off))   # the same host read as the cached runs
                        exm.moe_forward(x, ids, w, off, sf, fs, bank_bf, I, flags=exm.WEIGHTS_BF16, y=y,
                                        workspace=ws)

                for p in range(warm):
                    prompt(xs[p])
                torch.cuda.synchronize()
                n_active = 0
                times = []
                for p in range(warm, warm + timed):
                    t0 = time.time()
                    prompt(xs[p])
                    torch.cuda.synchronize()
                    times.append(time.time() - t0)
                ms = float(np.median(times)) * 1e3
                log(f"prefill of the bf16 comparator T={T}: {ms:.2f} ms for {layers} layers (resident)")
                out[f"prefill_bf16_resident_T{T}"] = {"layers": layers, "T": T, "prompts_timed": timed,
                                                      "ms_per_prompt": ms, "ms_per_prompt_min": min(times) * 1e3,
                                                      "active_experts_per_layer": n_active / timed / layers}
                continue
            cache = exm.SlotCache(layers, E, S, expert_bytes)
            for l in range(layers):
                for e in range(E):
                    cache.fill(l, e, olmoe_blobs[e])
            if S == E:
                cache.preload()
            n_waves = 0
            n_active = 0

            def prompt(x):
                nonlocal n_waves, n_active
                for l in range(layers):
                    logits, ids, w = exm.route_topk(x, wrs[l], k, bias=biases[l])
                    off, sf, fs = exm.group_tokens(ids, E)
                    active = exm.active_experts(off)
                    n_active += len(active)
                    W = S if len(active) <= S else max(S // 2, 1)   # the library's wave size
                    n_waves += -(-len(active) // W)
                    exm.moe_forward_cached(x, ids, w, off, sf, fs, cache, l, active, I, y=y, workspace=ws)

            for p in range(warm):
                prompt(xs[p])
            torch.cuda.synchronize()
            cache.reset_stats()
            n_waves = n_active = 0
            times = []
            for p in range(warm, warm + timed):
                t0 = time.time()
                prompt(xs[p])
                torch.cuda.synchronize()
                times.append(time.time() - t0)
            st = cache.stats()
            cache.close()
            ms = float(np.median(times)) * 1e3
            h2d = st["h2d_bytes"] / timed
            rec = {"slots": S, "layers": layers, "T": T, "prompts_timed": timed, "ms_per_prompt": ms,
                   "ms_per_prompt_min": min(times) * 1e3, "resident": bool(st["resident"]),
                   "active_experts_per_layer": n_active / timed / layers, "waves_per_layer": n_waves / timed / layers,
                   "hit_rate": st["hits"] / max(st["lookups"], 1), "misses_per_prompt": st["misses"] / timed,
                   "h2d_bytes_per_prompt": h2d, "h2d_ms_at_pinned_copy_rate": h2d / (h2d_gbs * 1e9) * 1e3,
                   "h2d_gbs_pinned_copy": h2d_gbs, "device_bytes": st["device_bytes"]}
            log(f"prefill through the cache T={T} S={S}: {ms:.2f} ms for {layers} layers, "
                f"{rec['waves_per_layer']:.2f} waves/layer, hit rate {rec['hit_rate'] * 100:.1f}%, "
                f"H2D {h2d / 1e9:.2f} GB/prompt ({rec['h2d_ms_at_pinned_copy_rate']:.1f} ms at {h2d_gbs:.1f} GB/s)")
            out[f"prefill_cache_T{T}_S{S}"] = rec
        return out

    if not args.no_secondary and args.only in (None, "prefill_cache"):
        secondary.update(run_prefill_cache([8, 16, 32, 64, "bf16"]))

    # ------------------------------------------------------------------ prefill lines
    def run_prefill(name, shape, syn, banks_p, wr_p, T, bias, steps, warmup, replays=5):
        xs = [to_dev_bf16(syn.x(T, stream=s)) for s in range(4)]
        bias_t = None if bias is None else torch.from_numpy(bias).cuda()
        wl = Workload(name, shape, T, {"wr": wr_p}, banks_p, xs, bias_t)
        spans = {}
        per_replay = []
        ms = time_layer(exm, torch, wl, steps, warmup, use_graph, spans=spans, replays=replays, per_replay=per_replay)
        flops = 6.0 * T * shape.k * shape.H * shape.I
        kt = kernel_times(exm, torch, wl, 8, warm=6, names=["prefill_gateup", "prefill_down", "xsum", "combine",
                                                          "route_logits", "topk", "group", "group_scan", "group_scatter", "topk_group",
                                                          "decode_gateup", "decode_down"])
        rec = {"T": T, "tokens_per_s": T / (ms * 1e-3), "ms_per_layer": ms, "layer_tflops": flops / (ms * 1e-3) / 1e12,
               "layer_mfma_frac": flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS,
               "layer_ms_median_of": len(per_replay), "layer_ms_per_replay": per_replay,
               "kernel_us": {n: v[0] * 1e3 for n, v in kt.items()},
               "kernel_span_us": {n: v[0] for n, v in spans.items()}}
        # the grouped GEMMs by their event-timed launches (the interval a rocprofv3 trace reports)
        gu_fl, d_fl = 4.0 * T * shape.k * shape.H * shape.I, 2.0 * T * shape.k * shape.H * shape.I
        if "prefill_gateup" in kt:
            rec["gateup_tflops"] = gu_fl / (kt["prefill_gateup"][0] * 1e-3) / 1e12
            rec["gateup_mfma_frac"] = rec["gateup_tflops"] / BF16_PEAK_TFLOPS
        if "prefill_down" in kt:
            rec["down_tflops"] = d_fl / (kt["prefill_down"][0] * 1e-3) / 1e12
            rec["down_mfma_frac"] = rec["down_tflops"] / BF16_PEAK_TFLOPS
        if "prefill_gateup" in kt and "prefill_down" in kt:
            gemm_ms = kt["prefill_gateup"][0] + kt["prefill_down"][0]
            rec["gemm_pair_ms"] = gemm_ms
            rec["gemm_pair_mfma_frac"] = flops / (gemm_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS
        log(f"{name}: {rec['tokens_per_s']:.0f} tok/s, {ms:.3f} ms/layer, {rec['layer_tflops']:.1f} TFLOP/s "
            f"({rec['layer_mfma_frac'] * 100:.1f}% of bf16 MFMA)")
        return rec

    if not args.no_secondary and args.only in (None, "prefill"):
        bias = olmoe_syn.zipf_bias()
        for T in args.prefill_tokens:
            secondary[f"olmoe_prefill_zipf_T{T}"] = run_prefill(f"olmoe_prefill_zipf_T{T}", OLMOE, olmoe_syn,
                                                                banks[:2], wr, T, bias, 20, 3)
    if banks is not None:
        del banks
        torch.cuda.empty_cache()
    if not args.no_secondary and args.only in (None, "large"):
        syn = SyntheticLayer(LARGE, seed=0)
        t0 = time.time()
        from concurrent.futures import ThreadPoolExecutor
        with ThreadPoolExecutor(4) as ex:
            blobs = [b for b in ex.map(lambda e: exm.quantize_pack(*syn.expert(e)), range(LARGE.E))]
        bank = exm.bank_from_blobs(blobs)
        del blobs
        log(f"built large-expert layer ({bank.base.numel() / 1e6:.0f} MB) in {time.time() - t0:.1f}s")
        secondary["large_prefill_T4096"] = run_prefill("large_prefill_T4096", LARGE, syn, [bank],
                                                       to_dev_bf16(syn.router()), 4096, None, 10, 2, replays=12)

    if not args.no_secondary and args.only in (None, "large", "blas"):
        secondary["blas_dense_bf16_reference"] = run_blas_reference(torch)

    if "head" not in result:
        print(json.dumps({"secondary": secondary}))
        return
    head = result["head"]
    cpu = None
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle) ...")
        cpu = cpu_baseline(olmoe_syn, OLMOE, args.tokens, args.cpu_seconds)
        log(f"cpu oracle: {cpu['value']:.2f} tok/s on {cpu['cores']} threads")
    line = {
        "metric": METRIC,
        "value": head["tokens_per_s"],
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["us_per_layer"] / 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"olmoe_decode_T{args.tokens}", "hidden": H, "experts": E, "top_k": k,
                   "intermediate": I, "tokens_per_call": args.tokens, "weights": "int4 group-128 symmetric, bf16 scales",
                   "rotated_banks": args.rotate, "hip_graph": use_graph,
                   "layer_hbm_gbs": head["layer_hbm_gbs"], "layer_hbm_frac": head["layer_hbm_frac"],
                   "distinct_experts_mean": head["distinct_experts_mean"], "kernel_us": head.get("kernel_us")},
        "roofline": head["roofline"],
        "roofline_prefill": prefill_roofline(secondary.get("large_prefill_T4096"), read_kernel_avg),
        "cpu_baseline": cpu,
        "secondary": secondary,
    }
    print(json.dumps(line))


if __name__ == "__main__":
    main()
