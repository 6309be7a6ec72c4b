#!/usr/bin/env python3
"""Summaries of rocprofv3 output for the library's kernels (standard library only).

    python3 rocprof_summary.py stats  DIR --cmd "..." --out FILE
    python3 rocprof_summary.py traffic --kernel decode_fused_kernel \\
        --fetch DIR --write DIR --copy-bytes N --cmd "..." --out FILE
    python3 rocprof_summary.py counters DIR [DIR ...] [--kernel PREFIX] [--copy-bytes N] \\
        --cmd "..." [--cmd "..."] --out FILE

`stats` turns a `rocprofv3 --kernel-trace --stats` run into a per-kernel table (calls,
average, median, min, max and total duration). `traffic` turns two `rocprofv3 --pmc`
runs, one of FETCH_SIZE and one of WRITE_SIZE (KiB per dispatch), into HBM bytes per
launch of one kernel. Each counter is scaled by the ratio between the known traffic of
`exmoe::copy_kernel` (N bytes read and N bytes written per dispatch, N larger than the
on-package caches) and what the same counter reads for that copy in the same run. The
traffic file records a hash of the kernel's sources; `read_traffic` returns nothing once
the sources have changed since the counters were taken. `stats` files record the same
hash for the kernels named in KERNEL_SOURCES, and `read_kernel_avg` returns a kernel's
average launch duration from such a file under the same rule. Measurement tooling only:
nothing in the library imports it; bench.py reads the committed summaries through it.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
import sqlite3
import statistics
import sys

CSRC = os.path.join(os.path.dirname(os.path.abspath(__file__)), "w4a16_mixture_experts_amd", "csrc")

# Sources each profiled kernel is compiled from.
_DECODE_SOURCES = ["moe_decode.hip", "device.h", "common.h", "group_block.h", "topk.h"]
KERNEL_SOURCES = {
    "decode_expert_kernel": _DECODE_SOURCES,
    "decode_fused_kernel": _DECODE_SOURCES,
    "decode_narrow_kernel": _DECODE_SOURCES,
    "prefill_kernel": ["moe_prefill.hip", "device.h", "common.h"],
}


def source_hash(kernel: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    n = name.split("(")[0].replace("void ", "").strip()
    return n.replace("exmoe::", "")


def _csv_rows(d: str, suffix: str):
    for f in sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)):
        with open(f, newline="") as fh:
            yield from csv.DictReader(fh)


def _grid(r) -> str:
    if "Grid_Size_X" in r:
        g = [int(r["Grid_Size_" + a]) for a in "XYZ"]
        w = [int(r.get("Workgroup_Size_" + a, 1) or 1) for a in "XYZ"]
        return "x".join(str(gi // max(wi, 1)) for gi, wi in zip(g, w) if gi > 0) + f" wg{w[0] * w[1] * w[2]}"
    return str(r.get("Grid_Size", "?"))


def kernel_durations(d: str) -> dict[tuple[str, str], list[float]]:
    """(kernel name, launch grid in workgroups) -> durations in microseconds, from a
    kernel-trace run."""
    out: dict[tuple[str, str], list[float]] = {}
    for r in _csv_rows(d, "kernel_trace.csv"):
        us = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1000.0
        out.setdefault((short_name(r["Kernel_Name"]), _grid(r)), []).append(us)
    if out:
        return out
    for db in sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True)):
        con = sqlite3.connect(db)
        for name, st, en in con.execute("select name, start, end from kernels"):
            out.setdefault((short_name(name), "?"), []).append((en - st) / 1000.0)
    return out


def dispatch_counters(d: str, counter: str) -> dict[str, list[float]]:
    """Kernel name -> per-dispatch values of one counter, from a --pmc run."""
    per: dict[tuple[str, str], float] = {}
    rows = list(_csv_rows(d, "counter_collection.csv"))
    if rows:
        for r in rows:
            if r["Counter_Name"] != counter:
                continue
            key = (short_name(r["Kernel_Name"]), r["Dispatch_Id"])
            per[key] = per.get(key, 0.0) + float(r["Counter_Value"])
    else:
        for db in sorted(glob.glob(os.path.join(d, "**", "*.db"), recursive=True)):
            con = sqlite3.connect(db)
            q = "select kernel_name, dispatch_id, value from counters_collection where counter_name = ?"
            for name, did, val in con.execute(q, (counter,)):
                key = (short_name(name), str(did))
                per[key] = per.get(key, 0.0) + float(val)
    out: dict[str, list[float]] = {}
    for (name, _), v in per.items():
        out.setdefault(name, []).append(v)
    return out


def _ours(name: str) -> bool:
    return name.split("<")[0] in ("route_logits_kernel", "topk_kernel", "topk_group_kernel", "group_kernel",
                                  "decode_gateup_kernel", "decode_down_kernel", "combine_kernel", "xsum_kernel",
                                  "prefill_kernel", "copy_kernel", "route_token_kernel", "decode_expert_kernel",
                                  "decode_fused_kernel", "combine_parts_kernel", "combine_parts_tok_kernel", "route_sel_kernel",
                                  "route_logits_mfma_kernel",
                                  "decode_narrow_kernel", "bf16_decode_kernel", "group_count_kernel",
                                  "group_scan_kernel", "group_scatter_kernel", "table_fill_kernel", "span_fill_kernel",
                                  "wave_union_kernel", "route_logits_split_kernel", "route_logits_split2_kernel",
                                  "group_scan_scatter_kernel")


def _match(values: dict[str, list[float]], kernel: str) -> list[float]:
    got = []
    for name, v in values.items():
        base = name.split("<")[0]
        if base == kernel:
            got += v
    return got


def cmd_stats(args):
    durs = kernel_durations(args.dir)
    lines = [f"# rocprofv3 kernel-trace summary: {args.title}", f"# command: {args.cmd}",
             "# one row per (kernel, launch grid in workgroups x workgroup size); durations in",
             "# microseconds per launch; library kernels first, then the rest",
             "# sources: " + " ".join(f"{k}={source_hash(k)}" for k in sorted(KERNEL_SOURCES)), "",
             f"{'kernel':44s} {'grid':>16s} {'calls':>7s} {'avg':>9s} {'median':>9s} {'min':>9s} {'max':>9s} "
             f"{'total_ms':>9s}"]
    order = sorted(durs.items(), key=lambda kv: (not _ours(kv[0][0]), -sum(kv[1])))
    for (name, grid), v in order:
        v = sorted(v)
        lines.append(f"{name[:44]:44s} {grid:>16s} {len(v):7d} {sum(v) / len(v):9.2f} {v[len(v) // 2]:9.2f} "
                     f"{v[0]:9.2f} {v[-1]:9.2f} {sum(v) / 1e3:9.3f}")
    text = "\n".join(lines) + "\n"
    _emit(text, args.out)


def cmd_traffic(args):
    fetch = dispatch_counters(args.fetch, "FETCH_SIZE")
    write = dispatch_counters(args.write, "WRITE_SIZE")
    kf, kw = _match(fetch, args.kernel), _match(write, args.kernel)
    cf, cw = _match(fetch, "copy_kernel"), _match(write, "copy_kernel")
    if not (kf and kw and cf and cw):
        sys.exit(f"missing dispatches: kernel fetch {len(kf)} write {len(kw)}, copy fetch {len(cf)} write {len(cw)}")
    copy_kib = args.copy_bytes / 1024.0
    f_fac = copy_kib / statistics.median(cf)
    w_fac = copy_kib / statistics.median(cw)
    fk, wk = statistics.mean(kf), statistics.mean(kw)
    traffic = (fk * f_fac + wk * w_fac) * 1024.0
    lines = [f"# HBM traffic per launch of exmoe::{args.kernel}: {args.title}",
             f"# fetch command: {args.cmd_fetch or args.cmd}",
             f"# write command: {args.cmd_write or args.cmd}",
             "# FETCH_SIZE and WRITE_SIZE are KiB per dispatch; each is scaled by",
             "# (known copy bytes) / (counter reading of exmoe::copy_kernel in the same run).",
             f"kernel: {args.kernel}",
             f"source_sha256: {source_hash(args.kernel)}",
             f"dispatches_fetch: {len(kf)}",
             f"dispatches_write: {len(kw)}",
             f"fetch_kib_per_dispatch_raw: {fk:.1f}",
             f"write_kib_per_dispatch_raw: {wk:.1f}",
             f"copy_bytes: {args.copy_bytes}",
             f"copy_fetch_kib_raw: {statistics.median(cf):.1f}",
             f"copy_write_kib_raw: {statistics.median(cw):.1f}",
             f"fetch_factor: {f_fac:.4f}",
             f"write_factor: {w_fac:.4f}",
             f"traffic_bytes_per_launch: {traffic:.0f}"]
    _emit("\n".join(lines) + "\n", args.out)


def cmd_counters(args):
    """Per-dispatch means of counters over one or more --pmc runs (one run per counter
    pass, e.g. two passes of 8 SQ counters), for the library's kernels (or those whose
    name starts with --kernel), then derived figures for each kernel whose counters are
    all present: MFMA-busy share of the CU-busy cycles (4 SIMDs), VALU (non-MFMA)
    instructions per MFMA, LDS instructions per MFMA, VALU co-issued with MFMA, LDS-index
    activity; and with --copy-bytes, FETCH_SIZE / WRITE_SIZE scaled to bytes by
    exmoe::copy_kernel's readings in the same run."""
    cmds = args.cmd
    lines = [f"# rocprofv3 --pmc per-dispatch means: {args.title}"] + [f"# command: {c}" for c in cmds] + [""]
    means: dict[str, dict[str, float]] = {}
    copy: dict[str, float] = {}
    for d in args.dirs:
        names = args.counter or sorted({r["Counter_Name"] for r in _csv_rows(d, "counter_collection.csv")})
        for c in names:
            vals = dispatch_counters(d, c)
            for name, v in sorted(vals.items()):
                if name.split("<")[0] == "copy_kernel":
                    copy[c] = statistics.median(v)
                if not _ours(name) or (args.kernel and not name.startswith(args.kernel)):
                    continue
                means.setdefault(name, {})[c] = statistics.mean(v)
                lines.append(f"{name[:44]:44s} {c:28s} dispatches={len(v):5d} mean={statistics.mean(v):.6g}")
    lines.append("")
    for name, m in sorted(means.items()):
        d = []
        if all(k in m for k in ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_BUSY_CU_CYCLES")):
            d.append(f"MFMA busy / (4 x SQ_BUSY_CU_CYCLES) = {m['SQ_VALU_MFMA_BUSY_CYCLES'] / (4 * m['SQ_BUSY_CU_CYCLES']):.3f}")
        if all(k in m for k in ("SQ_INSTS_VALU", "SQ_INSTS_MFMA")) and m["SQ_INSTS_MFMA"]:
            d.append(f"(SQ_INSTS_VALU - SQ_INSTS_MFMA) / SQ_INSTS_MFMA = "
                     f"{(m['SQ_INSTS_VALU'] - m['SQ_INSTS_MFMA']) / m['SQ_INSTS_MFMA']:.2f}")
        if all(k in m for k in ("SQ_INSTS_LDS", "SQ_INSTS_MFMA")) and m["SQ_INSTS_MFMA"]:
            d.append(f"SQ_INSTS_LDS / SQ_INSTS_MFMA = {m['SQ_INSTS_LDS'] / m['SQ_INSTS_MFMA']:.2f}")
        if all(k in m for k in ("SQ_VALU_MFMA_COEXEC_CYCLES", "SQ_VALU_MFMA_BUSY_CYCLES")) and m["SQ_VALU_MFMA_BUSY_CYCLES"]:
            d.append(f"VALU co-issued with MFMA / MFMA busy = "
                     f"{m['SQ_VALU_MFMA_COEXEC_CYCLES'] / m['SQ_VALU_MFMA_BUSY_CYCLES']:.3f}")
        if all(k in m for k in ("SQ_LDS_IDX_ACTIVE", "SQ_BUSY_CU_CYCLES")):
            d.append(f"SQ_LDS_IDX_ACTIVE / SQ_BUSY_CU_CYCLES = {m['SQ_LDS_IDX_ACTIVE'] / m['SQ_BUSY_CU_CYCLES']:.3f}")
        if args.copy_bytes:
            for c in ("FETCH_SIZE", "WRITE_SIZE"):
                if c in m and copy.get(c):
                    fac = args.copy_bytes / 1024.0 / copy[c]
                    d.append(f"{c} x {fac:.4f} = {m[c] * fac * 1024.0 / 1e6:.1f} MB per dispatch")
        for x in d:
            lines.append(f"derived {name[:44]:44s} {x}")
    _emit("\n".join(lines) + "\n", args.out)


def read_traffic(path: str, kernel: str):
    """HBM bytes per launch recorded in a traffic file, or None when the file is missing or
    the kernel's sources have changed since the counters were taken."""
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                a, b = line.split(":", 1)
                kv[a.strip()] = b.strip()
    if kv.get("kernel") != kernel or kv.get("source_sha256") != source_hash(kernel):
        return None
    return {"bytes": float(kv["traffic_bytes_per_launch"]), "fetch_factor": float(kv["fetch_factor"]),
            "write_factor": float(kv["write_factor"]), "source_sha256": kv["source_sha256"]}


def read_kernel_avg(path: str, kernel: str, grid: str):
    """(average, median, calls) in microseconds of one (kernel, grid) row of a `stats` file,
    or None when the file is missing, has no such row, or the kernel's sources changed
    since the trace was taken. kernel is the row's name up to its template arguments' end,
    e.g. 'decode_fused_kernel<2, true, 16>'; grid e.g. '257x1x1 wg1024'."""
    if not os.path.exists(path):
        return None
    base = kernel.split("<")[0]
    with open(path) as fh:
        lines = fh.read().splitlines()
    src = [ln for ln in lines if ln.startswith("# sources:")]
    if base in KERNEL_SOURCES:
        want = f"{base}={source_hash(base)}"
        if not src or want not in src[0].split():
            return None
    for ln in lines:
        if ln.startswith("#") or not ln.startswith(kernel):
            continue
        rest = ln[len(kernel):].split()
        if len(rest) >= 6 and f"{rest[0]} {rest[1]}" == grid:
            return float(rest[3]), float(rest[4]), int(rest[2])
    return None


def _emit(text: str, out: str | None):
    if out:
        os.makedirs(os.path.dirname(os.path.abspath(out)), exist_ok=True)
        with open(out, "w") as fh:
            fh.write(text)
    sys.stdout.write(text)


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="what", required=True)
    a = sub.add_parser("stats")
    a.add_argument("dir")
    a.add_argument("--cmd", required=True)
    a.add_argument("--title", default="")
    a.add_argument("--out")
    b = sub.add_parser("traffic")
    b.add_argument("--kernel", required=True)
    b.add_argument("--fetch", required=True)
    b.add_argument("--write", required=True)
    b.add_argument("--copy-bytes", type=int, required=True)
    b.add_argument("--cmd", default="")
    b.add_argument("--cmd-fetch", default="")
    b.add_argument("--cmd-write", default="")
    b.add_argument("--title", default="")
    b.add_argument("--out")
    c = sub.add_parser("counters")
    c.add_argument("dirs", nargs="+")
    c.add_argument("--counter", action="append", default=[])
    c.add_argument("--kernel", default="")
    c.add_argument("--copy-bytes", type=int, default=0)
    c.add_argument("--cmd", action="append", required=True)
    c.add_argument("--title", default="")
    c.add_argument("--out")
    args = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[args.what](args)


if __name__ == "__main__":
    main()
