#!/usr/bin/env python3
"""Benchmark: MoE dispatch + combine on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is the whole path over one batch already resident in HBM: the
dispatch layout (counts, offsets, maps) and the row permutation with fused FP8
quantization -- by default one moe_dispatch_fused call, which infers the
layout inside dispatch; with --separate, moe_dispatch_layout + moe_dispatch --
then moe_combine (weighted top-k reduction), all through the C ABI on torch's
current stream.  The stand-in expert outputs y
are a separate, pre-generated input (the expert GEMMs are not part of the
path), so combine reads them cold, as it would after real experts.

Prints ONE JSON line on stdout; progress goes to stderr.  The headline
workload is the DeepSeek-V3-shaped prefill batch (8192 tokens, hidden 7168,
256 experts, top-8, 8 virtual ranks, 128-row-aligned contiguous layout, FP8
E4M3 with packed UE8M0 scales).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import combine_topk_idx_amd as M  # noqa: E402
from combine_topk_idx_amd import workloads as W  # noqa: E402

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, vendor peak
QUANT_NAME = {W.QUANT_NONE: "bf16", W.QUANT_FP8_F32: "fp8_e4m3_fp32scale",
              W.QUANT_FP8_UE8M0: "fp8_e4m3_ue8m0", W.QUANT_MXFP8: "mxfp8_e4m3_e8m0_1x32"}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def algorithmic_bytes(wl, n_kept):
    """Bytes the method itself must move (padding rows, empty slots and
    re-reads excluded), per call."""
    T, K, H = wl.T, wl.K, wl.H
    nb = H // 128
    if wl.quant == W.QUANT_NONE:
        b_elt, scale_row = 2, 0
    elif wl.quant == W.QUANT_FP8_F32:
        b_elt, scale_row = 1, 4 * nb
    elif wl.quant == W.QUANT_MXFP8:
        b_elt, scale_row = 1, H // 32
    else:
        b_elt, scale_row = 1, 4 * ((nb + 3) // 4)
    layout = 4 * T * K + 4 * T * K + 4 * n_kept
    dispatch = 2 * T * H + 4 * T * K + n_kept * (H * b_elt + scale_row)
    combine = 2 * n_kept * H + 8 * T * K + 2 * T * H
    return {"layout": layout, "dispatch": dispatch, "combine": combine}


def dedup_bytes(wl, n_kept, n_rows):
    """Algorithmic bytes per call of the per-rank deduplicated path; n_rows =
    (token, rank) rows."""
    T, K, H, R = wl.T, wl.K, wl.H, wl.R
    nb = H // 128
    if wl.quant == W.QUANT_NONE:
        row = 2 * H
    elif wl.quant == W.QUANT_FP8_F32:
        row = H + 4 * nb
    elif wl.quant == W.QUANT_MXFP8:
        row = H + H // 32
    else:
        row = H + 4 * ((nb + 3) // 4)
    return {"rank_layout": 4 * T * K + 4 * T * R + 4 * n_rows,
            "layout": 4 * T * K + 4 * T * K + 4 * n_kept,
            "dispatch_dedup": 2 * T * H + 4 * T * R + n_rows * row,
            "expand": 12 * T * K + n_rows * row + n_kept * row,
            "combine_partial": 2 * n_kept * H + 16 * T * K + 2 * n_rows * H,
            "combine_reduce": 4 * T * R + 2 * n_rows * H + 2 * T * H}


def row_and_scale_bytes(wl):
    """(bytes of a dispatched row, bytes of its scales)."""
    H, nb = wl.H, wl.H // 128
    return {W.QUANT_NONE: (2 * H, 0), W.QUANT_FP8_F32: (H, 4 * nb),
            W.QUANT_FP8_UE8M0: (H, 4 * ((nb + 3) // 4)), W.QUANT_MXFP8: (H, H // 32)}[wl.quant]


def run_adapters(args, wl, cfg, d_idx, d_w, d_x, bufs, stream):
    """Times the grouped-GEMM adapters on a masked dispatch: per-row experts,
    masked -> contiguous repack, contiguous -> masked repack of bf16 expert
    outputs, MN-major scales; HIP events between the calls."""
    if wl.layout != W.LAYOUT_MASKED:
        raise SystemExit("--adapters needs a masked workload")
    T, H, E, C, A = wl.T, wl.H, wl.E, wl.capacity, args.align
    dev = d_x.device
    M.moe_dispatch_layout(cfg, T, d_idx, bufs.handle, bufs.workspace, stream)
    M.moe_dispatch(cfg, T, d_x, None, bufs.handle, bufs.out_x, bufs.out_scale, None, stream)
    crows = M.moe_repack_rows_capacity(cfg, A)
    rows = bufs.rows
    out_x = torch.empty((crows, H), dtype=bufs.out_x.dtype, device=dev)
    out_s = None if bufs.out_scale is None else torch.empty((crows, bufs.out_scale.shape[1]),
                                                            dtype=bufs.out_scale.dtype, device=dev)
    off = torch.empty(E + 1, dtype=torch.int32, device=dev)
    rex_c = torch.empty(crows, dtype=torch.int32, device=dev)
    rex = torch.empty(rows, dtype=torch.int32, device=dev)
    y_c = torch.randn((crows, H), device=dev).to(torch.bfloat16).view(torch.int16)
    y_m = torch.empty((rows, H), dtype=torch.int16, device=dev)
    S = M.moe_scale_words(cfg)
    ld = (rows + 3) // 4 * 4
    s_mn = torch.empty(max(S * ld, 1), dtype=torch.int32, device=dev)
    calls = [
        ("row_expert", lambda: M.moe_row_expert(cfg, bufs.handle, rex, stream)),
        ("repack_masked_to_contiguous", lambda: M.moe_repack_masked_to_contiguous(
            cfg, A, bufs.handle, bufs.out_x, bufs.out_scale, out_x, out_s, off, rex_c, stream)),
        ("repack_contiguous_to_masked", lambda: M.moe_repack_contiguous_to_masked(
            cfg, bufs.handle, off, y_c, y_m, stream)),
    ]
    if S > 0:
        calls.append(("scales_mn_major", lambda: M.moe_scales_mn_major(cfg, rows, bufs.out_scale, s_mn, stream)))
    for _ in range(args.warmup):
        for _, f in calls:
            f()
    torch.cuda.synchronize()
    n = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(n)]
    for row in ev:
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    log(f"[bench] adapters: timing {n} rounds")
    for i in range(n):
        for j, (_, f) in enumerate(calls):
            ev[i][j].record(stream)
            f()
        ev[i][-1].record(stream)
    torch.cuda.synchronize()
    ms = {name: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(n)]))
          for j, (name, _) in enumerate(calls)}
    kept = int(bufs.handle.recv_count.cpu().numpy().sum())
    used = int(off.cpu().numpy()[-1])
    rb, sb = row_and_scale_bytes(wl)
    ab = {"row_expert": 4 * rows + 8 * E,
          "repack_masked_to_contiguous": 2 * kept * (rb + sb) + 4 * crows + 12 * E,
          "repack_contiguous_to_masked": 2 * kept * 2 * H + 8 * E,
          "scales_mn_major": 4 * rows * S + 4 * S * ld}
    ab = {k: v for k, v in ab.items() if k in ms}
    gbs = {k: ab[k] / (ms[k] * 1e-3) / 1e9 for k in ab}
    copy_gbs = copy_ceiling(args.calib_copy_mib, dev, stream)
    return {"metric": "grouped-GEMM adapter GB/s per call (masked dispatch)", "value": gbs["repack_masked_to_contiguous"],
            "unit": "GB/s", "n_gpus": 1, "steps": n, "warmup": args.warmup, "higher_is_better": True,
            "vs_baseline": None, "dtype": "u8", "data": "synthetic", "library_sha256": library_hash(),
            "config": {"workload": wl.name, "tokens": T, "hidden": H, "experts": E, "capacity": C, "align": A,
                       "quant": QUANT_NAME[wl.quant]},
            "path": {"calls": [c for c, _ in calls], "per_call_ms_mean": ms, "algorithmic_bytes": ab,
                     "per_call_gbs": gbs, "kept_rows": kept, "contiguous_rows_used": used,
                     "contiguous_rows_capacity": crows, "copy_ceiling_gbs": copy_gbs}}


def copy_ceiling(mib, dev, stream):
    """GB/s of a plain device-to-device copy of `mib` MiB (the attainable
    ceiling next to the kernels; also the counter calibration)."""
    n_copy = mib * (1 << 20) // 4
    src = torch.empty(n_copy, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record(stream)
    for _ in range(10):
        dst.copy_(src)
    c1.record(stream)
    torch.cuda.synchronize()
    return 2 * n_copy * 4 * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9


def run_dedup(args, wl, cfg, d_idx, d_w, d_x, d_y, d_out, bufs, stream):
    """Times the per-rank deduplicated path: per-rank layout, per-expert
    layout, deduplicated dispatch, expansion, partial combine and the final
    reduction; steps back to back between two events, then the same steps
    with an event between the calls for the per-call times."""
    T = wl.T
    db = M.DedupBuffers(cfg, device=d_x.device)
    calls = [
        ("rank_layout", lambda: M.moe_rank_layout(cfg, T, d_idx, db.handle, stream)),
        ("layout", lambda: M.moe_dispatch_layout(cfg, T, d_idx, bufs.handle, bufs.workspace, stream)),
        ("dispatch_dedup", lambda: M.moe_dispatch_dedup(cfg, T, d_x, db.handle, db.send_x, db.send_scale,
                                                        stream)),
        ("expand", lambda: M.moe_expand(cfg, T, d_idx, db.send_x, db.send_scale, db.handle, bufs.handle,
                                        bufs.out_x, bufs.out_scale, stream)),
        ("combine_partial", lambda: M.moe_combine_partial(cfg, T, d_idx, d_y, d_w, bufs.handle, db.handle,
                                                          db.partial, stream)),
        ("combine_reduce", lambda: M.moe_combine_reduce(cfg, T, db.partial, db.handle, d_out, stream)),
    ]
    log(f"[bench] per-rank deduplicated path: warmup {args.warmup} steps")
    for _ in range(args.warmup):
        for _, f in calls:
            f()
    torch.cuda.synchronize()
    n = args.steps
    # the steps back to back between two events (an event between two calls
    # waits for the first one's cache write-back, so the per-call times come
    # from a second run with an event between every call)
    b0, e0 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(n)]
    for e in [b0, e0] + [e for row in ev for e in row]:  # create the events before the timed region
        e.record(stream)
    torch.cuda.synchronize()
    log(f"[bench] timing {n} steps")
    wall0 = time.perf_counter()
    b0.record(stream)
    for i in range(n):
        for _, f in calls:
            f()
    e0.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_step = b0.elapsed_time(e0) / n
    log(f"[bench] timing {n} steps with an event between the calls (per-call times)")
    for i in range(n):
        for j, (_, f) in enumerate(calls):
            ev[i][j].record(stream)
            f()
        ev[i][-1].record(stream)
    torch.cuda.synchronize()
    ms = {name: float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(n)]))
          for j, (name, _) in enumerate(calls)}
    n_kept = int(bufs.handle.recv_count.cpu().numpy().sum())
    n_rows = int(db.handle.rank_token_offset.cpu().numpy()[-1])
    ab = dedup_bytes(wl, n_kept, n_rows)
    gbs = {k: ab[k] / (ms[k] * 1e-3) / 1e9 for k in ab}
    step_gbs = sum(ab.values()) / (ms_step * 1e-3) / 1e9
    copy_gbs = copy_ceiling(args.calib_copy_mib, d_x.device, stream)
    return {
        "metric": "per-rank deduplicated dispatch+combine tokens/s (one GPU's local steps)",
        "value": T / (ms_step * 1e-3), "unit": "tokens/s", "n_gpus": 1, "steps": n,
        "warmup": args.warmup, "ms_per_step": ms_step, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": wl.name, "tokens": T, "hidden": wl.H, "experts": wl.E, "topk": wl.K,
                   "virtual_ranks": wl.R, "quant": QUANT_NAME[wl.quant],
                   "caches": "warm: steps back to back"},
        "library_sha256": library_hash(),
        "path": {"calls": [c for c, _ in calls], "per_call_ms_mean": ms, "algorithmic_bytes": ab,
                 "per_call_gbs": gbs, "gbs": step_gbs, "frac_of_peak": step_gbs / HBM_PEAK_GBS,
                 "kept_pairs": n_kept, "rank_rows": n_rows, "copy_ceiling_gbs": copy_gbs,
                 "wall_ms_per_step": wall * 1e3 / n,
                 "ms_per_step_with_call_events": float(np.mean([ev[i][0].elapsed_time(ev[i][-1]) for i in range(n)]))},
    }


def code_text(source):
    """C/C++ source with its comments removed and every run of whitespace
    reduced to one space: comment and layout edits leave it unchanged, any
    change to the code does not."""
    out, i, n = [], 0, len(source)
    while i < n:
        c = source[i]
        if source.startswith("//", i):
            j = source.find("\n", i)
            i = n if j < 0 else j
        elif source.startswith("/*", i):
            j = source.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif c in "\"'":  # string or character literal, escapes included
            j = i + 1
            while j < n and source[j] != c:
                j += 2 if source[j] == "\\" else 1
            out.append(source[i:j + 1])
            i = j + 1
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def library_hash():
    """sha256 over the code (comments and whitespace removed, see code_text)
    of every source the library is built from (kernels, launch plans, ABI):
    counter figures taken on other code are not reused."""
    h = hashlib.sha256()
    for sub in (("include",), ("combine_topk_idx_amd", "csrc")):
        d = os.path.join(ROOT, *sub)
        for name in sorted(os.listdir(d)):
            if name.endswith((".h", ".hip")):
                h.update(name.encode())
                with open(os.path.join(d, name), encoding="utf-8") as f:
                    h.update(code_text(f.read()).encode())
    return h.hexdigest()


def measured_traffic(kernel, section):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the library sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[section]
        if rec.get("library_sha256") != library_hash():
            return None
        return rec["kernels"][kernel]["bytes_per_launch"]
    except (OSError, KeyError, ValueError, TypeError):
        return None


# ---------------------------------------------------------------------------
# profile summaries: fold rocprofv3 output of this script into profiles/
# ---------------------------------------------------------------------------

QUANT_TEMPLATE = {"0": "bf16", "1": "fp8_f32", "2": "fp8_ue8m0", "3": "mxfp8"}


def short_kernel(name):
    """'void moe::(anonymous namespace)::dispatch_rows<2>(moe::DispatchArgs)'
    -> 'dispatch_rows_fp8_ue8m0'; combine_kernel<false, ...> -> 'combine_kernel',
    combine_kernel<true, ...> -> 'combine_kernel_partial' (the other arguments
    pick streamed output stores and loads, not a separate kernel);
    rank_layout_kernel<KV> (KV = id vectors per
    token, not a format) -> 'rank_layout_kernel'."""
    base = name.split("(moe::")[0].split("::")[-1]
    named = {"repack_kernel<true>": "repack_to_contiguous", "repack_kernel<false>": "repack_to_masked",
             "layout_single<false>": "layout_single", "layout_single<true>": "layout_prefetch"}
    if base in named:
        return named[base]
    if base.startswith("combine_kernel<"):
        return "combine_kernel_partial" if base.startswith("combine_kernel<true") else "combine_kernel"
    if base.startswith("rank_layout_kernel<"):
        return "rank_layout_kernel"
    if "<" in base:
        stem, arg = base[:-1].split("<")
        base = f"{stem}_{QUANT_TEMPLATE.get(arg, arg)}"
    return base


# Kernels of a fused call that also carry prefetch blocks: their counted bytes
# include token rows read ahead into the Infinity Cache, which the method reads
# once and which count in the dispatch's algorithmic bytes.
PREFETCH_NOTES = {
    "layout_prefetch": "Most of these bytes are the prefetch blocks of the fused call reading the token rows x "
                       "(all but the first 3/10 of the tokens) into the Infinity Cache; the row kernel then reads "
                       "them again from there. Algorithmic bytes here are the layout's alone (x belongs to the "
                       "dispatch).",
    "layout_rank": "Most of these bytes are the fused call's prefetch blocks reading 40 MB of token rows into the "
                   "Infinity Cache while the rank kernel runs; the row kernel then reads them again from there. "
                   "Algorithmic bytes here are the ids alone (x belongs to the dispatch).",
    "layout_index": "Most of these bytes are the fused call's prefetch blocks reading 60 MB of token rows into the "
                    "Infinity Cache while the index kernel runs; the row kernel then reads them again from there. "
                    "Algorithmic bytes here are the maps alone (x belongs to the dispatch).",
}


def kernel_bytes(bench):
    """Algorithmic bytes per launch of each library kernel a benchmark line ran."""
    ab = bench["path"]["algorithmic_bytes"]
    if "repack_masked_to_contiguous" in ab:  # grouped-GEMM adapters
        return {"row_expert_kernel": ab["row_expert"], "repack_to_contiguous": ab["repack_masked_to_contiguous"],
                "repack_to_masked": ab["repack_contiguous_to_masked"],
                "scales_mn_major_kernel": ab.get("scales_mn_major")}
    if isinstance(bench["path"]["calls"], list):  # per-rank deduplicated path
        algo = {"rank_layout_kernel": ab["rank_layout"], "layout_single": ab["layout"],
                "expand_kernel": ab["expand"], "combine_kernel_partial": ab["combine_partial"],
                "combine_kernel": ab["combine_reduce"]}
        for q in QUANT_TEMPLATE.values():
            algo[f"dispatch_rows_{q}"] = ab["dispatch_dedup"]
        return algo
    # the large fused dispatch reads x into the Infinity Cache in its layout
    # launch (layout_prefetch) and again from there in its row kernel; the
    # algorithmic read of x belongs to the dispatch
    # the two-launch layout of large batches: the rank kernel reads the ids,
    # the index kernel writes both maps (their table and slot traffic is the
    # workspace, not algorithmic)
    algo = {"combine_kernel": ab["combine"], "layout_single": ab["layout"], "layout_prefetch": ab["layout"]}
    tk4 = bench.get("config", {}).get("tokens", 0) * bench.get("config", {}).get("topk", 0) * 4
    if tk4:
        algo["layout_rank"] = tk4
        algo["layout_index"] = ab["layout"] - tk4
    for q in QUANT_TEMPLATE.values():
        algo[f"dispatch_rows_{q}"] = ab["dispatch"]
        algo[f"dispatch_fused_{q}"] = ab["dispatch"] + ab["layout"]
    return algo


def read_csv(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def find_file(d, suffix):
    for root, _, files in os.walk(d):
        for fn in files:
            if fn.endswith(suffix):
                return os.path.join(root, fn)
    raise FileNotFoundError(f"no *{suffix} under {d}")


def read_cmd(d, name):
    try:
        with open(os.path.join(d, name + ".cmd")) as f:
            return f.read().strip()
    except OSError:
        return "(command not recorded)"


EXTRA_COUNTERS = ("VALUBusy", "VALUUtilization", "LDSBankConflict", "TCC_HIT_sum", "TCC_MISS_sum")


def _counter_medians(run_dir, sub, names):
    """{(kernel, grid): {counter: median per dispatch}} from a --pmc run
    directory, or {} when the run is absent."""
    d = os.path.join(run_dir, sub)
    if not os.path.isdir(d):
        return {}
    vals = {}
    for row in read_csv(find_file(d, "counter_collection.csv")):
        if row["Counter_Name"] not in names:
            continue
        key = (row["Kernel_Name"], int(row["Grid_Size"]))
        vals.setdefault(key, {}).setdefault(row["Counter_Name"], []).append(float(row["Counter_Value"]))
    return {k: {c: float(np.median(v)) for c, v in cs.items()} for k, cs in vals.items()}


def _trace_stats(run_dir, sub):
    """{kernel name: (calls, avg, min, max, stddev in us)} of a kernel-trace run, or {}."""
    d = os.path.join(run_dir, sub)
    if not os.path.isdir(d):
        return {}
    out = {}
    for row in read_csv(find_file(d, "kernel_stats.csv")):
        out[row["Name"]] = (row["Calls"],) + tuple(float(row[k]) / 1e3 for k in ("AverageNs", "MinNs", "MaxNs",
                                                                                   "StdDev"))
    return out


def summarize(run_dir, calib_mib):
    """Write profiles/traffic.json and one Markdown summary per library
    kernel from a run directory holding: prof_bench/ (kernel trace + stats of
    back-to-back steps) and optionally prof_bench_cold/ (steps after a cache
    flush), pmc_FETCH_SIZE/ and pmc_WRITE_SIZE/ (one counter per run, with a
    `calib_mib` MiB device copy in the same runs), optionally pmc_extra/ and
    pmc_extra_cold/ (VALU, LDS and L2 counters), bench.json (the benchmark
    line of the same build) and the *.cmd files naming the commands."""
    with open(os.path.join(run_dir, "bench.json")) as f:
        bench = json.loads(f.read().strip().splitlines()[-1])
    wl = W.WORKLOADS[bench["config"]["workload"]]
    adapters = "repack_masked_to_contiguous" in bench["path"]["algorithmic_bytes"]
    dedup = isinstance(bench["path"]["calls"], list) and not adapters
    separate = isinstance(bench["path"]["calls"], str) and bench["path"]["calls"].startswith("moe_dispatch_layout")
    section = wl.name + (":dedup" if dedup else ":adapters" if adapters else ":separate" if separate else "")
    built = bench.get("library_sha256")
    if built is None:
        raise SystemExit("bench.json names no library_sha256: rerun the benchmark with the current library")
    algo = kernel_bytes(bench)

    stats = _trace_stats(run_dir, "prof_bench")
    stats_cold = _trace_stats(run_dir, "prof_bench_cold")
    counters = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        for row in read_csv(find_file(os.path.join(run_dir, f"pmc_{c}"), "counter_collection.csv")):
            if row["Counter_Name"] != c:
                continue
            key = (row["Kernel_Name"], int(row["Grid_Size"]))
            counters.setdefault(c, {}).setdefault(key, []).append(float(row["Counter_Value"]))
    extra = _counter_medians(run_dir, "pmc_extra", EXTRA_COUNTERS)
    extra_cold = _counter_medians(run_dir, "pmc_extra_cold", EXTRA_COUNTERS)
    # calibration: the device copy is the copy kernel with the largest grid
    copies = {k: v for k, v in counters["FETCH_SIZE"].items() if "copyBuffer" in k[0]}
    ckey = max(copies, key=lambda k: k[1])
    copy_kib = calib_mib * 1024.0
    cf, cw = float(np.median(counters["FETCH_SIZE"][ckey])), float(np.median(counters["WRITE_SIZE"][ckey]))
    fscale, wscale = copy_kib / cf, copy_kib / cw

    try:
        with open(TRAFFIC_FILE) as f:
            traffic = json.load(f)
    except (OSError, ValueError):
        traffic = {}
    traffic = {k: v for k, v in traffic.items() if isinstance(v, dict) and "kernels" in v}
    traffic[section] = {"library_sha256": built,
                        "_calibration": {"copy_bytes": calib_mib << 20, "copy_kernel": ckey[0],
                                         "copy_grid": ckey[1], "copy_fetch_kib_median": cf,
                                         "copy_write_kib_median": cw, "fetch_scale": fscale,
                                         "write_scale": wscale},
                        "kernels": {}}
    per_kernel = {}
    for (name, grid), vals in counters["FETCH_SIZE"].items():
        if "moe::" not in name:
            continue
        short = short_kernel(name)
        f_kib = float(np.median(vals))
        w_kib = float(np.median(counters["WRITE_SIZE"].get((name, grid), [float("nan")])))
        nbytes = (f_kib * fscale + w_kib * wscale) * 1024.0
        rec = {"kernel": name, "grid": grid, "dispatches": len(vals), "fetch_kib": f_kib,
               "write_kib": w_kib, "bytes_per_launch": int(round(nbytes)),
               "algorithmic_bytes": algo.get(short)}
        if rec["algorithmic_bytes"]:
            rec["ratio"] = nbytes / rec["algorithmic_bytes"]
        for tag, src in (("counters", extra), ("counters_cold", extra_cold)):
            if (name, grid) in src:
                rec[tag] = src[(name, grid)]
        traffic[section]["kernels"][short] = rec
        per_kernel[short] = rec
    os.makedirs(os.path.dirname(TRAFFIC_FILE), exist_ok=True)
    with open(TRAFFIC_FILE, "w") as f:
        json.dump(dict(sorted(traffic.items())), f, indent=1)
        f.write("\n")

    layout = "contiguous A=%d" % wl.align if wl.layout == W.LAYOUT_CONTIGUOUS else "masked C=%d" % wl.capacity
    title = (f"T={wl.T}, H={wl.H}, E={wl.E}, top-{wl.K}, {wl.R} virtual ranks, {layout}, "
             f"{QUANT_NAME[wl.quant]}")
    bench_cmd = read_cmd(run_dir, "bench")
    per_call = bench["path"]
    names = {n for n in list(stats) + list(stats_cold) if "moe::" in n}
    for name in sorted(names):
        short = short_kernel(name)
        if adapters and short not in algo:
            continue  # the dispatch that sets up the adapters run is profiled on its own
        path_name = (" (per-rank deduplicated path)" if dedup else " (grouped-GEMM adapters)" if adapters else
                     " (separate layout and dispatch calls)" if separate else "")
        lines = [f"# {short} -- {wl.name}{path_name} ({title})", "", f"Kernel: `{name}`", ""]
        a = algo.get(short)
        for label, st, sub in (("back-to-back steps", stats, "prof_bench"),
                               ("steps after a cache flush", stats_cold, "prof_bench_cold")):
            if name not in st:
                continue
            calls, avg, mn, mx, sd = st[name]
            lines += [f"## Kernel trace, {label} (rocprofv3 --kernel-trace --stats)", "", "Command:", "",
                      "    " + read_cmd(run_dir, sub), "",
                      "| Calls | Average | Min | Max | StdDev |", "|---|---|---|---|---|",
                      f"| {calls} | {avg:.1f} us | {mn:.1f} us | {mx:.1f} us | {sd:.2f} us |", ""]
            if a:
                lines += [f"Algorithmic bytes per launch: {a:,} B -> {a / (avg * 1e3):,.0f} GB/s at the traced "
                          f"average ({a / (avg * 1e3) / HBM_PEAK_GBS:.1%} of the 8 TB/s HBM peak).", ""]
        sep = {k: v for k, v in per_call.get("separate_calls_ms_mean", {}).items() if v}
        step = (f"step {bench['ms_per_step'] * 1e3:.1f} us ({bench['config'].get('caches', '')}), "
                if "ms_per_step" in bench else "")
        lines += [f"Benchmark line of the same build (`{bench_cmd}`), HIP events on the launch stream: "
                  f"{step}per call "
                  + ", ".join(f"{k} {v * 1e3:.1f} us" for k, v in per_call["per_call_ms_mean"].items())
                  + ("" if not sep else "; separate calls (back to back) "
                     + ", ".join(f"{k} {v * 1e3:.1f} us" for k, v in sep.items())) + ".", ""]
        rec = per_kernel.get(short)
        if rec:
            lines += ["## HBM traffic (rocprofv3 --pmc, one counter per run, back-to-back steps)", "",
                      "Commands:", ""]
            lines += ["    " + read_cmd(run_dir, f"pmc_{c}") for c in ("FETCH_SIZE", "WRITE_SIZE")]
            lines += ["", f"| Counter | KiB per dispatch (median of {rec['dispatches']}) | Scale | Bytes |",
                      "|---|---|---|---|",
                      f"| FETCH_SIZE | {rec['fetch_kib']:,.1f} | x{fscale:.4f} | {rec['fetch_kib'] * fscale * 1024:,.0f} |",
                      f"| WRITE_SIZE | {rec['write_kib']:,.1f} | x{wscale:.4f} | {rec['write_kib'] * wscale * 1024:,.0f} |",
                      f"| **total** | | | **{rec['bytes_per_launch']:,}**"
                      + (f" ({rec['ratio']:.4f} x algorithmic) |" if a else " |"), "",
                      f"Scale factors: the same runs copy {calib_mib} MiB device to device (kernel "
                      f"`{ckey[0]}`, grid {ckey[1]}); per {copy_kib:,.0f} KiB moved its FETCH_SIZE reads "
                      f"{cf:,.1f} KiB and its WRITE_SIZE {cw:,.1f} KiB, so FETCH_SIZE is multiplied by "
                      f"{fscale:.4f} and WRITE_SIZE by {wscale:.4f}. Both count L2 requests to the data "
                      f"fabric: an Infinity Cache hit and an HBM access look the same to them.", ""]
            fused = isinstance(bench["path"]["calls"], str) and bench["path"]["calls"].startswith("moe_dispatch_fused")
            if fused and short in PREFETCH_NOTES and a and rec["ratio"] > 2:
                lines += [PREFETCH_NOTES[short], ""]
            for tag, label, sub in (("counters", "back-to-back steps", "pmc_extra"),
                                    ("counters_cold", "steps after a cache flush", "pmc_extra_cold")):
                cs = rec.get(tag)
                if not cs:
                    continue
                hit, miss = cs.get("TCC_HIT_sum", 0.0), cs.get("TCC_MISS_sum", 0.0)
                lines += [f"## VALU, LDS and L2 counters, {label} (rocprofv3 --pmc, median per dispatch)", "",
                          "Command:", "", "    " + read_cmd(run_dir, sub), "",
                          "| VALUBusy | VALUUtilization | LDSBankConflict | L2 hits | L2 misses | L2 hit rate |",
                          "|---|---|---|---|---|---|",
                          f"| {cs.get('VALUBusy', float('nan')):.1f}% | {cs.get('VALUUtilization', float('nan')):.1f}% "
                          f"| {cs.get('LDSBankConflict', float('nan')):.2f}% | {hit:,.0f} | {miss:,.0f} | "
                          f"{hit / max(hit + miss, 1.0):.1%} |", ""]
        suffix = "_dedup_path" if dedup else "_adapters" if adapters else "_separate" if separate else ""
        fname = f"{short}_{wl.name}{suffix}.md"
        with open(os.path.join(ROOT, "profiles", fname), "w") as f:
            f.write("\n".join(lines))
    print(f"wrote {TRAFFIC_FILE} and summaries for {sorted(per_kernel)}")


CPU_BASELINE_REPEATS = 3         # oracle passes per leg, prefill-sized samples
CPU_BASELINE_REPEATS_SMALL = 10  # decode-sized samples (at most 1024 tokens)


def cpu_model():
    """The host CPU's model name from /proc/cpuinfo (Linux), or None."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.lower().startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_threads():
    """Threads for the all-cores leg: OMP_NUM_THREADS when set (the share of
    the host this process is given), else every CPU the process may run on."""
    env = os.environ.get("OMP_NUM_THREADS", "")
    if env.strip().isdigit() and int(env) > 0:
        return int(env)
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:
        return os.cpu_count() or 1


def cpu_baseline(wl, inp, y, max_tokens, gpu=None):
    """The CPU oracle (as it stands) on a bounded sample: the first
    `max_tokens` tokens of the same batch, layout + dispatch + combine, timed
    on one thread and with the token loops of dispatch and combine split over
    all host cores (OpenMP; the layout stays serial), median of
    CPU_BASELINE_REPEATS passes each (CPU_BASELINE_REPEATS_SMALL for samples of
    at most 1024 tokens).
    When the sample is the whole batch and `gpu` holds the benchmark's final
    outputs (host copies), they are checked against the oracle's: layout and
    dispatched bytes bit for bit, combine within |g - o| <= 1e-2 |o| + 1e-5 S."""
    import oracle
    T = min(wl.T, max_tokens)
    repeats = CPU_BASELINE_REPEATS_SMALL if T <= 1024 else CPU_BASELINE_REPEATS
    sub = wl.replace(T=T)
    idx, w, x = inp.topk_idx[:T], inp.topk_w[:T], inp.x[:T]
    rows = sub.rows_capacity
    oracle._load()

    def one_pass():
        h = oracle.dispatch_layout(idx, wl.E, wl.R, wl.layout, wl.align, wl.capacity, rows_cap=rows)
        ox, osc, _ = oracle.dispatch(x, h["pair_to_row"], wl.K, wl.quant, rows)
        return h, ox, osc, oracle.combine(y[:rows], w, h["pair_to_row"])

    def leg(threads):
        used = oracle.set_threads(threads)
        times = []
        try:
            for _ in range(repeats):
                t0 = time.perf_counter()
                out = one_pass()
                times.append(time.perf_counter() - t0)
        finally:
            oracle.set_threads(1)
        return used, float(np.median(times)), out

    n_all = cpu_threads()
    all_used, all_s, _ = leg(n_all)
    one_used, one_s, (h, ox, osc, out) = leg(1)
    res = {"value": T / all_s, "unit": "tokens/s", "cores": all_used, "kind": "oracle",
           "sample": f"first {T} of {wl.T} tokens of the same batch, layout + dispatch + combine, median of "
                     f"{repeats} passes ({all_s:.2f} s each) with dispatch and combine split over "
                     f"{all_used} OpenMP threads (layout serial)",
           "cpu_model": cpu_model(), "os_cpu_count": os.cpu_count(),
           "gbs": None, "single_thread": {"value": T / one_s, "unit": "tokens/s", "cores": one_used,
                                          "seconds_per_pass": one_s}}
    n_kept = int((h["pair_to_row"] >= 0).sum())
    ab = sum(algorithmic_bytes(sub, n_kept).values())
    res["gbs"] = ab / all_s / 1e9
    res["single_thread"]["gbs"] = ab / one_s / 1e9
    if gpu is not None and T == wl.T:
        check = {}
        check["layout_bit_exact"] = all(np.array_equal(gpu[k][:h[k].size], h[k]) for k in (
            "expert_count", "recv_count", "expert_offset", "rank_offset", "pair_to_row", "row_to_pair", "status"))
        kept = h["row_to_pair"] >= 0
        check["dispatch_bit_exact"] = bool(
            np.array_equal(gpu["out_x"].reshape(rows, -1)[kept], ox.view(np.uint8).reshape(rows, -1)[kept])
            and (osc is None or np.array_equal(gpu["out_scale"].reshape(rows, -1)[kept],
                                               osc.view(np.uint8).reshape(rows, -1)[kept])))
        g = W.bf16_bits_to_f32(gpu["out"]).astype(np.float64)
        o = W.bf16_bits_to_f32(out).astype(np.float64)
        diff = g != o
        check["combine_unequal_elements"] = int(diff.sum())
        if diff.any():  # tolerance on the differing elements only
            p2r = h["pair_to_row"].reshape(T, wl.K)
            tt, jj = np.nonzero(diff)
            S = np.zeros(tt.size)
            for k in range(wl.K):
                r = p2r[tt, k]
                ok = r >= 0
                S[ok] += np.abs(w[tt[ok], k] * W.bf16_bits_to_f32(y[r[ok], jj[ok]]))
            check["combine_within_tolerance"] = bool(np.all(np.abs(g[diff] - o[diff]) <= 1e-2 * np.abs(o[diff]) + 1e-5 * S))
        else:
            check["combine_within_tolerance"] = True
        res["oracle_check"] = check
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=W.HEADLINE, choices=sorted(W.WORKLOADS))
    ap.add_argument("--num-cus", type=int, default=0)
    ap.add_argument("--separate", action="store_true",
                    help="time layout and dispatch as two calls instead of the fused call")
    ap.add_argument("--graph", action="store_true",
                    help="capture steps in a HIP graph and time graph replays (launch-bound "
                         "decode batches); per-call times then come from the eager calls after "
                         "the timed region")
    ap.add_argument("--graph-steps", type=int, default=1,
                    help="steps captured in one graph (--graph); --steps counts steps, not replays")
    ap.add_argument("--dedup", action="store_true",
                    help="time the per-rank deduplicated path instead (rank layout, dedup dispatch, "
                         "expansion, partial combine, reduction)")
    ap.add_argument("--adapters", action="store_true",
                    help="time the grouped-GEMM adapters on a masked workload instead")
    ap.add_argument("--align", type=int, default=128, help="segment alignment for --adapters")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-warm", action="store_true",
                    help="skip the secondary back-to-back steps (profiling runs of cold steps)")
    ap.add_argument("--no-breakdown", action="store_true",
                    help="skip the per-call breakdown after the timed region (profiling runs)")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    ap.add_argument("--flush-mib", type=int, default=512,
                    help="scratch read before each timed step so that it starts with cold caches "
                         "(0: time the headline steps back to back instead)")
    ap.add_argument("--calib-copy-mib", type=int, default=1024,
                    help="size of the plain device copy run after the timed region (copy "
                         "ceiling, and the counter calibration for --summarize)")
    ap.add_argument("--summarize", metavar="RUN_DIR",
                    help="no benchmark: fold the rocprofv3 output in RUN_DIR into profiles/")
    args = ap.parse_args()
    if args.summarize:
        summarize(args.summarize, args.calib_copy_mib)
        return

    if args.graph_steps < 1 or (args.graph_steps > 1 and not args.graph):
        raise SystemExit("--graph-steps needs --graph and a count >= 1")
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the library has no multi-GPU path "
              "(destination ranks are virtual partitions of one device's buffers). "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a HIP device", file=sys.stderr)
        sys.exit(2)

    wl = W.WORKLOADS[args.workload]
    log(f"[bench] workload {wl.name}: generating inputs")
    inp = W.make_inputs(wl)
    cfg = M.MoeConfig(max_tokens=wl.T, hidden=wl.H, num_experts=wl.E, num_topk=wl.K,
                      num_ranks=wl.R, layout=wl.layout, align=wl.align, capacity=wl.capacity,
                      quant=wl.quant, num_cus=args.num_cus)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    bufs = M.DispatchBuffers(cfg, device=dev)
    d_idx = torch.from_numpy(inp.topk_idx).to(dev)
    d_w = torch.from_numpy(inp.topk_w).to(dev)
    d_x = torch.from_numpy(inp.x.view(np.int16)).to(dev)
    if args.adapters:  # needs no expert outputs
        print(json.dumps(run_adapters(args, wl, cfg, d_idx, d_w, d_x, bufs, torch.cuda.current_stream())),
              flush=True)
        return
    if wl.expert_output == "random":
        y = W.expert_outputs(wl, inp)
    else:  # outputs that follow the rows' experts: take the row map from the library
        M.moe_dispatch_layout(cfg, wl.T, d_idx, bufs.handle, bufs.workspace)
        torch.cuda.synchronize()
        y = W.expert_outputs(wl, inp, bufs.handle.row_to_pair.cpu().numpy())
    d_y = torch.from_numpy(y.view(np.int16)).to(dev)
    d_out = torch.empty((wl.T, wl.H), dtype=torch.int16, device=dev)
    T = wl.T
    stream = torch.cuda.current_stream()
    if args.dedup:
        print(json.dumps(run_dedup(args, wl, cfg, d_idx, d_w, d_x, d_y, d_out, bufs, stream)), flush=True)
        return

    fused = not args.separate

    def layout_dispatch(st):
        if fused:  # the layout is inferred inside the dispatch call
            M.moe_dispatch_fused(cfg, T, d_idx, d_x, None, bufs.handle, bufs.workspace, bufs.out_x,
                                 bufs.out_scale, None, st)
        else:
            M.moe_dispatch_layout(cfg, T, d_idx, bufs.handle, bufs.workspace, st)
            M.moe_dispatch(cfg, T, d_x, None, bufs.handle, bufs.out_x, bufs.out_scale, None, st)

    def combine(st):
        M.moe_combine(cfg, T, d_y, d_w, bufs.handle, d_out, st)

    enqueue_ms = []  # host time to issue one step, per eager run

    def new_events(n):
        """n timing events, created (first record) before any timed region."""
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(n)]
        for e in evs:
            e.record(stream)
        torch.cuda.synchronize()
        return evs

    # cold caches: before each headline step an untimed read of a scratch
    # buffer larger than L2 plus the 256 MB Infinity Cache evicts what the
    # step reads.  The flush reads rather than writes: a written scratch would
    # leave the cache full of dirty lines whose write-back the step would pay
    # for, which is not the path's own cost.
    scratch = torch.ones(max(args.flush_mib, 1) << 18, dtype=torch.int32, device=dev)

    def flush():
        return scratch.sum()  # on the current stream, which the library calls use too

    graph = None
    if args.graph:  # one step captured on a side stream, replayed on this one
        side = torch.cuda.Stream()
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            layout_dispatch(side)
            combine(side)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            cap = torch.cuda.current_stream()
            for _ in range(args.graph_steps):
                layout_dispatch(cap)
                combine(cap)
        torch.cuda.synchronize()

    def run_step(st):
        if graph is not None:
            graph.replay()
        else:
            layout_dispatch(st)
            combine(st)

    def timed_steps(n, cold, split=False):
        """n steps between two device synchronisations.  With `cold`, each
        step follows an untimed flush and is bracketed by HIP events on the
        launch stream; back to back, two events bracket all n steps.  With
        `split` (eager steps only), every step also gets an event between its
        dispatch and combine calls, for the per-call times: an event between
        two kernels waits for the first one's end-of-kernel cache write-back
        (3-6 us on the DeepSeek-V3 prefill batch), so the step times come from
        runs without one.  Returns per-step, per-dispatch and per-combine
        event times (ms) and the wall time of the whole region (flushes
        included)."""
        per = args.graph_steps if graph is not None else 1  # steps per replay
        n = -(-n // per)
        beg, mid, end = new_events(n), new_events(n) if split else None, new_events(n)
        flushed = None
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        h0 = time.perf_counter()
        for i in range(n):
            if cold:
                flushed = flush()
            if cold or split or i == 0:
                beg[i].record(stream)
            if graph is not None:
                graph.replay()
            else:
                layout_dispatch(stream)
                if split:
                    mid[i].record(stream)
                combine(stream)
            if cold or split or i == n - 1:
                end[i].record(stream)
        if not cold and not split:
            enqueue_ms.append((time.perf_counter() - h0) * 1e3 / n)
        torch.cuda.synchronize()
        wall_s = time.perf_counter() - w0
        if flushed is not None:
            assert int(flushed.item()) == scratch.numel()
        if cold or split:
            step = [beg[i].elapsed_time(end[i]) / per for i in range(n)]
        else:  # back to back: the mean step is the span of all steps over their number
            step = [beg[0].elapsed_time(end[n - 1]) / (n * per)] * n
        if not split:
            return step, None, None, wall_s
        return (step, [beg[i].elapsed_time(mid[i]) for i in range(n)],
                [mid[i].elapsed_time(end[i]) for i in range(n)], wall_s)

    # warmup
    log(f"[bench] warmup {args.warmup} steps ({'fused' if fused else 'separate'} dispatch"
        f"{', graph replay' if graph is not None else ''})")
    for _ in range(args.warmup):
        run_step(stream)
    torch.cuda.synchronize()

    # timed region: exactly K steps between two device synchronisations.  The
    # headline steps run with cold caches (an untimed flush before each);
    # ms_per_step is the mean HIP-event time of the steps themselves.  With
    # --flush-mib 0 the headline steps run back to back instead.
    cold_headline = args.flush_mib > 0
    log(f"[bench] timing {args.steps} steps ({'each after a cache flush' if cold_headline else 'back to back'})")
    step_ms, _, _, wall = timed_steps(args.steps, cold_headline)
    ms_step = float(np.mean(step_ms))
    # secondary: the same number of steps back to back (the inputs stay
    # cached from step to step as far as the traffic in between allows)
    warm = None
    if cold_headline and not args.no_warm:
        log(f"[bench] timing {args.steps} steps back to back (warm caches)")
        w_step, _, _, w_wall = timed_steps(args.steps, False)
        w_ms = float(np.mean(w_step))  # span of the back-to-back steps over their number (HIP events)
        warm = {"ms_per_step": w_ms, "wall_ms_per_step": w_wall * 1e3 / args.steps, "tokens_per_s": T / (w_ms * 1e-3)}
    # per-call times (and the roofline's combine duration): the same steps,
    # eager, under the headline's cache condition, with an event between the
    # calls of each step
    log(f"[bench] timing {args.steps} steps with an event between the calls (per-call times)")
    saved, graph = graph, None
    split_step_ms, dispatch_ms, combine_ms, _ = timed_steps(args.steps, cold_headline, split=True)
    graph = saved

    # after the timed region: the same step as separate calls, each bracketed
    # by events (back to back), for the per-call breakdown
    n_sep = 0 if args.no_breakdown else min(args.steps, 50)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_sep)]
    for i in range(n_sep):
        ev[i][0].record(stream)
        M.moe_dispatch_layout(cfg, T, d_idx, bufs.handle, bufs.workspace, stream)
        ev[i][1].record(stream)
        M.moe_dispatch(cfg, T, d_x, None, bufs.handle, bufs.out_x, bufs.out_scale, None, stream)
        ev[i][2].record(stream)
        combine(stream)
        ev[i][3].record(stream)
    torch.cuda.synchronize()
    sep = {k: (float(np.mean([ev[i][j].elapsed_time(ev[i][j + 1]) for i in range(n_sep)])) if n_sep else None)
           for j, k in enumerate(("layout", "dispatch", "combine"))}
    # the headline step's own outputs for the oracle check below
    if cold_headline:
        flush()
    run_step(stream)
    torch.cuda.synchronize()

    per_ms = {"layout+dispatch": float(np.mean(dispatch_ms)), "combine": float(np.mean(combine_ms))}
    per_med = {"layout+dispatch": float(np.median(dispatch_ms)), "combine": float(np.median(combine_ms))}
    per_p10_p90 = {k: [float(np.percentile(v, 10)), float(np.percentile(v, 90))]
                   for k, v in (("layout+dispatch", dispatch_ms), ("combine", combine_ms))}

    status = bufs.handle.status.cpu().numpy()
    n_kept = int(bufs.handle.recv_count.cpu().numpy().sum())
    ab = algorithmic_bytes(wl, n_kept)
    total_bytes = sum(ab.values())
    gbs = {"layout+dispatch": (ab["layout"] + ab["dispatch"]) / (per_ms["layout+dispatch"] * 1e-3) / 1e9,
           "combine": ab["combine"] / (per_ms["combine"] * 1e-3) / 1e9}
    sep_gbs = {k: ab[k] / (sep[k] * 1e-3) / 1e9 for k in ab if sep[k]}
    path_gbs = total_bytes / (ms_step * 1e-3) / 1e9
    if warm is not None:
        warm["gbs"] = total_bytes / (warm["ms_per_step"] * 1e-3) / 1e9
        warm["frac_of_peak"] = warm["gbs"] / HBM_PEAK_GBS
    del scratch

    copy_gbs = copy_ceiling(args.calib_copy_mib, dev, stream)

    traffic = measured_traffic("combine_kernel", wl.name)
    result = {
        "metric": "dispatch+combine tokens/s and achieved HBM GB/s (% of peak), DSV3 shape",
        "value": T / (ms_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",  # scales and the weighted sum are computed in fp32; the layout in int32
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": T, "hidden": wl.H, "experts": wl.E,
                   "topk": wl.K, "virtual_ranks": wl.R,
                   "io": ("bf16 tokens and expert outputs, " +
                          ("e4m3 dispatched rows" if wl.quant != W.QUANT_NONE else "bf16 dispatched rows") +
                          ", bf16 combined rows"),
                   "layout": "contiguous" if wl.layout == W.LAYOUT_CONTIGUOUS else "masked",
                   "align": wl.align, "capacity": wl.capacity, "quant": QUANT_NAME[wl.quant],
                   "num_cus": args.num_cus,
                   "caches": (f"cold: each timed step follows an untimed {args.flush_mib} MiB read"
                              if cold_headline else "warm: steps back to back")},
        "library_sha256": library_hash(),
        "roofline": {"bound": "hbm", "kernel": "combine_kernel",
                     "achieved": gbs["combine"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs["combine"] / HBM_PEAK_GBS, "traffic": traffic},
        "path": {"calls": ("moe_dispatch_fused + moe_combine" if fused else
                           "moe_dispatch_layout + moe_dispatch + moe_combine")
                          + (f", HIP graph replays of {args.graph_steps} step(s)" if args.graph else ""),
                 "algorithmic_bytes": ab, "gbs": path_gbs, "frac_of_peak": path_gbs / HBM_PEAK_GBS,
                 "ms_per_step_median": float(np.median(step_ms)),
                 "ms_per_step_p10_p90": [float(np.percentile(step_ms, 10)), float(np.percentile(step_ms, 90))],
                 "timed_region_wall_s": wall,
                 "per_call_ms_mean": per_ms, "per_call_ms_median": per_med,
                 "ms_per_step_with_call_events": float(np.mean(split_step_ms)),
                 "per_call_ms_p10_p90": per_p10_p90, "per_call_gbs": gbs,
                 "separate_calls_ms_mean": sep, "separate_calls_gbs": sep_gbs,
                 "host_enqueue_ms_per_step": enqueue_ms[0] if enqueue_ms else None, "kept_pairs": n_kept,
                 "status": status.tolist(), "copy_ceiling_gbs": copy_gbs, "warm_caches": warm},
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle), and the last step's outputs against it")
        gpu = {k: v.cpu().numpy() for k, v in bufs.handle.tensors().items()}
        gpu["out_x"] = bufs.out_x.cpu().numpy().view(np.uint8)
        gpu["out_scale"] = None if bufs.out_scale is None else bufs.out_scale.cpu().numpy().view(np.uint8)
        gpu["out"] = d_out.cpu().numpy().view(np.uint16)
        result["cpu_baseline"] = cpu_baseline(wl, inp, y, args.cpu_sample_tokens, gpu)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
