#!/usr/bin/env python3
"""Benchmark: MoE dispatch + combine on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

One step is the whole path over one batch already resident in HBM:
moe_dispatch_layout (counts, offsets, maps) + moe_dispatch (row permutation
with fused FP8 quantization) + moe_combine (weighted top-k reduction), all
through the C ABI on torch's current stream.  The stand-in expert outputs y
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
              W.QUANT_FP8_UE8M0: "fp8_e4m3_ue8m0"}
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
    else:
        b_elt, scale_row = 1, 4 * ((nb + 3) // 4)
    layout = 4 * T * K + 4 * T * K + 4 * n_kept
    dispatch = 2 * T * H + 4 * T * K + n_kept * (H * b_elt + scale_row)
    combine = 2 * n_kept * H + 8 * T * K + 2 * T * H
    return {"layout": layout, "dispatch": dispatch, "combine": combine}


def kernel_source_hash(name):
    with open(os.path.join(ROOT, "combine_topk_idx_amd", "csrc", name), "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(kernel, source, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)[workload][kernel]
    except (OSError, KeyError, ValueError):
        return None
    if rec.get("source_sha256") != kernel_source_hash(source):
        return None
    return rec.get("bytes_per_launch")


def cpu_baseline(wl, inp, y, max_tokens):
    """The CPU oracle (single thread, as it stands) on a bounded sample: the
    first `max_tokens` tokens of the same batch, layout + dispatch + combine."""
    import oracle
    T = min(wl.T, max_tokens)
    sub = wl.replace(T=T)
    idx, w, x = inp.topk_idx[:T], inp.topk_w[:T], inp.x[:T]
    rows = sub.rows_capacity
    oracle._load()
    t0 = time.perf_counter()
    h = oracle.dispatch_layout(idx, wl.E, wl.R, wl.layout, wl.align, wl.capacity, rows_cap=rows)
    oracle.dispatch(x, h["pair_to_row"], wl.K, wl.quant, rows)
    oracle.combine(y[:rows], w, h["pair_to_row"])
    dt = time.perf_counter() - t0
    return {"value": T / dt, "unit": "tokens/s", "cores": 1, "kind": "oracle",
            "sample": f"first {T} of {wl.T} tokens of the same batch, one layout+dispatch+combine "
                      f"pass, single-threaded C oracle ({dt:.1f} s)"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=W.HEADLINE, choices=sorted(W.WORKLOADS))
    ap.add_argument("--num-cus", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-tokens", type=int, default=8192)
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run a plain device copy of this many MiB (counter calibration)")
    args = ap.parse_args()

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
    y = W.expert_outputs(wl, inp) if wl.expert_output == "random" else None
    if y is None:
        import oracle
        h = oracle.dispatch_layout(inp.topk_idx, wl.E, wl.R, wl.layout, wl.align, wl.capacity)
        y = W.expert_outputs(wl, inp, h["row_to_pair"])

    cfg = M.MoeConfig(max_tokens=wl.T, hidden=wl.H, num_experts=wl.E, num_topk=wl.K,
                      num_ranks=wl.R, layout=wl.layout, align=wl.align, capacity=wl.capacity,
                      quant=wl.quant, num_cus=args.num_cus)
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    bufs = M.DispatchBuffers(cfg, device=dev)
    d_idx = torch.from_numpy(inp.topk_idx).to(dev)
    d_w = torch.from_numpy(inp.topk_w).to(dev)
    d_x = torch.from_numpy(inp.x.view(np.int16)).to(dev)
    d_y = torch.from_numpy(y.view(np.int16)).to(dev)
    d_out = torch.empty((wl.T, wl.H), dtype=torch.int16, device=dev)
    T = wl.T
    stream = torch.cuda.current_stream()

    nev = args.steps
    ev = {k: [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
          for k in ("layout", "dispatch", "combine")}

    def step(i=None):
        if i is not None:
            ev["layout"][i].record(stream)
        M.moe_dispatch_layout(cfg, T, d_idx, bufs.handle, bufs.workspace, stream)
        if i is not None:
            ev["dispatch"][i].record(stream)
        M.moe_dispatch(cfg, T, d_x, None, bufs.handle, bufs.out_x, bufs.out_scale, None, stream)
        if i is not None:
            ev["combine"][i].record(stream)
        M.moe_combine(cfg, T, d_y, d_w, bufs.handle, d_out, stream)

    # warmup
    log(f"[bench] warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    ends = [torch.cuda.Event(enable_timing=True) for _ in range(nev)]
    log(f"[bench] timing {args.steps} steps")
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
        ends[i].record(stream)
    t_end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0

    ms_total = t_start.elapsed_time(t_end)
    ms_step = wall * 1e3 / args.steps
    per = {"layout": [], "dispatch": [], "combine": []}
    for i in range(args.steps):
        per["layout"].append(ev["layout"][i].elapsed_time(ev["dispatch"][i]))
        per["dispatch"].append(ev["dispatch"][i].elapsed_time(ev["combine"][i]))
        per["combine"].append(ev["combine"][i].elapsed_time(ends[i]))
    per_ms = {k: float(np.mean(v)) for k, v in per.items()}
    per_med = {k: float(np.median(v)) for k, v in per.items()}

    status = bufs.handle.status.cpu().numpy()
    n_kept = int(bufs.handle.recv_count.cpu().numpy().sum())
    ab = algorithmic_bytes(wl, n_kept)
    total_bytes = sum(ab.values())
    gbs = {k: ab[k] / (per_ms[k] * 1e-3) / 1e9 for k in ab}
    path_gbs = total_bytes / (ms_step * 1e-3) / 1e9

    # attainable ceiling next to it: a plain device copy of 1 GiB
    n_copy = (args.calib_copy_mib or 1024) * (1 << 20) // 4
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
    copy_gbs = 2 * n_copy * 4 * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
    del src, dst

    traffic = measured_traffic("moe_combine", "moe_combine.hip", wl.name)
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
        "dtype": "bf16 in, e4m3 dispatch, f32 accumulate" if wl.quant != W.QUANT_NONE
                 else "bf16 in, bf16 dispatch, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": wl.name, "tokens": T, "hidden": wl.H, "experts": wl.E,
                   "topk": wl.K, "virtual_ranks": wl.R,
                   "layout": "contiguous" if wl.layout == W.LAYOUT_CONTIGUOUS else "masked",
                   "align": wl.align, "capacity": wl.capacity, "quant": QUANT_NAME[wl.quant],
                   "num_cus": args.num_cus},
        "roofline": {"bound": "hbm", "kernel": "combine_kernel",
                     "achieved": gbs["combine"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": gbs["combine"] / HBM_PEAK_GBS, "traffic": traffic},
        "path": {"algorithmic_bytes": ab, "gbs": path_gbs, "frac_of_peak": path_gbs / HBM_PEAK_GBS,
                 "per_call_ms_mean": per_ms, "per_call_ms_median": per_med, "per_call_gbs": gbs,
                 "event_ms_per_step": ms_total / args.steps, "kept_pairs": n_kept,
                 "status": status.tolist(), "copy_ceiling_gbs": copy_gbs},
    }
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(wl, inp, y, args.cpu_sample_tokens)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
