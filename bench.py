#!/usr/bin/env python3
"""Benchmark of one GPU's share of MoE EP dispatch + combine on an MI355X.

A step is one pass of the whole path -- COUNT, SCAN, FINALIZE (epdc_dispatch)
then COMBINE (epdc_combine) -- over one batch of seeded synthetic input that
is already resident in HBM.  The default workload is the 4096-token,
hiddenDim-7168 configuration (worldSize 8, 32 experts per rank, topk 8,
Zipf(1.1) expert popularity, softmax weights).

Prints one JSON line: whole-job HBM throughput from the algorithmic bytes of
a step and the time per step (events around the timed loop only), a roofline
entry for the dominant kernel (HIP events around each launch, in a second
pass over the same steps) and the CPU oracle timed on a bounded sample of the
same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = "dispatch+combine µs and achieved HBM GB/s (% of peak), 1×MI355X"
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "combine_count_amd", "csrc", f)
                  for f in ("dispatch.hip", "combine.hip", "epdc_internal.h")]


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="gen_zipf_h7168")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--wire", default="bf16", choices=["bf16", "fp32", "fp8", "fp4x2"],
                    help="dispatch row type (fp8/fp4x2: narrow wire, hiddenDim in bytes for fp4x2)")
    ap.add_argument("--combine-dtype", default="bf16", choices=["bf16", "fp32"])
    ap.add_argument("--rotate", type=int, default=3,
                    help="independent buffer sets (inputs and outputs) cycled step by step, so that a "
                         "step never finds its data in the 256 MB Infinity Cache (1 = hot)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the CPU-oracle sample (0 disables it)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain torch device copy of MIB MiB 5 times first: the known-size "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    return ap.parse_args()


def algorithmic_bytes(w, U):
    """Bytes the method must move (each input read once, each output written
    once); U = unique (token, PE) pairs of the seeded input."""
    import workloads
    T, K, W = w.numTokens, w.numExpertPerToken, w.worldSize
    xr = w.dispatchHidden * workloads.WIRE_BYTES[w.wire]       # dispatch row bytes
    yr = w.hiddenDim * workloads.WIRE_BYTES[w.combineDtype]    # combine row bytes
    wt = 1 if w.useWeights else 0
    disp = (T * xr + T * K * 4 + wt * T * K * 4               # x, expertIds, weights
            + U * xr + U * 4 + U * K * 4 + wt * U * K * 4     # rows, token idx, ids, weights
            + T * K * 4 + W * 4)                               # sendMap, recvCount
    comb = T * K * 4 + wt * (T * K * 4 + T * K * 4) + U * yr + T * yr
    return disp, comb


def kernel_source_hash():
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def read_traffic(kernel, workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None if there is none or the kernels changed since it was taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as f:
        for line in f:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def cpu_baseline(w, inp, budget_s, disp_b, comb_b):
    import oracle
    step, _ = oracle.timed_step(w.worldSize, w.maxTokPerRank, w.numExpertPerRank, w.numExpertPerToken,
                                w.useWeights, inp.x, inp.expertIds, inp.weights, inp.y)
    step()  # untimed: page in the buffers
    n, t0 = 0, time.perf_counter()
    while True:
        step()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 1000:
            break
    return {"value": round((disp_b + comb_b) * n / el / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} full dispatch+combine steps of {w.name} (seed {inp.seed}), single-threaded C "
                      f"oracle, {el:.1f} s wall",
            "ms_per_step": round(el / n * 1e3, 2)}


def main():
    args = parse_args()
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus}: this build runs one GPU's share of dispatch/combine on a "
              "single GPU; multi-GPU runs are not part of it.", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import combine_count_amd as epdc
    import workloads
    from gpu_harness import GpuRun

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(5):
            dst.copy_(src)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / 5
        print(f"[bench] copy calibration: {n} bytes read + {n} written, {ms * 1e3:.1f} us per copy, "
              f"{2 * n / ms / 1e6:.0f} GB/s", file=sys.stderr, flush=True)
        del src, dst

    w = workloads.CONFIGS[args.workload]
    if (args.wire, args.combine_dtype) != ("bf16", "bf16"):
        w = w.with_(name=f"{w.name}_{args.wire}_{args.combine_dtype}", wire=args.wire,
                    combineDtype=args.combine_dtype)
    print(f"[bench] generating {w.name} seed {args.seed}", file=sys.stderr, flush=True)
    inp = workloads.make_inputs(w, args.seed)
    sets = [GpuRun(w, inp) for _ in range(max(1, args.rotate))]
    g = sets[0]
    g.dispatch()
    g.combine()
    torch.cuda.synchronize()
    U = int(g.recvCount.sum().item())
    disp_b, comb_b = algorithmic_bytes(w, U)
    stream = torch.cuda.current_stream()

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        sets[i % len(sets)].dispatch()
        sets[i % len(sets)].combine()
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps between two events, nothing else on
    # the stream (per-launch events cost about 10 us a step on this stack).
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        s = sets[i % len(sets)]
        s.dispatch()
        s.combine()
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps

    # Per-kernel durations: the same steps again, with HIP events around each
    # launch on the launch stream.
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        s = sets[i % len(sets)]
        ev[i][0].record(stream)
        s.dispatch()
        ev[i][1].record(stream)
        s.combine()
        ev[i][2].record(stream)
    torch.cuda.synchronize()
    d_ms = float(np.mean([e[0].elapsed_time(e[1]) for e in ev]))
    c_ms = float(np.mean([e[1].elapsed_time(e[2]) for e in ev]))
    scratch_ok = all(s.scratch_clean() for s in sets)
    print(f"[bench] U={U} dispatch {d_ms * 1e3:.1f} us ({disp_b / d_ms / 1e6:.0f} GB/s), combine "
          f"{c_ms * 1e3:.1f} us ({comb_b / c_ms / 1e6:.0f} GB/s), step {ms_step * 1e3:.1f} us",
          file=sys.stderr, flush=True)

    if d_ms >= c_ms:
        dom, dom_b, dom_ms = "dispatch", disp_b, d_ms
    else:
        dom, dom_b, dom_ms = "combine", comb_b, c_ms
    achieved = dom_b / dom_ms / 1e6
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": read_traffic(dom, w.name),
                "us_per_launch": round(dom_ms * 1e3, 2), "algorithmic_bytes_per_launch": dom_b}

    cpu = None
    if args.cpu_seconds > 0:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, inp, args.cpu_seconds, disp_b, comb_b)

    value = (disp_b + comb_b) / (ms_step * 1e-3) / 1e9
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.wire if w.wire == w.combineDtype else f"{w.wire}+{w.combineDtype}",
        "data": "synthetic",
        "config": {"workload": w.name, "worldSize": w.worldSize, "numExpertPerRank": w.numExpertPerRank,
                   "numTokens": w.numTokens, "maxTokPerRank": w.maxTokPerRank,
                   "numExpertPerToken": w.numExpertPerToken, "hiddenDim": w.hiddenDim,
                   "routing": w.routing + ("(s=1.1)" if w.routing == "zipf" else ""),
                   "useWeights": w.useWeights, "seed": args.seed, "unique_token_pe_pairs": U,
                   "dispatch_dtype": w.wire, "combine_dtype": w.combineDtype,
                   "bytes_per_step": disp_b + comb_b,
                   "dispatch_us": round(d_ms * 1e3, 2), "combine_us": round(c_ms * 1e3, 2),
                   "buffer_sets_rotated": len(sets), "scratch_clean": scratch_ok,
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4)},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
