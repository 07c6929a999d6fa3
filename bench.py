#!/usr/bin/env python3
"""Benchmark of one GPU's share of MoE EP dispatch + combine on an MI355X.

A step is one pass of the whole path -- COUNT, SCAN, FINALIZE (epdc_dispatch)
then COMBINE (epdc_combine) -- over one batch of seeded synthetic input that
is already resident in HBM.  The default workload is the 4096-token,
hiddenDim-7168 configuration (worldSize 8, 32 experts per rank, topk 8,
Zipf(1.1) expert popularity, softmax weights).

Prints one JSON line: whole-job HBM throughput from the algorithmic bytes of
a step and the time per step (events around the timed loop only), a roofline
entry for the dominant kernel (each kernel then timed alone over the same
number of back-to-back launches, HIP events on the launch stream) and the CPU
oracle timed on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = "dispatch+combine µs and achieved HBM GB/s (% of peak), 1×MI355X"
HBM_PEAK_GBPS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "combine_count_amd", "csrc", f)
                  for f in ("dispatch.hip", "combine.hip", "combine_push.hip", "epdc_internal.h")]


def parse_args():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300,
                    help="untimed steps first (300, ~25 ms: with 20 the first timed loop ran ~0.7 us per step slower)")
    ap.add_argument("--workload", default="gen_zipf_h7168")
    ap.add_argument("--seed", type=int, default=1)
    ap.add_argument("--wire", default="bf16", choices=["bf16", "fp32", "fp8", "fp4x2"],
                    help="dispatch row type (fp8/fp4x2: narrow wire, hiddenDim in bytes for fp4x2)")
    ap.add_argument("--combine-dtype", default="bf16", choices=["bf16", "fp32"])
    ap.add_argument("--combine", default="gather", choices=["gather", "push"],
                    help="gather combine (one kernel) or scatter combine (push + reduce kernels)")
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


def push_bytes(w, U):
    """Algorithmic bytes of the scatter combine's two kernels.  Push: each
    landed row read and written once, with (weighted) its K ids and weights
    read and one scale written; the W counts.  Reduce: the token's sendMap,
    the counts, each landed row and scale read once, the out row written."""
    import workloads
    T, K, W = w.numTokens, w.numExpertPerToken, w.worldSize
    yr = w.hiddenDim * workloads.WIRE_BYTES[w.combineDtype]
    wt = 1 if w.useWeights else 0
    push = 2 * U * yr + wt * (U * K * 8 + U * 4) + W * 4
    red = T * K * 4 + W * 4 + U * yr + wt * U * 4 + T * yr
    return push, red


def kernel_source_hash():
    """sha256[:16] of the kernel sources' code: comments and whitespace are
    dropped first, so an edit of a comment does not void committed counters."""
    h = hashlib.sha256()
    for p in KERNEL_SOURCES:
        with open(p, encoding="utf-8") as f:
            code = re.sub(r"/\*.*?\*/|//[^\n]*", " ", f.read(), flags=re.S)
        h.update(" ".join(code.split()).encode())
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


def stream_reference(torch, nbytes=1 << 30, launches=20):
    """Plain streaming on the same GPU, for context beside the roofline: torch's
    device copy (nbytes read + nbytes written) and fill (nbytes written), GB/s
    over `launches` launches between two HIP events."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").random_(0, 255)
    dst = torch.empty_like(src)
    out = {}
    for name, run, moved in (("copy", lambda: dst.copy_(src), 2 * nbytes), ("fill", lambda: dst.fill_(7), nbytes)):
        for _ in range(3):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(launches):
            run()
        e1.record()
        torch.cuda.synchronize()
        out[name] = round(moved * launches / e0.elapsed_time(e1) / 1e6, 1)
    del src, dst
    torch.cuda.empty_cache()
    return out


def cpu_baseline(w, inp, budget_s, step_bytes, push):
    import oracle
    step, _ = oracle.timed_step(w.worldSize, w.maxTokPerRank, w.numExpertPerRank, w.numExpertPerToken,
                                w.useWeights, inp.x, inp.expertIds, inp.weights, inp.y, push=push)
    step()  # untimed: page in the buffers
    n, t0 = 0, time.perf_counter()
    while True:
        step()
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n >= 1000:
            break
    what = "dispatch+push+reduce" if push else "dispatch+combine"
    return {"value": round(step_bytes * n / el / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": f"{n} full {what} steps of {w.name} (seed {inp.seed}), single-threaded C "
                      f"oracle, {el:.1f} s wall",
            "ms_per_step": round(el / n * 1e3, 2),
            "host": host_cpu()}


def host_cpu():
    """The host the CPU figure was taken on: its CPU model, the cores the
    OS reports and the cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        usable = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        usable = None
    return {"cpu_model": model, "nproc": os.cpu_count(), "usable_cores": usable}


def main():
    args = parse_args()
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus}: the library runs one GPU's share of dispatch/combine on a "
              "single GPU; multi-GPU runs are not part of it.", file=sys.stderr)
        return 2
    import numpy as np
    import torch

    import combine_count_amd as epdc
    import workloads
    from gpu_harness import DeviceRun

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
    if args.combine == "push":
        w = w.with_(name=f"{w.name}_push")
    print(f"[bench] generating {w.name} seed {args.seed}", file=sys.stderr, flush=True)
    inp = workloads.make_inputs(w, args.seed)
    sets = [DeviceRun(w, inp) for _ in range(max(1, args.rotate))]
    push = args.combine == "push"
    for s in sets:
        if push:
            s.alloc_landing()
        s.prepare()  # launch loops reuse the buffers: arguments marshalled once per entry point
    g = sets[0]
    g.dispatch()
    torch.cuda.synchronize()
    U = int(g.recvCount.sum().item())
    disp_b, comb_b = algorithmic_bytes(w, U)
    # The kernels of one step, in order: (name, launch on a buffer set, algorithmic bytes per launch).
    if push:
        push_b, red_b = push_bytes(w, U)
        stages = [("dispatch", lambda s: s.p_dispatch(), disp_b), ("push", lambda s: s.p_push(), push_b),
                  ("reduce", lambda s: s.p_reduce(), red_b)]
    else:
        stages = [("dispatch", lambda s: s.p_dispatch(), disp_b), ("combine", lambda s: s.p_combine(), comb_b)]
    step_b = sum(b for _, _, b in stages)

    def step(s):
        for _, run, _ in stages:
            run(s)

    stream = torch.cuda.current_stream()
    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for i in range(args.warmup):
        step(sets[i % len(sets)])
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps between two events, nothing else on
    # the stream (per-launch events cost about 10 us a step on this stack).
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step(sets[i % len(sets)])
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step = t_start.elapsed_time(t_end) / args.steps

    # Spread and cache state, reported beside `value` (which is the loop above
    # alone): the same cold loop four more times, then `steps` steps on one
    # buffer set, whose ~490 MB then partly sit in the 256 MB Infinity Cache.
    def loop_ms(sel):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(args.steps):
            step(sel(i))
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    repeats = [ms_step] + [loop_ms(lambda i: sets[i % len(sets)]) for _ in range(4)]
    hot_ms = loop_ms(lambda i: sets[0])

    # Per-kernel durations: each kernel alone, `steps` launches back to back
    # over the same rotating buffer sets, between two HIP events on the launch
    # stream (an event pair around every launch adds ~2 us to each reading).
    def per_launch_ms(run):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(args.steps):
            run(sets[i % len(sets)])
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / args.steps

    kern_ms = {name: per_launch_ms(run) for name, run, _ in stages}

    # Launch latency: the same `steps` steps captured once into a HIP graph
    # and replayed, which takes the per-launch host cost (Python, ctypes, the
    # HIP launch call) out of the step; at a few tokens that cost is the step.
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(args.steps):
                step(sets[i % len(sets)])
    stream.wait_stream(cap)
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    graph_ms = g0.elapsed_time(g1) / args.steps
    del graph
    scratch_ok = all(s.scratch_clean() for s in sets)
    print(f"[bench] U={U} " + ", ".join(f"{n} {kern_ms[n] * 1e3:.1f} us ({b / kern_ms[n] / 1e6:.0f} GB/s)"
                                        for n, _, b in stages)
          + f", step {ms_step * 1e3:.1f} us, graph-replayed step {graph_ms * 1e3:.1f} us",
          file=sys.stderr, flush=True)

    dom, _, dom_b = max(stages, key=lambda st: kern_ms[st[0]])
    dom_ms = kern_ms[dom]
    achieved = dom_b / dom_ms / 1e6
    roofline = {"bound": "hbm", "kernel": dom, "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                "traffic": read_traffic(dom, w.name),
                "us_per_launch": round(dom_ms * 1e3, 2), "algorithmic_bytes_per_launch": dom_b}

    # (not in counter runs: their copies would mix with the calibration copy's)
    ref = None
    if not args.copy_calibration:
        ref = stream_reference(torch)
        print(f"[bench] stream reference: copy {ref['copy']:.0f} GB/s, fill {ref['fill']:.0f} GB/s",
              file=sys.stderr, flush=True)

    cpu = None
    if args.cpu_seconds > 0:
        print("[bench] timing the CPU oracle", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, inp, args.cpu_seconds, step_b, push)

    value = step_b / (ms_step * 1e-3) / 1e9
    config = {"workload": w.name, "worldSize": w.worldSize, "numExpertPerRank": w.numExpertPerRank,
              "numTokens": w.numTokens, "maxTokPerRank": w.maxTokPerRank,
              "numExpertPerToken": w.numExpertPerToken, "hiddenDim": w.hiddenDim,
              "routing": w.routing + ("(s=1.1)" if w.routing == "zipf" else ""),
              "useWeights": w.useWeights, "seed": args.seed, "unique_token_pe_pairs": U,
              "dispatch_dtype": w.wire, "combine_dtype": w.combineDtype, "combine_accumulate": "fp32",
              "combine": "scatter (push + reduce)" if push else "gather",
              "bytes_per_step": step_b}
    config.update({f"{n}_us": round(kern_ms[n] * 1e3, 2) for n, _, _ in stages})
    config["kernels"] = {n: {"us": round(kern_ms[n] * 1e3, 2), "algorithmic_bytes": b,
                             "GB/s": round(b / kern_ms[n] / 1e6, 1),
                             "frac": round(b / kern_ms[n] / 1e6 / HBM_PEAK_GBPS, 4),
                             "traffic": read_traffic(n, w.name)} for n, _, b in stages}
    config.update({"step_us_cold_repeats": [round(m * 1e3, 2) for m in repeats],
                   "step_us_hot": round(hot_ms * 1e3, 2),
                   "graph_replay_step_us": round(graph_ms * 1e3, 2),
                   "buffer_sets_rotated": len(sets), "scratch_clean": scratch_ok,
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
                   "stream_reference_GBps": dict(ref, what="torch copy_ (1 GiB read + 1 GiB written) and fill_ "
                                                           "(1 GiB written) on the same GPU, 20 launches each")
                   if ref else None})
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.wire if w.wire == w.combineDtype else f"{w.wire}+{w.combineDtype}",
        "data": "synthetic",
        "config": config,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
