#!/usr/bin/env python3
"""Benchmark of one GPU's share of MoE EP dispatch + combine on an MI355X.

A step is one pass of the whole path -- COUNT, SCAN, FINALIZE (epdc_dispatch)
then COMBINE (epdc_combine) -- over one batch of seeded synthetic input that
is already resident in HBM.  The headline workload is the 4096-token,
hiddenDim-7168 configuration (worldSize 8, 32 experts per rank, topk 8,
Zipf(1.1) expert popularity, softmax weights).

Prints one JSON line: whole-job HBM throughput from the algorithmic bytes of
a step and the time per step (events around the timed loop only), a roofline
entry for the dominant kernel (each kernel then timed alone over the same
number of back-to-back launches, HIP events on the launch stream), the CPU
oracle timed on a bounded sample of the same workload, and the same
measurements for every other configuration (config.all_configs).  Input
sets are rotated step by step, as many as it takes to make each measured
working set exceed twice the 256 MB Infinity Cache, so that no step finds
its data there.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)
sys.path.insert(0, os.path.join(ROOT, "tests"))

METRIC = "dispatch+combine µs and achieved HBM GB/s (% of peak), 1×MI355X"
HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
COLD_BYTES = 2 * MALL_BYTES  # rotated working set of every measurement
PROFILES = os.path.join(ROOT, "profiles")
KERNEL_SOURCES = [os.path.join(ROOT, "combine_count_amd", "csrc", f)
                  for f in ("dispatch.hip", "combine.hip", "combine_push.hip", "epdc_internal.h")]
# the other configurations, measured after the headline one
SWEEP = ["tiny", "pr_scale", "epcfg_defaults", "gen_zipf_h2048", "gen_edge_t1", "gen_edge_t8",
         "large_unweighted", "large_weighted"]


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
    ap.add_argument("--combine-dtype", default="bf16", choices=["bf16", "fp32"], help="returned-row type")
    ap.add_argument("--out-dtype", default="", choices=["", "bf16", "fp32"],
                    help="combine output type (default: the returned-row type)")
    ap.add_argument("--scale-dim", type=int, default=0, help="fp32 scales per token forwarded by the dispatch")
    ap.add_argument("--combine", default="gather", choices=["gather", "push"],
                    help="gather combine (one kernel) or scatter combine (push + reduce kernels)")
    ap.add_argument("--rotate", type=int, default=0,
                    help="independent buffer sets (inputs and outputs) cycled step by step; 0 (default) = as "
                         "many as make the rotated bytes exceed 512 MB, twice the Infinity Cache; 1 = hot")
    ap.add_argument("--sweep", type=int, default=1,
                    help="1: also measure every other configuration (config.all_configs); 0: headline only")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="wall-clock budget of the CPU-oracle sample (0 disables it)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="also run a plain torch device copy of MIB MiB 5 times first: the known-size "
                         "kernel that scales rocprofv3 FETCH_SIZE / WRITE_SIZE readings")
    return ap.parse_args()


def row_bytes(w):
    """Bytes of a dispatch row, a returned (combine input) row and an output row."""
    import workloads
    out = {"bf16": 2, "fp32": 4}[w.outType]
    return (w.dispatchHidden * workloads.WIRE_BYTES[w.wire], w.hiddenDim * workloads.WIRE_BYTES[w.combineDtype],
            w.hiddenDim * out)


def algorithmic_bytes(w, U):
    """Bytes the method must move (each input read once, each output written
    once); U = unique (token, PE) pairs of the seeded input."""
    T, K, W, S = w.numTokens, w.numExpertPerToken, w.worldSize, w.scaleDim
    xr, yr, orow = row_bytes(w)
    wt = 1 if w.useWeights else 0
    disp = (T * xr + T * K * 4 + wt * T * K * 4 + T * S * 4          # x, expertIds, weights, scales
            + U * xr + U * 4 + U * K * 4 + wt * U * K * 4 + U * S * 4  # rows, token idx, ids, weights, scales
            + T * K * 4 + W * 4)                                       # sendMap, recvCount
    comb = T * K * 4 + wt * (T * K * 4 + T * K * 4) + U * yr + T * orow
    return disp, comb


def push_bytes(w, U):
    """Algorithmic bytes of the scatter combine's two kernels.  Push: each
    landed row read and written once, with (weighted) its K ids and weights
    read and one scale written; the W counts.  Reduce: the token's sendMap,
    the counts, each landed row and scale read once, the out row written."""
    T, K, W = w.numTokens, w.numExpertPerToken, w.worldSize
    _, yr, orow = row_bytes(w)
    wt = 1 if w.useWeights else 0
    push = 2 * U * yr + wt * (U * K * 8 + U * 4) + W * 4
    red = T * K * 4 + W * 4 + U * yr + wt * U * 4 + T * orow
    return push, red


def set_bytes(w, push):
    """Device bytes of one buffer set (inputs, outputs, landing rows)."""
    T, K, W, M, S = w.numTokens, w.numExpertPerToken, w.worldSize, w.maxTokPerRank, w.scaleDim
    xr, yr, orow = row_bytes(w)
    b = T * xr + T * K * 8 + T * S * 4 + W * M * (xr + yr + 4 + K * 8 + S * 4) + T * K * 4 + T * orow
    if push:
        b += T * min(W, K) * (yr + 4)
    return b


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


def cpu_baseline(w, inp, budget_s, step_b, push):
    """The oracle, single-threaded, on whole steps of the workload for about
    budget_s seconds: the median step time gives the rate, the fastest and
    slowest steps the spread."""
    import oracle
    step, _ = oracle.timed_step(w.worldSize, w.maxTokPerRank, w.numExpertPerRank, w.numExpertPerToken,
                                w.useWeights, inp.x, inp.expertIds, inp.weights, inp.y, push=push,
                                scales=inp.scales, out_fp32=w.outType == "fp32")
    step()  # untimed: page in the buffers
    times, t0 = [], time.perf_counter()
    while True:
        a = time.perf_counter()
        step()
        times.append(time.perf_counter() - a)
        el = time.perf_counter() - t0
        if el >= budget_s or len(times) >= 1000:
            break
    med = statistics.median(times)
    what = "dispatch+push+reduce" if push else "dispatch+combine"
    return {"value": round(step_b / med / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{len(times)} whole {what} steps of {w.name} (seed {inp.seed}), the single-threaded C "
                      f"oracle as it stands, {el:.1f} s wall; value from the median step",
            "ms_per_step_median": round(med * 1e3, 2),
            "ms_per_step_min_max": [round(min(times) * 1e3, 2), round(max(times) * 1e3, 2)],
            "steps_timed": len(times), "host": host_cpu()}


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


def cacheable_bytes(w):
    """Bytes of one buffer set that the path reads or writes with plain
    (cache-allocating) accesses and that the next use of the set would find
    again: the token inputs (x, ids, weights, scales), sendMap and the
    received rows' metadata (at most min(W, K) rows per token).  The row
    copies themselves use non-temporal accesses, which do not keep a set's
    data in the 256 MB memory-side cache; x did stay there between uses of a
    set when only the whole step's bytes were counted (4096 tokens x h7168:
    dispatch 40.1 us with 3 sets, 54.0 with 6, 55.6 with 10)."""
    T, K, W, S = w.numTokens, w.numExpertPerToken, w.worldSize, w.scaleDim
    xr, _, _ = row_bytes(w)
    u_max = T * min(W, K)
    return T * (xr + K * 8 + S * 4) + T * K * 4 + u_max * (4 + K * 8 + S * 4)


def rotation(torch, w, push, requested):
    """Buffer sets to cycle: the requested number, or as many as make the
    cacheable bytes of the rotated sets exceed COLD_BYTES (at least 3, and at
    least 2 where memory allows no more), within 1024 sets, 24 GB of buffers
    and half the free device memory.  Configurations of a few tokens touch
    too little to leave the cache that way (they are bound by launch
    latency, not bytes)."""
    b = set_bytes(w, push)
    if requested > 0:
        return requested
    free, _ = torch.cuda.mem_get_info()
    n = max(3, math.ceil(COLD_BYTES / max(cacheable_bytes(w), 1)))
    return max(1, min(n, 1024, int((24 << 30) // b), int(free * 0.5 // b)))


# Launches per loop of the per-kernel durations and graph replays (and the
# warmup and steps of the other configurations): at least this many whatever
# --steps says, so that a short timed region (--steps 20) does not leave
# microsecond kernels measured over 20 launches, where the loop's start and
# end dominate.
MIN_AUX_STEPS = 200
MIN_SWEEP_WARMUP = 50


def measure(torch, w, inp, args, push, headline=False):
    """Every figure of one workload: the timed step loop, per-kernel
    back-to-back durations, the graph-replayed step and (headline) the
    spread and a hot loop.  The headline's timed loop (and its repeats and
    hot loop) is exactly --steps steps after --warmup warmup steps; the
    other loops, and every loop of the other configurations, take at least
    MIN_AUX_STEPS launches (the other configurations warm up for at least
    MIN_SWEEP_WARMUP steps)."""
    from gpu_harness import DeviceRun
    nsets = rotation(torch, w, push, args.rotate)
    sets = [DeviceRun(w, inp) for _ in range(nsets)]
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
    steps = args.steps if headline else max(args.steps, MIN_AUX_STEPS)
    aux = max(args.steps, MIN_AUX_STEPS)
    warmup = args.warmup if headline else max(args.warmup, MIN_SWEEP_WARMUP)
    for i in range(warmup):
        step(sets[i % nsets])
    torch.cuda.synchronize()

    def loop_ms(run, sel, n):
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(n):
            run(sel(i))
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / n

    # Timed region: exactly `steps` steps between two events, nothing else on
    # the stream (per-launch events cost about 10 us a step on this stack).
    ms_step = loop_ms(step, lambda i: sets[i % nsets], steps)
    res = {"U": U, "stages": stages, "step_b": step_b, "ms_step": ms_step, "sets": nsets,
           "rotated_bytes": nsets * step_b, "warmup": warmup, "steps": steps, "aux_launches": aux}
    if headline:
        # Spread and cache state, beside `value` (the loop above alone): the
        # same cold loop four more times, then `steps` steps on one set.
        res["repeats"] = [ms_step] + [loop_ms(step, lambda i: sets[i % nsets], steps) for _ in range(4)]
        res["hot_ms"] = loop_ms(step, lambda i: sets[0], steps)
    # Per-kernel durations: each kernel alone, `aux` launches back to back
    # over the same rotating sets, between two HIP events on the launch stream
    # (an event pair around every launch adds ~2 us to each reading).
    res["kern_ms"] = {name: loop_ms(run, lambda i: sets[i % nsets], aux) for name, run, _ in stages}
    # Launch latency: `aux` steps captured once into a HIP graph and
    # replayed, which takes the per-launch host cost (Python, ctypes, the HIP
    # launch call) out of the step; at a few tokens that cost is the step.
    graph = torch.cuda.CUDAGraph()
    cap = torch.cuda.Stream()
    cap.wait_stream(stream)
    with torch.cuda.stream(cap):
        with torch.cuda.graph(graph, stream=cap):
            for i in range(aux):
                step(sets[i % nsets])
    stream.wait_stream(cap)
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    g0.record(stream)
    graph.replay()
    g1.record(stream)
    torch.cuda.synchronize()
    res["graph_ms"] = g0.elapsed_time(g1) / aux
    del graph
    res["scratch_ok"] = all(s.scratch_clean() for s in sets)
    del sets, g
    torch.cuda.empty_cache()
    return res


def summary(w, r):
    """The per-configuration entry of config.all_configs."""
    kern = {n: {"us": round(r["kern_ms"][n] * 1e3, 2), "algorithmic_bytes": b,
                "GB/s": round(b / r["kern_ms"][n] / 1e6, 1),
                "frac": round(b / r["kern_ms"][n] / 1e6 / HBM_PEAK_GBPS, 4)} for n, _, b in r["stages"]}
    return {"numTokens": w.numTokens, "worldSize": w.worldSize, "numExpertPerRank": w.numExpertPerRank,
            "numExpertPerToken": w.numExpertPerToken, "hiddenDim": w.hiddenDim, "maxTokPerRank": w.maxTokPerRank,
            "routing": w.routing, "useWeights": w.useWeights, "unique_token_pe_pairs": r["U"],
            "step_us": round(r["ms_step"] * 1e3, 2), "step_GB/s": round(r["step_b"] / r["ms_step"] / 1e6, 1),
            "graph_replay_step_us": round(r["graph_ms"] * 1e3, 2), "kernels": kern,
            "buffer_sets_rotated": r["sets"], "rotated_step_bytes": r["rotated_bytes"],
            "warmup": r["warmup"], "steps": r["steps"], "scratch_clean": r["scratch_ok"]}


def main():
    args = parse_args()
    if args.steps < 1 or args.warmup < 0:
        print("bench.py: --steps must be >= 1 and --warmup >= 0", file=sys.stderr)
        return 2
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus}: the library runs one GPU's share of dispatch/combine on a "
              "single GPU; multi-GPU runs are not part of it.", file=sys.stderr)
        return 2
    import torch

    import combine_count_amd as epdc  # noqa: F401  (fails loudly if the library is not built)
    import workloads

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

    push = args.combine == "push"

    def variant(w):
        over = dict(wire=args.wire, combineDtype=args.combine_dtype, outDtype=args.out_dtype,
                    scaleDim=args.scale_dim)
        tag = "" if (args.wire, args.combine_dtype) == ("bf16", "bf16") else f"_{args.wire}_{args.combine_dtype}"
        tag += f"_out{args.out_dtype}" if args.out_dtype else ""
        tag += f"_s{args.scale_dim}" if args.scale_dim else ""
        tag += "_push" if push else ""
        return w.with_(name=w.name + tag, **over)

    w = variant(workloads.CONFIGS[args.workload])
    print(f"[bench] generating {w.name} seed {args.seed}", file=sys.stderr, flush=True)
    inp = workloads.make_inputs(w, args.seed)
    r = measure(torch, w, inp, args, push, headline=True)
    stages, U, step_b, ms_step, kern_ms = r["stages"], r["U"], r["step_b"], r["ms_step"], r["kern_ms"]
    print(f"[bench] U={U} " + ", ".join(f"{n} {kern_ms[n] * 1e3:.1f} us ({b / kern_ms[n] / 1e6:.0f} GB/s)"
                                        for n, _, b in stages)
          + f", step {ms_step * 1e3:.1f} us, graph-replayed step {r['graph_ms'] * 1e3:.1f} us, "
            f"{r['sets']} sets rotated ({r['rotated_bytes'] / 1e6:.0f} MB touched per cycle)", file=sys.stderr, flush=True)

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
    del inp

    all_configs = {}
    if args.sweep:
        for name in SWEEP:
            if name == args.workload:
                continue
            wc = variant(workloads.CONFIGS[name])
            inc = workloads.make_inputs(wc, args.seed)
            rc = measure(torch, wc, inc, args, push)
            del inc
            all_configs[name] = summary(wc, rc)
            print(f"[bench] {name}: step {all_configs[name]['step_us']} us, graph {rc['graph_ms'] * 1e3:.2f} us, "
                  + ", ".join(f"{n} {v['us']} us ({v['frac']:.3f})" for n, v in all_configs[name]["kernels"].items()),
                  file=sys.stderr, flush=True)

    value = step_b / (ms_step * 1e-3) / 1e9
    config = {"workload": w.name, "worldSize": w.worldSize, "numExpertPerRank": w.numExpertPerRank,
              "numTokens": w.numTokens, "maxTokPerRank": w.maxTokPerRank,
              "numExpertPerToken": w.numExpertPerToken, "hiddenDim": w.hiddenDim,
              "routing": w.routing + ("(s=1.1)" if w.routing == "zipf" else ""),
              "useWeights": w.useWeights, "scaleDim": w.scaleDim, "seed": args.seed, "unique_token_pe_pairs": U,
              "dispatch_dtype": w.wire, "combine_dtype": w.combineDtype, "out_dtype": w.outType,
              "combine_accumulate": "fp32", "combine": "scatter (push + reduce)" if push else "gather",
              "bytes_per_step": step_b}
    config.update({f"{n}_us": round(kern_ms[n] * 1e3, 2) for n, _, _ in stages})
    config["kernels"] = {n: {"us": round(kern_ms[n] * 1e3, 2), "algorithmic_bytes": b,
                             "GB/s": round(b / kern_ms[n] / 1e6, 1),
                             "frac": round(b / kern_ms[n] / 1e6 / HBM_PEAK_GBPS, 4),
                             "traffic": read_traffic(n, w.name)} for n, _, b in stages}
    config.update({"step_us_cold_repeats": [round(m * 1e3, 2) for m in r["repeats"]],
                   "step_us_hot": round(r["hot_ms"] * 1e3, 2),
                   "graph_replay_step_us": round(r["graph_ms"] * 1e3, 2),
                   "buffer_sets_rotated": r["sets"], "rotated_step_bytes": r["rotated_bytes"],
                   "scratch_clean": r["scratch_ok"],
                   "per_kernel_and_graph_launches": r["aux_launches"],
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBPS, 4),
                   "stream_reference_GBps": dict(ref, what="torch copy_ (1 GiB read + 1 GiB written) and fill_ "
                                                           "(1 GiB written) on the same GPU, 20 launches each")
                   if ref else None,
                   "all_configs": all_configs})
    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.wire if w.wire == w.combineDtype == w.outType else f"{w.wire}+{w.combineDtype}->{w.outType}",
        "data": "synthetic",
        "config": config,
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
