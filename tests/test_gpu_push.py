"""Scatter (push) combine on an MI355X vs the CPU oracle, through the C ABI.

Push: the whole landing buffer (landed rows and the sentinel rows past the
landed total) and every forwarded scale, bit for bit.  Reduce: bit for bit
against the oracle reduce, and equal to the GPU gather combine of the same
rows.  Cases: every workload at full size, fp32 rows, and edge shapes (no
tokens, rows that are not whole 1 KiB chunks, more than 8 destinations, the
64-PE / 64-slot maximum, one PE, invalid expert ids); then two host-forced
conditions a dispatch never produces (counts past the landing capacity,
sendMap entries outside the windows) that must stay in bounds.
"""
import dataclasses

import numpy as np
import pytest
import torch

import combine_count_amd as epdc
import workloads
from gpu_harness import (SENT_LAND_BYTE, DeviceRun, assert_bits_equal, assert_dispatch_equal, assert_landing_equal,
                         oracle_combine, oracle_dispatch, oracle_push, oracle_reduce, out_as)

pytestmark = pytest.mark.gpu


def _check_push(w: workloads.Workload, inp: workloads.Inputs, tag: str):
    print(f"[push] {tag}: {w}", flush=True)
    g = DeviceRun(w, inp)
    g.alloc_landing()
    g.dispatch()
    torch.cuda.synchronize()
    o = oracle_dispatch(w, inp)
    assert_dispatch_equal(g, o, tag)
    g.push()
    torch.cuda.synchronize()
    land, sc = oracle_push(w, inp.y, o)
    assert_landing_equal(g, land, sc, tag)
    if w.numTokens == 0:
        return
    g.reduce()
    torch.cuda.synchronize()
    exp = oracle_reduce(w, land, sc, o)
    assert_bits_equal(out_as(g), exp, f"{tag} reduce")
    reduced = g.out.clone()
    g.combine()
    torch.cuda.synchronize()
    assert torch.equal(g.out, reduced), f"{tag}: reduce and gather combine differ on the GPU"


CONFIGS = ["tiny", "pr_scale", "epcfg_defaults", "gen_zipf_h2048", "gen_zipf_h7168", "gen_edge_t1",
           "gen_edge_t8", "large_unweighted", "large_weighted"]


@pytest.mark.parametrize("name", CONFIGS)
def test_push_config_parity(name):
    _check_push(workloads.CONFIGS[name], workloads.cached_inputs(name, 1), f"{name} seed 1")


EDGE = [
    # name, worldSize, numExpertPerRank, maxTokPerRank, numTokens, topk, hiddenDim, routing, useWeights
    ("empty", 4, 4, 64, 0, 2, 128, "uniform", 1),
    ("ragged_w5_epr3_h1056", 5, 3, 700, 650, 7, 1056, "uniform", 1),
    ("more_than_8_dest", 16, 2, 320, 300, 12, 512, "uniform", 1),
    ("max_w64_k64", 64, 1, 80, 70, 64, 64, "uniform", 1),
    ("single_pe", 1, 8, 96, 65, 3, 8, "uniform", 0),
    ("topk1", 8, 4, 200, 129, 1, 2048, "uniform", 1),
    ("m_gt_t", 8, 32, 4096, 777, 8, 7168, "zipf", 1),
    ("ragged_rows_9p5k", 8, 16, 200, 130, 8, 4864, "uniform", 0),
]


@pytest.mark.parametrize("case", EDGE, ids=[e[0] for e in EDGE])
def test_push_edge_parity(case):
    name, W, Epr, M, T, K, H, routing, useW = case
    w = workloads.Workload(name, W, Epr, M, T, K, H, routing, useW)
    _check_push(w, workloads.make_inputs(w, 6), name)


@pytest.mark.parametrize("base,wire", [("pr_scale", "fp32"), ("epcfg_defaults", "bf16"), ("tiny", "fp8")])
def test_push_fp32_rows(base, wire):
    w = workloads.CONFIGS[base].with_(name=f"{base}_fp32_push", wire=wire, combineDtype="fp32")
    _check_push(w, workloads.make_inputs(w, 7), w.name)


@pytest.mark.parametrize("base,rows,out", [("pr_scale", "bf16", "fp32"), ("epcfg_defaults", "fp32", "bf16"),
                                          ("gen_zipf_h7168", "bf16", "fp32")])
def test_push_reduce_output_types(base, rows, out):
    """The reduce writes either output type from either landing-row type,
    bit-identical to the gather combine's."""
    w = workloads.CONFIGS[base].with_(name=f"{base}_{rows}_rows_{out}_out", wire=rows, combineDtype=rows,
                                      outDtype=out)
    _check_push(w, workloads.make_inputs(w, 8), w.name)


def test_push_invalid_expert_ids():
    """Dropped slots (ids outside [0, E)) land no row and add no weight."""
    w = workloads.Workload("push_invalid_ids", 8, 4, 256, 250, 6, 1024, "uniform", 1)
    inp = workloads.make_inputs(w, 9)
    rng = np.random.Generator(np.random.PCG64(98))
    ids = inp.expertIds.copy()
    mask = rng.random(ids.shape) < 0.25
    bad = rng.choice(np.array([-1, -2, w.numExperts, 2**31 - 1, -(2**31)], dtype=np.int64), size=ids.shape)
    ids[mask] = bad[mask].astype(np.int32)
    ids[3, :] = -1
    _check_push(w, dataclasses.replace(inp, expertIds=ids), "push_invalid_ids")


def test_push_counts_past_capacity_stay_in_bounds():
    """Counts a dispatch never writes (every window full, plus a negative one)
    are clamped to [0, M] and nothing lands at or past T*min(W, K): guard
    rows after the landing buffer stay untouched, and the rows below it are
    the windows' rows in the clamped layout."""
    w = workloads.Workload("push_clamp", 4, 2, 64, 40, 2, 512, "uniform", 1)
    inp = workloads.make_inputs(w, 3)
    g = DeviceRun(w, inp)
    rows = epdc.epdc_landing_rows(g.ccfg, w.numTokens)
    assert rows == 80
    rowB = w.hiddenDim * 2
    guard = 16
    buf = torch.full((rows + guard, rowB), SENT_LAND_BYTE, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((rows + guard,), -3.25, dtype=torch.float32, device="cuda")
    g.landing, g.landScale = buf[:rows], sbuf[:rows]
    g.recvExpertIds.fill_(0)
    g.recvWeights.fill_(0.5)
    g.recvCount.copy_(torch.tensor([w.maxTokPerRank + 7, -5, 30, w.maxTokPerRank], dtype=torch.int32))
    g.push()
    torch.cuda.synchronize()
    b = buf.cpu().numpy()
    assert (b[rows:] == SENT_LAND_BYTE).all(), "push wrote past the landing capacity"
    assert (sbuf[rows:].cpu().numpy() == np.float32(-3.25)).all(), "push wrote a scale past the capacity"
    y = inp.y.view(np.uint8).reshape(w.worldSize, w.maxTokPerRank, rowB)
    counts = [64, 0, 30, 64]  # clamped; offsets 0, 64, 64, 94: only 80 rows fit
    L = 0
    for p, c in enumerate(counts):
        for r in range(c):
            if L < rows:
                assert np.array_equal(b[L], y[p, r]), f"landing row {L} is not window {p} row {r}"
            L += 1


def test_reduce_treats_out_of_window_entries_as_dropped():
    """sendMap entries outside [0, W*M) (never written by a dispatch) are
    dropped by both the reduce and the gather combine: both equal the oracle
    on the sendMap with those entries nulled."""
    w = workloads.CONFIGS["pr_scale"]
    inp = workloads.cached_inputs("pr_scale", 1)
    g = DeviceRun(w, inp)
    g.alloc_landing()
    g.dispatch()
    g.push()
    torch.cuda.synchronize()
    o = oracle_dispatch(w, inp)
    smap = o.sendMap.copy()
    kept = np.argwhere(smap >= 0)
    rng = np.random.Generator(np.random.PCG64(5))
    pick = kept[rng.choice(len(kept), 40, replace=False)]
    vals = np.array([w.worldSize * w.maxTokPerRank, 2**31 - 1], dtype=np.int64)
    for i, (t, k) in enumerate(pick):
        smap[t, k] = vals[i % 2]
    g.sendMap.copy_(torch.from_numpy(smap))
    g.reduce()
    torch.cuda.synchronize()
    red = out_as(g).copy()
    g.combine()
    torch.cuda.synchronize()
    gat = out_as(g).copy()
    nulled = smap.copy()
    nulled[nulled >= w.worldSize * w.maxTokPerRank] = -1
    exp = oracle_combine(w, inp.y, inp, nulled)
    assert_bits_equal(red, exp, "reduce with out-of-window entries")
    assert_bits_equal(gat, exp, "gather with out-of-window entries")


def test_push_reduce_graph_replay():
    """dispatch + push + reduce captured once and replayed several times
    (eager work and syncs in between) equal the eager results."""
    w = workloads.CONFIGS["pr_scale"]
    inp = workloads.cached_inputs("pr_scale", 2)
    g = DeviceRun(w, inp)
    g.alloc_landing()
    g.dispatch()
    g.push()
    g.reduce()
    torch.cuda.synchronize()
    U = int(g.recvCount.sum().item())  # rows past the landed total are never rewritten
    ref = {"landing": g.landing[:U].clone(), "landScale": g.landScale[:U].clone(), "out": g.out.clone()}
    s = torch.cuda.Stream()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        g.dispatch(stream=s)
        g.push(stream=s)
        g.reduce(stream=s)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph, stream=s):
        g.dispatch(stream=s)
        g.push(stream=s)
        g.reduce(stream=s)
    for rep in range(3):
        g.landing.fill_(1)
        g.landScale.fill_(2.0)
        g.out.fill_(3)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert g.scratch_clean()
        got = {"landing": g.landing[:U], "landScale": g.landScale[:U], "out": g.out}
        for k, v in ref.items():
            assert torch.equal(got[k], v), f"graph replay {rep} differs from eager: {k}"


def test_buffer_helpers_drive_every_call():
    """DispatchBuffers / LandingBuffers give buffers every call accepts:
    dispatch, gather combine, push and reduce on them match the oracle."""
    w = workloads.CONFIGS["epcfg_defaults"]
    inp = workloads.cached_inputs("epcfg_defaults", 1)
    c = epdc.EpCfg(w.worldSize, w.hiddenDim, w.maxTokPerRank, w.numExpertPerRank, w.numExpertPerToken,
                   epdc.EPDC_BF16, w.useWeights)
    b = epdc.DispatchBuffers(c)
    lb = epdc.LandingBuffers(c, w.numTokens)
    x = torch.from_numpy(inp.x.view(np.int16)).cuda().view(torch.bfloat16)
    y = torch.from_numpy(inp.y.view(np.int16)).cuda().view(torch.bfloat16)
    ids = torch.from_numpy(inp.expertIds).cuda()
    wts = torch.from_numpy(inp.weights).cuda()
    out_g = torch.empty((w.numTokens, w.hiddenDim), dtype=torch.bfloat16, device="cuda")
    out_r = torch.empty_like(out_g)
    epdc.epdc_dispatch(c, w.numTokens, x, ids, wts, None, b.recvX, b.recvTokIdx, b.recvExpertIds, b.recvWeights,
                       None, b.recvCount, b.sendMap, b.scratch)
    epdc.epdc_combine(c, w.numTokens, y, ids, wts, b.sendMap, out_g)
    epdc.epdc_combine_push(c, w.numTokens, y, b.recvExpertIds, b.recvWeights, b.recvCount, lb.landing, lb.landScale)
    epdc.epdc_combine_reduce(c, w.numTokens, lb.landing, lb.landScale, b.recvCount, b.sendMap, out_r)
    torch.cuda.synchronize()
    o = oracle_dispatch(w, inp)
    assert np.array_equal(b.sendMap[:w.numTokens].cpu().numpy(), o.sendMap)
    exp = oracle_combine(w, inp.y, inp, o.sendMap)
    got_g = out_g.view(torch.int16).cpu().numpy().view(np.uint16)
    got_r = out_r.view(torch.int16).cpu().numpy().view(np.uint16)
    assert_bits_equal(got_g, exp, "helpers gather")
    assert_bits_equal(got_r, exp, "helpers reduce")


@pytest.mark.parametrize("combine_dtype", ["bf16", "fp32"])
def test_non_finite_rows(combine_dtype):
    """Returned rows holding +-Inf and quiet / signalling NaNs, and zero
    weights (so 0 * Inf makes NaN): every finite or infinite result is bit
    for bit the oracle's, and every NaN result is a NaN on both sides (its
    payload may differ between the CPU's and the GPU's fused multiply-add),
    for the gather combine and for push + reduce."""
    base = workloads.CONFIGS["pr_scale"]
    w = base.with_(name=f"non_finite_{combine_dtype}", hiddenDim=512, wire=combine_dtype,
                   combineDtype=combine_dtype)
    inp = workloads.make_inputs(w, 31)
    rng = np.random.Generator(np.random.PCG64(32))
    y = inp.y.copy()
    pick = rng.random(y.shape) < 0.01
    if combine_dtype == "bf16":
        specials = np.array([0x7F80, 0xFF80, 0x7FC0, 0x7F81, 0xFFC1], dtype=np.uint16)
    else:
        specials = np.array([0x7F800000, 0xFF800000, 0x7FC00000, 0x7F800001, 0xFFC00001],
                            dtype=np.uint32).view(np.float32)
    y[pick] = rng.choice(specials, size=int(pick.sum()))
    wts = inp.weights.copy()
    wts[rng.random(wts.shape) < 0.1] = 0.0
    inp = dataclasses.replace(inp, y=y, weights=wts)
    g = DeviceRun(w, inp)
    g.alloc_landing()
    g.dispatch()
    torch.cuda.synchronize()
    o = oracle_dispatch(w, inp)
    assert_dispatch_equal(g, o, w.name)
    exp = oracle_combine(w, y, inp, o.sendMap)
    land, sc = oracle_push(w, y, o)
    g.combine()
    torch.cuda.synchronize()
    got_g = out_as(g).copy()
    g.push()
    g.reduce()
    torch.cuda.synchronize()
    got_r = out_as(g).copy()
    ef = exp.astype(np.float32) if combine_dtype == "fp32" else \
        (exp.astype(np.uint32) << 16).view(np.float32)
    nan = np.isnan(ef)
    assert nan.any() and np.isinf(ef).any(), "the case should produce NaN and Inf results"
    for got, what in ((got_g, "gather"), (got_r, "reduce")):
        gf = got.astype(np.float32) if combine_dtype == "fp32" else (got.astype(np.uint32) << 16).view(np.float32)
        assert np.isnan(gf[nan]).all(), f"{what}: a NaN result is not NaN on the GPU"
        assert not np.isnan(gf[~nan]).any(), f"{what}: a NaN where the oracle has none"
        eb = exp.view(np.uint16 if combine_dtype == "bf16" else np.uint32)
        gb = got.view(eb.dtype)
        bad = (gb != eb) & ~nan
        assert not bad.any(), f"{what}: {int(bad.sum())} non-NaN results differ from the oracle"


def test_prepared_calls_match_direct_calls():
    """Prepared calls (arguments marshalled once) write exactly what the
    direct calls write, for all four entry points."""
    w = workloads.CONFIGS["pr_scale"]
    inp = workloads.cached_inputs("pr_scale", 3)
    g = DeviceRun(w, inp)
    g.alloc_landing()
    g.dispatch()
    g.combine()
    torch.cuda.synchronize()
    gather = g.out.clone()
    g.push()
    g.reduce()
    torch.cuda.synchronize()
    ref = {k: getattr(g, k).clone() for k in ("recvX", "recvTokIdx", "recvExpertIds", "recvWeights", "recvCount",
                                              "sendMap", "landing", "landScale", "out")}
    for k in ("recvX", "recvTokIdx", "recvExpertIds", "recvWeights", "sendMap", "landing", "landScale", "out"):
        getattr(g, k).fill_(0)
    g.prepare()
    g.p_dispatch()
    g.p_combine()
    torch.cuda.synchronize()
    assert torch.equal(g.out, gather), "prepared combine differs"
    g.p_push()
    g.p_reduce()
    torch.cuda.synchronize()
    for k, v in ref.items():
        if k in ("recvX", "recvTokIdx", "recvExpertIds", "recvWeights"):  # rows past recvCount were zeroed
            cnt = g.recvCount.cpu().tolist()
            for p_, c in enumerate(cnt):
                assert torch.equal(getattr(g, k)[p_, :c], v[p_, :c]), f"prepared dispatch differs: {k}"
        elif k in ("landing", "landScale"):
            U = int(g.recvCount.sum().item())
            assert torch.equal(getattr(g, k)[:U], v[:U]), f"prepared push differs: {k}"
        else:
            assert torch.equal(getattr(g, k), v), f"prepared call differs: {k}"
    assert g.scratch_clean()
