"""Seeded random shapes through every entry point, against the oracle bit
for bit: worldSize 1..64, 1..8 experts per rank, topk 1..min(E, 64), token
counts 0..M with M up to 3000, rows of any multiple of 16 bytes up to ~10 KB
(bf16 or fp32, into a bf16 or fp32 output), 0..100 forwarded scales per token,
both useWeights, uniform or Zipf routing, ~10% invalid ids.
The shapes are drawn once from a fixed seed, so the cases are the same on
every run."""
import dataclasses

import numpy as np
import pytest
import torch

import workloads
from gpu_harness import (DeviceRun, assert_bits_equal, assert_dispatch_equal, assert_landing_equal, oracle_combine,
                         oracle_dispatch, oracle_push, oracle_reduce, out_as)

pytestmark = pytest.mark.gpu


def _draw_cases(n=24, seed=2024):
    rng = np.random.Generator(np.random.PCG64(seed))
    cases = []
    while len(cases) < n:
        W = int(rng.integers(1, 65))
        Epr = int(rng.integers(1, 9))
        E = W * Epr
        K = int(rng.integers(1, min(E, 64) + 1))
        M = int(rng.integers(1, 3001))
        T = int(rng.integers(0, M + 1))
        dt = "fp32" if rng.random() < 0.3 else "bf16"
        per16 = 4 if dt == "fp32" else 8          # elements per 16 bytes
        H = per16 * int(rng.integers(1, 10240 // (4 * per16) + 1))
        if W * M * H > 60_000_000:                # keep host and device copies small
            continue
        cases.append((len(cases), W, Epr, M, T, K, H, dt, int(rng.integers(0, 2)),
                      "zipf" if rng.random() < 0.4 else "uniform"))
    return cases


CASES = _draw_cases()


def _extras(i):
    """Forwarded scales (0..100 per token) and the combine output type of
    case i, from a stream of their own (the shapes above stay as drawn)."""
    rng = np.random.Generator(np.random.PCG64([2024, i]))
    S = int(rng.integers(1, 101)) if rng.random() < 0.5 else 0
    return S, ("fp32" if rng.random() < 0.5 else "bf16")


@pytest.mark.parametrize("case", CASES, ids=[f"r{c[0]}_W{c[1]}_K{c[5]}_T{c[4]}_H{c[6]}_{c[7]}" for c in CASES])
def test_random_shape_parity(case):
    i, W, Epr, M, T, K, H, dt, useW, routing = case
    S, out = _extras(i)
    w = workloads.Workload(f"random{i}", W, Epr, M, T, K, H, routing, useW, wire=dt, combineDtype=dt,
                           outDtype=out, scaleDim=S)
    inp = workloads.make_inputs(w, 100 + i)
    rng = np.random.Generator(np.random.PCG64(500 + i))
    ids = inp.expertIds.copy()
    mask = rng.random(ids.shape) < 0.1
    ids[mask] = rng.choice(np.array([-1, W * Epr, -7, 2**31 - 1], dtype=np.int64), size=ids.shape)[mask]
    inp = dataclasses.replace(inp, expertIds=ids.astype(np.int32))
    tag = f"random{i} W{W} Epr{Epr} M{M} T{T} K{K} H{H} {dt}->{out} S{S} w{useW} {routing}"
    print(f"[random] {tag}", flush=True)
    g = DeviceRun(w, inp)
    g.alloc_landing()
    g.dispatch()
    torch.cuda.synchronize()
    o = oracle_dispatch(w, inp)
    assert_dispatch_equal(g, o, tag)
    assert g.scratch_clean(), f"{tag}: scratch not clean"
    g.push()
    torch.cuda.synchronize()
    land, sc = oracle_push(w, inp.y, o)
    assert_landing_equal(g, land, sc, tag)
    if T == 0:
        return
    g.combine()
    torch.cuda.synchronize()
    exp = oracle_combine(w, inp.y, inp, o.sendMap)
    assert_bits_equal(out_as(g), exp, f"{tag} combine")
    g.reduce()
    torch.cuda.synchronize()
    assert_bits_equal(out_as(g), exp, f"{tag} reduce")
