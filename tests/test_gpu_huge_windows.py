"""Windows of 2^31 - 8 rows: byte offsets up to ~30 GB and flat row indices
up to ~1.9e9, near the int32 limit the boundary allows (W * maxTokPerRank <=
INT32_MAX).  Every address past 4 GB must be computed in 64 bits.

The device runs with maxTokPerRank M = 2^28 - 1 (about 104 GB of windows,
returned rows and metadata); the oracle runs the same tokens with M' = T.
maxTokPerRank only places rows (flat index p * M + r), so the two agree row
for row on [0, recvCount[p]) of every window, on the sendMap after mapping
p * M + r to p * M' + r, and bit for bit on the combine, push and reduce
outputs.  Sentinel rows just past each window's count and at its very end
show nothing else was written.
"""
import numpy as np
import pytest
import torch

import combine_count_amd as epdc
import workloads
from gpu_harness import (SENT_I32, SENT_IDS, SENT_LAND_BYTE, SENT_MAP, SENT_OUT_BYTE, SENT_SCALE, SENT_W,
                         SENT_X_BYTE, assert_bits_equal, bits_to_dev, dev_to_bits, oracle_combine,
                         oracle_dispatch, oracle_push, oracle_reduce, to_dev_bytes)

pytestmark = pytest.mark.gpu

W, EPR, K, H, T = 8, 4, 2, 8, 3000
M = (2**31 - 1) // W  # 268435455: W * M = 2^31 - 8


def _window_rows(t: torch.Tensor, counts, extra_rows):
    """Per PE: rows [0, count) and the given single rows past it, to the host."""
    return [(t[p, :c].cpu().numpy(), [t[p, r:r + 1].cpu().numpy() for r in extra_rows(c)])
            for p, c in enumerate(counts)]


def test_windows_past_4_gib_and_flat_indices_near_int32_max():
    try:
        _run()
    finally:
        torch.cuda.empty_cache()  # hand the ~104 GB back before the next test


def _run():
    w = workloads.Workload("huge_windows", W, EPR, T, T, K, H, "uniform", 1)  # oracle side: M' = T
    inp = workloads.make_inputs(w, 21)
    o = oracle_dispatch(w, inp)
    counts = [int(c) for c in o.recvCount]
    assert all(0 < c < T for c in counts)

    cfg = epdc.EpCfg(W, H, M, EPR, K, epdc.EPDC_BF16, 1)
    print(f"[huge windows] W={W} M={M} K={K} H={H} T={T}: allocating ~104 GB", flush=True)
    dev = "cuda"
    x = to_dev_bytes(inp.x, dev)
    ids = torch.from_numpy(inp.expertIds).to(dev)
    wts = torch.from_numpy(inp.weights).to(dev)
    recvX = torch.full((W, M, H * 2), SENT_X_BYTE, dtype=torch.uint8, device=dev)
    recvTokIdx = torch.full((W, M), SENT_I32, dtype=torch.int32, device=dev)
    recvExpertIds = torch.full((W, M, K), SENT_IDS, dtype=torch.int32, device=dev)
    recvWeights = torch.full((W, M, K), SENT_W, dtype=torch.float32, device=dev)
    recvCount = torch.full((W,), -7, dtype=torch.int32, device=dev)
    sendMap = torch.full((T, K), SENT_MAP, dtype=torch.int32, device=dev)
    nb = epdc.epdc_dispatch_scratch_bytes(cfg)
    scratch = torch.zeros(nb // 4 + 1, dtype=torch.int32, device=dev)

    print("[huge windows] dispatch", flush=True)
    epdc.epdc_dispatch(cfg, T, x, ids, wts, None, recvX, recvTokIdx, recvExpertIds, recvWeights, None, recvCount,
                       sendMap, scratch)
    torch.cuda.synchronize()
    assert recvCount.cpu().numpy().tolist() == counts
    assert bool((scratch == 0).all().item()), "scratch not left zeroed"

    past = lambda c: (c, M - 1)  # the first row past the count and the window's last row
    for name, dev_t, ora in [("recvX", recvX, o.recvX.view(np.uint8).reshape(W, T, H * 2)),
                             ("recvTokIdx", recvTokIdx, o.recvTokIdx),
                             ("recvExpertIds", recvExpertIds, o.recvExpertIds),
                             ("recvWeights", recvWeights, o.recvWeights)]:
        for p, (rows, tail) in enumerate(_window_rows(dev_t, counts, past)):
            c = counts[p]
            assert np.array_equal(rows.view(np.uint8), np.ascontiguousarray(ora[p, :c]).view(np.uint8)), \
                f"{name} PE {p}"
            for got in tail:  # untouched: the sentinel on the oracle side too (row c < M' = T)
                assert np.array_equal(got.view(np.uint8), np.ascontiguousarray(ora[p, c:c + 1]).view(np.uint8)), \
                    f"{name} PE {p} tail"

    sm = sendMap.cpu().numpy().astype(np.int64)
    assert sm.max() > 6 * M, "rows of the last PEs sit above 1.6e9"
    mapped = np.where(sm >= 0, (sm // M) * T + sm % M, sm)
    assert np.array_equal(mapped, o.sendMap), "sendMap"

    # Returned rows: the oracle's y' [W][T][H] in rows [0, count) of each huge window.
    y = torch.empty((W, M, H), dtype=torch.bfloat16, device=dev)
    y.view(torch.int16).fill_(0x7F01)
    for p, c in enumerate(counts):
        y[p, :c] = bits_to_dev(inp.y[p, :c], dev)
    out = torch.full((T, H * 2), SENT_OUT_BYTE, dtype=torch.uint8, device=dev)
    print("[huge windows] combine", flush=True)
    epdc.epdc_combine(cfg, T, y, ids, wts, sendMap, out)
    torch.cuda.synchronize()
    exp = oracle_combine(w, inp.y, inp, o.sendMap)
    assert_bits_equal(dev_to_bits(out.view(torch.bfloat16)), exp, "huge windows combine")

    rows = epdc.epdc_landing_rows(cfg, T)
    landing = torch.full((rows, H * 2), SENT_LAND_BYTE, dtype=torch.uint8, device=dev)
    landScale = torch.full((rows,), SENT_SCALE, dtype=torch.float32, device=dev)
    out.fill_(SENT_OUT_BYTE)
    print("[huge windows] push + reduce", flush=True)
    epdc.epdc_combine_push(cfg, T, y, recvExpertIds, recvWeights, recvCount, landing, landScale)
    epdc.epdc_combine_reduce(cfg, T, landing, landScale, recvCount, sendMap, out)
    torch.cuda.synchronize()
    land_o, scale_o = oracle_push(w, inp.y, o)
    assert np.array_equal(landing.cpu().numpy(), land_o.view(np.uint8).reshape(rows, H * 2)), "landing rows"
    assert np.array_equal(landScale.cpu().numpy().view(np.uint32), scale_o.view(np.uint32)), "landing scales"
    assert_bits_equal(dev_to_bits(out.view(torch.bfloat16)), oracle_reduce(w, land_o, scale_o, o),
                      "huge windows reduce")
