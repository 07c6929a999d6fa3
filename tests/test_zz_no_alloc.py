"""epdc_dispatch_noalloc: the dispatch on the library's own device scratch
(a file-scope array per GPU, no allocation on any call) against
epdc_dispatch with a caller scratch, bit for bit, through the C ABI: two
calls in a row on one GPU, the second with fewer tokens (the array keeps
the first call's contents), over each SCAN form (tile leaders, every block,
local) and with forwarded scales; plus the host-side size limit."""
import ctypes

import numpy as np
import pytest
import torch

import combine_count_amd as epdc
import workloads
from gpu_harness import DeviceRun, SENT_MAP

P16 = 0x10000  # a fake 16-byte aligned device address: never dereferenced on the host-check paths


def _limit_cfg(T_max):
    return epdc.EpCfg(64, 1024, T_max, 1, 8, epdc.EPDC_BF16, 1, 0)


def test_size_limit_is_checked_before_any_launch():
    """4224 + 8 * ceil(T / 64) * W' bytes must fit the 1 MiB array: at 64
    PEs, 130,496 tokens fit and 130,497 do not; the refusal names the limit."""
    c = _limit_cfg(200000)
    args = [P16] * 11
    rc = epdc.epdc_dispatch_noalloc(c, 130497, *args, stream=0, check=False)
    assert rc == -6, epdc.epdc_last_error()
    assert "1048576" in epdc.epdc_last_error()
    if not torch.cuda.is_available():  # the checks pass; with no device the launch reports EPDC_ERR_HIP
        assert epdc.epdc_dispatch_noalloc(c, 130496, *args, stream=0, check=False) == -7
    assert epdc.epdc_dispatch_noalloc(c, -1, *args, stream=0, check=False) == -1
    assert epdc.epdc_dispatch_noalloc(c, 8, *args[:10], None, stream=0, check=False) == -5  # sendMap


def _run_pair(w, seed):
    """The same inputs through both entry points (outputs sentinel-filled
    alike); returns the two DeviceRuns."""
    inp = workloads.make_inputs(w, seed, with_y=False)
    a, b = DeviceRun(w, inp), DeviceRun(w, inp)
    a.dispatch()
    epdc.epdc_dispatch_noalloc(b.cfg, w.numTokens, b.x, b.ids, b.wts, b.scales, b.recvX, b.recvTokIdx,
                               b.recvExpertIds, b.recvWeights if w.useWeights else None, b.recvScales,
                               b.recvCount, b.sendMap)
    return a, b


def _assert_same(a, b, tag):
    for k in ("recvCount", "sendMap", "recvTokIdx", "recvExpertIds", "recvWeights", "recvX"):
        assert torch.equal(getattr(a, k), getattr(b, k)), f"{tag}: {k} differs between the two entry points"
    if a.recvScales is not None:
        assert torch.equal(a.recvScales.view(torch.int32), b.recvScales.view(torch.int32)), f"{tag}: recvScales"


SEQUENCES = [
    # (first workload, second with fewer tokens): the SCAN forms of the first call
    ("leader_scan_then_self_scan", workloads.CONFIGS["gen_zipf_h7168"].with_(numTokens=3072), dict(numTokens=777)),
    ("self_scan_then_local", workloads.CONFIGS["gen_zipf_h7168"].with_(wire="fp8", scaleDim=56),
     dict(numTokens=300)),
    ("large_leader_then_leader_scan", workloads.CONFIGS["large_unweighted"], dict(numTokens=3000)),
    ("local_then_one_token", workloads.CONFIGS["pr_scale"], dict(numTokens=1)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("name,first,second", SEQUENCES, ids=[s[0] for s in SEQUENCES])
def test_noalloc_matches_dispatch_twice_in_a_row(name, first, second):
    print(f"[no-alloc] {name}: {first.name} T={first.numTokens} then T={second['numTokens']}", flush=True)
    w1 = first.with_(name=f"{name}_1")
    w2 = first.with_(name=f"{name}_2", **second)
    a1, b1 = _run_pair(w1, 3)
    a2, b2 = _run_pair(w2, 4)  # enqueued right behind the first, same array
    torch.cuda.synchronize()
    _assert_same(a1, b1, f"{name} call 1")
    _assert_same(a2, b2, f"{name} call 2")
    assert a1.scratch_clean() and a2.scratch_clean()
    assert int(b2.recvCount.sum().item()) == int((b2.sendMap >= 0).sum().item())
    assert not bool((b2.sendMap == SENT_MAP).any().item()), "sendMap not fully written"
