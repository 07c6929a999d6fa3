"""Calls on different streams run concurrently and stay independent: the
library keeps no device state of its own (each dispatch has its own scratch),
so two workloads whose launches are interleaved on two streams, with no
synchronisation between them, both match the oracle.  Also: the current
stream (torch.cuda.stream context) is the one a call without stream= uses.
"""
import numpy as np
import pytest
import torch

import workloads
from gpu_harness import (DeviceRun, assert_bits_equal, assert_dispatch_equal, assert_landing_equal, dev_to_bits,
                         oracle_combine, oracle_dispatch, oracle_push, oracle_reduce, out_as)

pytestmark = pytest.mark.gpu


def _expect(w, inp):
    o = oracle_dispatch(w, inp)
    return o, oracle_combine(w, inp.y, inp, o.sendMap)


def test_two_streams_interleaved():
    cases = [(workloads.CONFIGS["gen_zipf_h2048"], 3), (workloads.CONFIGS["pr_scale"], 4)]
    runs, exps = [], []
    for w, seed in cases:
        inp = workloads.make_inputs(w, seed)
        runs.append(DeviceRun(w, inp))
        exps.append(_expect(w, inp))
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    print("[streams] 3 rounds of interleaved dispatch/combine on two streams", flush=True)
    for _ in range(3):
        for g, s in zip(runs, streams):
            g.dispatch(stream=s)
        for g, s in zip(runs, streams):
            g.combine(stream=s)
    torch.cuda.synchronize()
    for (w, _), g, (o, exp) in zip(cases, runs, exps):
        assert_dispatch_equal(g, o, f"{w.name} on its own stream")
        assert g.scratch_clean()
        assert_bits_equal(out_as(g), exp, f"{w.name} combine")


def test_current_stream_is_used():
    """Inside `with torch.cuda.stream(s)` a call without stream= goes to s:
    work queued on s after it sees its results without any other wait."""
    w = workloads.CONFIGS["epcfg_defaults"]
    inp = workloads.make_inputs(w, 5)
    g = DeviceRun(w, inp)
    g.alloc_landing()
    o, exp = _expect(w, inp)
    land_o, scale_o = oracle_push(w, inp.y, o)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        g.dispatch()
        g.combine()
        out_gather = g.out.clone()  # ordered after the combine on s
        g.push()
        g.reduce()
        out_reduce = g.out.clone()
    s.synchronize()
    assert_dispatch_equal(g, o, "current stream")
    assert_bits_equal(dev_to_bits(out_gather.view(torch.bfloat16)), exp, "gather on the current stream")
    assert_landing_equal(g, land_o, scale_o, "push on the current stream")
    assert_bits_equal(dev_to_bits(out_reduce.view(torch.bfloat16)), oracle_reduce(w, land_o, scale_o, o),
                      "reduce on the current stream")
    assert np.array_equal(dev_to_bits(out_gather.view(torch.bfloat16)), dev_to_bits(out_reduce.view(torch.bfloat16)))


def test_strided_device_tensor_is_refused():
    """A strided view would be read densely from its base address: the
    binding refuses it before anything is launched."""
    import combine_count_amd as epdc
    w = workloads.CONFIGS["tiny"]
    inp = workloads.make_inputs(w, 2)
    g = DeviceRun(w, inp)
    wide = torch.zeros((w.numTokens, 2 * w.hiddenDim), dtype=torch.bfloat16, device="cuda")
    strided = wide[:, ::2]
    with pytest.raises(ValueError, match="contiguous"):
        epdc.epdc_combine(g.ccfg, w.numTokens, g.y, g.ids, g.wts, g.sendMap, strided, g.outDtype)
