"""The torch buffer helpers allocate what include/epdc.h states for every
row type (on the CPU here: only shapes, dtypes and the zeroed scratch are
checked)."""
import pytest
import torch

import combine_count_amd as epdc

CFG = dict(worldSize=8, hiddenDim=7168, maxTokPerRank=256, numExpertPerRank=32, numExpertPerToken=8, useWeights=1)


@pytest.mark.parametrize("dtype,tdt", [(0, torch.bfloat16), (1, torch.float32), (2, torch.uint8), (3, torch.uint8)])
def test_dispatch_buffers(dtype, tdt):
    c = epdc.EpCfg(dtype=dtype, **CFG)
    b = epdc.DispatchBuffers(c, device="cpu")
    assert b.recvX.shape == (8, 256, 7168) and b.recvX.dtype == tdt
    assert b.recvTokIdx.shape == (8, 256) and b.recvTokIdx.dtype == torch.int32
    assert b.recvExpertIds.shape == (8, 256, 8)
    assert b.recvWeights.shape == (8, 256, 8) and b.recvWeights.dtype == torch.float32
    assert b.recvCount.shape == (8,)
    assert b.sendMap.shape == (256, 8)
    assert b.scratch.numel() * 4 >= epdc.epdc_dispatch_scratch_bytes(c)
    assert int(b.scratch.abs().sum()) == 0


def test_dispatch_buffers_unweighted_and_invalid():
    b = epdc.DispatchBuffers(epdc.EpCfg(dtype=0, **dict(CFG, useWeights=0)), device="cpu")
    assert b.recvWeights is None
    with pytest.raises(epdc.EpdcError):
        epdc.DispatchBuffers(epdc.EpCfg(dtype=0, **dict(CFG, hiddenDim=7163)), device="cpu")


@pytest.mark.parametrize("dtype,tdt", [(0, torch.bfloat16), (1, torch.float32)])
def test_landing_buffers(dtype, tdt):
    c = epdc.EpCfg(dtype=dtype, **CFG)
    b = epdc.LandingBuffers(c, 200, device="cpu")
    assert b.landing.shape == (200 * 8, 7168) and b.landing.dtype == tdt
    assert b.landScale.shape == (1600,) and b.landScale.dtype == torch.float32
    b = epdc.LandingBuffers(epdc.EpCfg(dtype=dtype, **dict(CFG, numExpertPerToken=3, useWeights=0)), 10, device="cpu")
    assert b.landing.shape == (30, 7168) and b.landScale is None


def test_landing_buffers_reject_byte_types_and_capacity():
    with pytest.raises(epdc.EpdcError):
        epdc.LandingBuffers(epdc.EpCfg(dtype=2, **CFG), 8, device="cpu")
    with pytest.raises(epdc.EpdcError):
        epdc.LandingBuffers(epdc.EpCfg(dtype=0, **CFG), 257, device="cpu")
