"""Helpers that run the HIP library and the oracle on the same seeded inputs.

Windows are pre-filled with the same sentinels on both sides, so whole-buffer
equality also proves that rows past recvCount are left untouched and that no
row is written twice or elsewhere.

The oracle is imported only by the oracle_* helpers: DeviceRun, which
bench.py's timed path uses, never loads it.
"""
from __future__ import annotations

import numpy as np
import torch

import combine_count_amd as epdc
import workloads


def _oracle():
    import oracle
    return oracle

SENT_X_BYTE = 0xAD        # every byte of recvX before the dispatch
SENT_OUT_BYTE = 0x7F
SENT_I32 = -12345
SENT_IDS = -777
SENT_W = -3.5
SENT_MAP = -99
SENT_LAND_BYTE = 0xA5     # landing rows before the push (the oracle's fill too)
SENT_SCALE = -3.25
SENT_RECV_SCALES = -6.75
FILL = {"recvX_byte": SENT_X_BYTE, "recvTokIdx": SENT_I32, "recvExpertIds": SENT_IDS, "recvWeights": SENT_W,
        "recvScales": SENT_RECV_SCALES}
OUT_BYTES = {"bf16": 2, "fp32": 4}


def cfg_of(w: workloads.Workload, combine: bool = False) -> epdc.EpCfg:
    """The dispatch cfg (wire type, hiddenDim in wire elements) or the
    combine cfg (combine type, logical hiddenDim)."""
    if combine:
        return epdc.EpCfg(w.worldSize, w.hiddenDim, w.maxTokPerRank, w.numExpertPerRank, w.numExpertPerToken,
                          workloads.EPDC_DTYPE[w.combineDtype], w.useWeights)
    return epdc.EpCfg(w.worldSize, w.dispatchHidden, w.maxTokPerRank, w.numExpertPerRank, w.numExpertPerToken,
                      workloads.EPDC_DTYPE[w.wire], w.useWeights, w.scaleDim)


def to_dev_bytes(a: np.ndarray, dev="cuda") -> torch.Tensor:
    """Any numpy array as a device uint8 tensor of the same bytes, rows kept."""
    a = np.ascontiguousarray(a)
    return torch.from_numpy(a.view(np.uint8).reshape(*a.shape[:-1], a.shape[-1] * a.itemsize)).to(dev)


def bits_to_dev(bits: np.ndarray, dev="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def dev_to_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


class DeviceRun:
    """Device copies of one input set plus sentinel-filled dispatch outputs.
    Payload buffers are raw bytes; their element type is the cfg's."""

    def __init__(self, w: workloads.Workload, inp: workloads.Inputs, dev="cuda"):
        self.w = w
        self.cfg = cfg_of(w)
        self.ccfg = cfg_of(w, combine=True)
        W, M, K, T = w.worldSize, w.maxTokPerRank, w.numExpertPerToken, w.numTokens
        rowB = w.dispatchHidden * workloads.WIRE_BYTES[w.wire]
        outB = w.hiddenDim * OUT_BYTES[w.outType]
        self.outDtype = workloads.EPDC_DTYPE[w.outType]
        self.x = to_dev_bytes(inp.x, dev)
        self.ids = torch.from_numpy(inp.expertIds).to(dev)
        self.wts = torch.from_numpy(inp.weights).to(dev) if w.useWeights else None
        S = w.scaleDim
        self.scales = torch.from_numpy(inp.scales).to(dev) if S else None
        self.recvScales = torch.full((W, M, S), SENT_RECV_SCALES, dtype=torch.float32, device=dev) if S else None
        self.y = to_dev_bytes(inp.y, dev) if inp.y is not None else None
        self.recvX = torch.full((W, M, rowB), SENT_X_BYTE, dtype=torch.uint8, device=dev)
        self.recvTokIdx = torch.full((W, M), SENT_I32, dtype=torch.int32, device=dev)
        self.recvExpertIds = torch.full((W, M, K), SENT_IDS, dtype=torch.int32, device=dev)
        self.recvWeights = torch.full((W, M, K), SENT_W, dtype=torch.float32, device=dev)
        self.recvCount = torch.full((W,), -7, dtype=torch.int32, device=dev)
        self.sendMap = torch.full((T, K), SENT_MAP, dtype=torch.int32, device=dev)
        nb = epdc.epdc_dispatch_scratch_bytes(self.cfg)
        self.scratch = torch.zeros(max(nb, 4) // 4 + 1, dtype=torch.int32, device=dev)
        self.out = torch.full((T, outB), SENT_OUT_BYTE, dtype=torch.uint8, device=dev)

    def alloc_landing(self, dev="cuda"):
        """Landing rows and scales of the scatter combine, sentinel-filled."""
        w = self.w
        rows = epdc.epdc_landing_rows(self.ccfg, w.numTokens)
        outB = w.hiddenDim * workloads.WIRE_BYTES[w.combineDtype]
        self.landing = torch.full((rows, outB), SENT_LAND_BYTE, dtype=torch.uint8, device=dev)
        self.landScale = torch.full((rows,), SENT_SCALE, dtype=torch.float32, device=dev)

    def push(self, y=None, stream=None):
        w = self.w
        return epdc.epdc_combine_push(self.ccfg, w.numTokens, self.y if y is None else y,
                                      self.recvExpertIds if w.useWeights else None,
                                      self.recvWeights if w.useWeights else None, self.recvCount,
                                      self.landing, self.landScale if w.useWeights else None, stream=stream)

    def reduce(self, stream=None):
        w = self.w
        return epdc.epdc_combine_reduce(self.ccfg, w.numTokens, self.landing,
                                        self.landScale if w.useWeights else None, self.recvCount, self.sendMap,
                                        self.out, self.outDtype, stream=stream)

    def prepare(self):
        """Prepared calls (arguments marshalled once) for the same buffers:
        self.p_dispatch, p_combine and, once landing rows exist, p_push and
        p_reduce."""
        w = self.w
        wt = self.wts if w.useWeights else None
        self.p_dispatch = epdc.prepare_dispatch(self.cfg, w.numTokens, self.x, self.ids, wt, self.scales, self.recvX,
                                                self.recvTokIdx, self.recvExpertIds,
                                                self.recvWeights if w.useWeights else None, self.recvScales,
                                                self.recvCount, self.sendMap, self.scratch)
        self.p_combine = epdc.prepare_combine(self.ccfg, w.numTokens, self.y, self.ids if w.useWeights else None, wt,
                                              self.sendMap, self.out, self.outDtype)
        if hasattr(self, "landing"):
            self.p_push = epdc.prepare_combine_push(self.ccfg, w.numTokens, self.y,
                                                    self.recvExpertIds if w.useWeights else None,
                                                    self.recvWeights if w.useWeights else None, self.recvCount,
                                                    self.landing, self.landScale if w.useWeights else None)
            self.p_reduce = epdc.prepare_combine_reduce(self.ccfg, w.numTokens, self.landing,
                                                        self.landScale if w.useWeights else None, self.recvCount,
                                                        self.sendMap, self.out, self.outDtype)
        return self

    def scratch_clean(self) -> bool:
        """After a dispatch the scratch is all zero again (status word included)."""
        return bool((self.scratch == 0).all().item())

    def dispatch(self, stream=None):
        w = self.w
        return epdc.epdc_dispatch(self.cfg, w.numTokens, self.x, self.ids, self.wts, self.scales, self.recvX,
                                  self.recvTokIdx, self.recvExpertIds,
                                  self.recvWeights if w.useWeights else None, self.recvScales, self.recvCount,
                                  self.sendMap, self.scratch, stream=stream)

    def combine(self, y=None, weights="default", stream=None):
        w = self.w
        wts = self.wts if weights == "default" else weights
        return epdc.epdc_combine(self.ccfg, w.numTokens, self.y if y is None else y,
                                 self.ids if w.useWeights else None, wts if w.useWeights else None, self.sendMap,
                                 self.out, self.outDtype, stream=stream)


def oracle_dispatch(w: workloads.Workload, inp: workloads.Inputs):
    return _oracle().dispatch(w.worldSize, w.dispatchHidden, w.maxTokPerRank, w.numExpertPerRank,
                           w.numExpertPerToken, w.useWeights, inp.x, inp.expertIds,
                           inp.weights if w.useWeights else None, inp.scales, fill=FILL)


def oracle_combine(w: workloads.Workload, y_bits, inp: workloads.Inputs, sendMap, tokens=None, weights=None):
    wts = inp.weights if weights is None else weights
    return _oracle().combine(w.worldSize, w.hiddenDim, w.maxTokPerRank, w.numExpertPerRank,
                          w.numExpertPerToken, w.useWeights, y_bits, inp.expertIds,
                          wts if w.useWeights else None, sendMap, tokens=tokens, out_fp32=w.outType == "fp32")


def oracle_push(w: workloads.Workload, y, o):
    """The oracle push over returned rows y, from the oracle dispatch o."""
    return _oracle().combine_push(w.worldSize, w.hiddenDim, w.maxTokPerRank, w.numExpertPerRank,
                               w.numExpertPerToken, w.useWeights, w.numTokens, y, o.recvExpertIds,
                               o.recvWeights if w.useWeights else None, o.recvCount,
                               fill_byte=SENT_LAND_BYTE, scale_fill=SENT_SCALE)


def oracle_reduce(w: workloads.Workload, landing, landScale, o, tokens=None):
    return _oracle().combine_reduce(w.worldSize, w.hiddenDim, w.maxTokPerRank, w.numExpertPerRank,
                                 w.numExpertPerToken, w.useWeights, landing, landScale, o.recvCount, o.sendMap,
                                 tokens=tokens, out_fp32=w.outType == "fp32")


def assert_landing_equal(g: DeviceRun, landing, landScale, tag=""):
    """Every landing row (landed or sentinel) and every scale, bit for bit."""
    gl = g.landing.cpu().numpy()
    ol = landing.view(np.uint8).reshape(gl.shape)
    if not np.array_equal(gl, ol):
        bad = np.argwhere(gl != ol)[0]
        raise AssertionError(f"{tag} landing differs first at byte {bad.tolist()}")
    gs = g.landScale.cpu().numpy()
    if not np.array_equal(gs.view(np.uint32), landScale.view(np.uint32)):
        bad = int(np.argwhere(gs.view(np.uint32) != landScale.view(np.uint32))[0, 0])
        raise AssertionError(f"{tag} landScale[{bad}] = {gs[bad]!r} vs oracle {landScale[bad]!r}")


def assert_dispatch_equal(g: DeviceRun, o, tag=""):
    """Every dispatch output, whole buffers, bit for bit."""
    w = g.w
    cnt = g.recvCount.cpu().numpy()
    assert np.array_equal(cnt, o.recvCount), f"{tag} recvCount {cnt} != oracle {o.recvCount}"
    smap = g.sendMap.cpu().numpy()
    if not np.array_equal(smap, o.sendMap):
        bad = np.argwhere(smap != o.sendMap)[0]
        raise AssertionError(f"{tag} sendMap differs first at {bad.tolist()}: "
                             f"{smap[tuple(bad)]} vs {o.sendMap[tuple(bad)]}")
    tok = g.recvTokIdx.cpu().numpy()
    assert np.array_equal(tok, o.recvTokIdx), f"{tag} recvTokIdx differs"
    ids = g.recvExpertIds.cpu().numpy()
    assert np.array_equal(ids, o.recvExpertIds), f"{tag} recvExpertIds differs"
    wt = g.recvWeights.cpu().numpy()
    if w.useWeights:
        assert np.array_equal(wt.view(np.uint32), o.recvWeights.view(np.uint32)), f"{tag} recvWeights differs"
    else:
        assert (wt == np.float32(SENT_W)).all(), f"{tag} recvWeights written with useWeights=0"
    if w.scaleDim:
        sc = g.recvScales.cpu().numpy()
        if not np.array_equal(sc.view(np.uint32), o.recvScales.view(np.uint32)):
            bad = np.argwhere(sc.view(np.uint32) != o.recvScales.view(np.uint32))[0]
            raise AssertionError(f"{tag} recvScales differs first at {bad.tolist()}: {sc[tuple(bad)]} vs "
                                 f"{o.recvScales[tuple(bad)]}")
    rx = g.recvX.cpu().numpy()
    ox = o.recvX.view(np.uint8).reshape(rx.shape)
    if not np.array_equal(rx, ox):
        bad = np.argwhere(rx != ox)[0]
        raise AssertionError(f"{tag} recvX differs first at byte {bad.tolist()}")


def out_as(g: DeviceRun) -> np.ndarray:
    """The device out rows as the output type (uint16 bf16 bits or float32)."""
    dt = np.uint16 if g.w.outType == "bf16" else np.float32
    return g.out.cpu().numpy().view(dt)


def assert_bits_equal(got: np.ndarray, exp: np.ndarray, tag=""):
    gb = got.view(np.uint16 if got.dtype == np.uint16 else np.uint32)
    eb = exp.view(gb.dtype)
    if not np.array_equal(gb, eb):
        bad = np.argwhere(gb != eb)
        t, h = bad[0]
        raise AssertionError(f"{tag} {len(bad)} elements differ; first out[{t}][{h}] = "
                             f"{hex(int(gb[t, h]))} vs oracle {hex(int(eb[t, h]))}")
