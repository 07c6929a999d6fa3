"""The C ABI on a host with or without a GPU: the library loads, exports
every symbol include/epdc.h declares, and rejects every invalid argument on
the host with its documented code before anything is launched."""
import ctypes
import os
import re
import subprocess

import pytest

import combine_count_amd as epdc
from combine_count_amd.binding import LIB_PATH

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "epdc.h")

OK_CFG = dict(worldSize=8, hiddenDim=7168, maxTokPerRank=4096, numExpertPerRank=32,
              numExpertPerToken=8, dtype=0, useWeights=1, scaleDim=0)
P16 = 0x10000  # a fake, 16-byte aligned device address: never dereferenced on these paths


def cfg(**kw):
    d = dict(OK_CFG)
    d.update(kw)
    return epdc.EpCfg(**d)


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(epdc_[a-z_]+)\s*\(", src)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(epdc.EXPORTS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", LIB_PATH], capture_output=True, text=True, check=True)
    exported = set(re.findall(r" T (epdc_\w+)", nm.stdout))
    assert set(declared_functions()) <= exported


def test_header_compiles_as_c():
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-fsyntax-only", "-x", "c", HEADER],
                       capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_scratch_bytes():
    assert epdc.epdc_dispatch_scratch_bytes(cfg()) == 4224 + 2 * (4096 // 64) * 8 * 4
    assert epdc.epdc_dispatch_scratch_bytes(cfg(worldSize=5, maxTokPerRank=65)) == 4224 + 2 * 2 * 8 * 4
    assert epdc.epdc_dispatch_scratch_bytes(cfg(hiddenDim=7170)) == 0


def _dispatch(c, T, **ptrs):
    args = dict(x=P16, expertIds=P16, weights=P16, scales=P16, recvX=P16, recvTokIdx=P16, recvExpertIds=P16,
                recvWeights=P16, recvScales=P16, recvCount=P16, sendMap=P16, scratch=P16)
    args.update(ptrs)
    return epdc.epdc_dispatch(c, T, args["x"], args["expertIds"], args["weights"], args["scales"], args["recvX"],
                              args["recvTokIdx"], args["recvExpertIds"], args["recvWeights"], args["recvScales"],
                              args["recvCount"], args["sendMap"], args["scratch"],
                              scratchBytes=ptrs.get("scratchBytes", 1 << 20), stream=0, check=False)


def _combine(c, T, outDtype=None, **ptrs):
    args = dict(y=P16, expertIds=P16, weights=P16, sendMap=P16, out=P16)
    args.update(ptrs)
    return epdc.epdc_combine(c, T, args["y"], args["expertIds"], args["weights"], args["sendMap"],
                             args["out"], outDtype, stream=0, check=False)


REJECT = [
    # (what, cfg overrides, numTokens, pointer overrides, expected code)
    ("worldSize 0", dict(worldSize=0), 8, {}, -1),
    ("worldSize 65", dict(worldSize=65), 8, {}, -1),
    ("topk 0", dict(numExpertPerToken=0), 8, {}, -1),
    ("topk 65", dict(numExpertPerToken=65), 8, {}, -1),
    ("topk > experts", dict(worldSize=2, numExpertPerRank=2, numExpertPerToken=5), 8, {}, -1),
    ("numExpertPerRank 0", dict(numExpertPerRank=0), 8, {}, -1),
    ("hiddenDim 0", dict(hiddenDim=0), 8, {}, -1),
    ("maxTokPerRank 0", dict(maxTokPerRank=0), 0, {}, -1),
    ("flat index overflow", dict(worldSize=64, maxTokPerRank=40_000_000), 8, {}, -1),
    ("negative tokens", {}, -1, {}, -1),
    ("dtype 4", dict(dtype=4), 8, {}, -2),
    ("dtype -1", dict(dtype=-1), 8, {}, -2),
    ("useWeights 2", dict(useWeights=2), 8, {}, -2),
    ("capacity", {}, 4097, {}, -3),
    ("row bytes not 16-aligned", dict(hiddenDim=7164), 8, {}, -4),
    ("fp32 row of 24 bytes", dict(hiddenDim=6, dtype=1), 8, {}, -4),
    ("fp8 row of 8 bytes", dict(hiddenDim=8, dtype=2), 8, {}, -4),
    ("fp4x2 row of 7160 bytes", dict(hiddenDim=7160, dtype=3), 8, {}, -4),
    ("x misaligned", {}, 8, dict(x=P16 + 8), -4),
    ("recvX misaligned", {}, 8, dict(recvX=P16 + 4), -4),
    ("ids misaligned", {}, 8, dict(expertIds=P16 + 2), -4),
    ("scratch misaligned", {}, 8, dict(scratch=P16 + 4), -4),
    ("x null", {}, 8, dict(x=None), -5),
    ("sendMap null", {}, 8, dict(sendMap=None), -5),
    ("recvCount null", {}, 0, dict(recvCount=None), -5),
    ("weights null with useWeights", {}, 8, dict(weights=None), -5),
    ("recvWeights null with useWeights", {}, 8, dict(recvWeights=None), -5),
    ("scratch too small", {}, 8, dict(scratchBytes=16), -6),
    ("scaleDim -1", dict(scaleDim=-1), 8, {}, -1),
    ("scaleDim above the maximum", dict(scaleDim=1025), 8, {}, -1),
    ("scales null with scaleDim", dict(scaleDim=4), 8, dict(scales=None), -5),
    ("recvScales null with scaleDim", dict(scaleDim=4), 8, dict(recvScales=None), -5),
    ("scales misaligned", dict(scaleDim=4), 8, dict(scales=P16 + 2), -4),
    ("recvScales misaligned", dict(scaleDim=4), 8, dict(recvScales=P16 + 1), -4),
]


@pytest.mark.parametrize("what,over,T,ptrs,code", REJECT, ids=[r[0] for r in REJECT])
def test_dispatch_rejects(what, over, T, ptrs, code):
    assert _dispatch(cfg(**over), T, **ptrs) == code
    assert epdc.epdc_last_error() != ""


COMBINE_REJECT = [
    ("worldSize 65", dict(worldSize=65), 8, {}, -1),
    ("dtype fp8 cannot be summed", dict(dtype=2), 8, {}, -2),
    ("dtype fp4x2 cannot be summed", dict(dtype=3), 8, {}, -2),
    ("dtype 4", dict(dtype=4), 8, {}, -2),
    ("fp32 row of 24 bytes", dict(hiddenDim=6, dtype=1), 8, {}, -4),
    ("capacity", {}, 4097, {}, -3),
    ("out misaligned", {}, 8, dict(out=P16 + 8), -4),
    ("y misaligned", {}, 8, dict(y=P16 + 2), -4),
    ("y null", {}, 8, dict(y=None), -5),
    ("weights null with useWeights", {}, 8, dict(weights=None), -5),
    ("expertIds null with useWeights", {}, 8, dict(expertIds=None), -5),
    ("sendMap null", {}, 8, dict(sendMap=None), -5),
    ("outDtype fp8", {}, 8, dict(outDtype=2), -2),
    ("outDtype 7", {}, 8, dict(outDtype=7), -2),
    ("outDtype fp4x2 with no tokens", {}, 0, dict(outDtype=3), -2),
]


@pytest.mark.parametrize("what,over,T,ptrs,code", COMBINE_REJECT, ids=[r[0] for r in COMBINE_REJECT])
def test_combine_rejects(what, over, T, ptrs, code):
    assert _combine(cfg(**over), T, **ptrs) == code
    assert epdc.epdc_last_error() != ""


def _push(c, T, **ptrs):
    args = dict(y=P16, recvExpertIds=P16, recvWeights=P16, recvCount=P16, landing=P16, landScale=P16)
    args.update(ptrs)
    return epdc.epdc_combine_push(c, T, args["y"], args["recvExpertIds"], args["recvWeights"], args["recvCount"],
                                  args["landing"], args["landScale"], stream=0, check=False)


def _reduce(c, T, outDtype=None, **ptrs):
    args = dict(landing=P16, landScale=P16, recvCount=P16, sendMap=P16, out=P16)
    args.update(ptrs)
    return epdc.epdc_combine_reduce(c, T, args["landing"], args["landScale"], args["recvCount"], args["sendMap"],
                                    args["out"], outDtype, stream=0, check=False)


PUSH_REJECT = [
    ("worldSize 0", dict(worldSize=0), 8, {}, -1),
    ("dtype fp8 cannot be summed", dict(dtype=2), 8, {}, -2),
    ("dtype fp4x2 cannot be summed", dict(dtype=3), 8, {}, -2),
    ("capacity", {}, 4097, {}, -3),
    ("negative tokens", {}, -1, {}, -1),
    ("row bytes not 16-aligned", dict(hiddenDim=7164), 8, {}, -4),
    ("y misaligned", {}, 8, dict(y=P16 + 8), -4),
    ("landing misaligned", {}, 8, dict(landing=P16 + 4), -4),
    ("recvCount misaligned", {}, 8, dict(recvCount=P16 + 2), -4),
    ("landScale misaligned", {}, 8, dict(landScale=P16 + 2), -4),
    ("y null", {}, 8, dict(y=None), -5),
    ("recvCount null", {}, 8, dict(recvCount=None), -5),
    ("landing null", {}, 8, dict(landing=None), -5),
    ("recvWeights null with useWeights", {}, 8, dict(recvWeights=None), -5),
    ("recvExpertIds null with useWeights", {}, 8, dict(recvExpertIds=None), -5),
    ("landScale null with useWeights", {}, 8, dict(landScale=None), -5),
]


@pytest.mark.parametrize("what,over,T,ptrs,code", PUSH_REJECT, ids=[r[0] for r in PUSH_REJECT])
def test_push_rejects(what, over, T, ptrs, code):
    assert _push(cfg(**over), T, **ptrs) == code
    assert epdc.epdc_last_error() != ""


REDUCE_REJECT = [
    ("topk 0", dict(numExpertPerToken=0), 8, {}, -1),
    ("dtype fp8 cannot be summed", dict(dtype=2), 8, {}, -2),
    ("capacity", {}, 4097, {}, -3),
    ("landing misaligned", {}, 8, dict(landing=P16 + 8), -4),
    ("out misaligned", {}, 8, dict(out=P16 + 8), -4),
    ("sendMap misaligned", {}, 8, dict(sendMap=P16 + 1), -4),
    ("landing null", {}, 8, dict(landing=None), -5),
    ("sendMap null", {}, 8, dict(sendMap=None), -5),
    ("recvCount null", {}, 8, dict(recvCount=None), -5),
    ("landScale null with useWeights", {}, 8, dict(landScale=None), -5),
    ("outDtype fp8", {}, 8, dict(outDtype=2), -2),
    ("outDtype -1", {}, 8, dict(outDtype=-1), -2),
]


@pytest.mark.parametrize("what,over,T,ptrs,code", REDUCE_REJECT, ids=[r[0] for r in REDUCE_REJECT])
def test_reduce_rejects(what, over, T, ptrs, code):
    assert _reduce(cfg(**over), T, **ptrs) == code
    assert epdc.epdc_last_error() != ""


def test_landing_rows():
    assert epdc.epdc_landing_rows(cfg(), 4096) == 4096 * 8
    assert epdc.epdc_landing_rows(cfg(worldSize=4, numExpertPerToken=6, numExpertPerRank=32), 512) == 512 * 4
    assert epdc.epdc_landing_rows(cfg(numExpertPerToken=2), 100) == 200
    assert epdc.epdc_landing_rows(cfg(), 0) == 0
    assert epdc.epdc_landing_rows(cfg(dtype=2), 8) == -1   # combine dtypes only
    assert epdc.epdc_landing_rows(cfg(), 4097) == -1       # numTokens > maxTokPerRank


def test_push_and_reduce_without_gpu():
    """Valid arguments pass every host check (the launch then reports
    EPDC_ERR_HIP with no GPU); no tokens is a no-op that needs no pointers;
    without useWeights the metadata and scale pointers may be NULL."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("host without a GPU only")
    assert _push(cfg(), 8) == -7
    assert _reduce(cfg(), 8) == -7
    assert _push(cfg(dtype=1), 8) == -7
    c = cfg(useWeights=0)
    assert _push(c, 8, recvExpertIds=None, recvWeights=None, landScale=None) == -7
    assert _reduce(c, 8, landScale=None) == -7
    n = dict(y=None, recvExpertIds=None, recvWeights=None, recvCount=None, landing=None, landScale=None)
    assert _push(cfg(), 0, **n) == 0
    assert _reduce(cfg(), 0, landing=None, landScale=None, recvCount=None, sendMap=None, out=None) == 0


def test_unweighted_accepts_null_weights_without_gpu():
    """Valid unweighted arguments pass every host check; with no GPU the
    launch itself reports EPDC_ERR_HIP instead of crashing."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("host without a GPU only")
    c = cfg(useWeights=0)
    assert _dispatch(c, 8, weights=None, recvWeights=None) == -7
    assert _combine(c, 8, weights=None) == -7
    assert _combine(c, 8, weights=None, expertIds=None) == -7  # unweighted: no expert ids needed
    assert "dispatch" in epdc.epdc_last_error() or "combine" in epdc.epdc_last_error()


def test_every_wire_dtype_passes_dispatch_checks_without_gpu():
    """bf16, fp32, fp8 and fp4x2 rows pass every host check of dispatch (the
    launch then reports EPDC_ERR_HIP on a host with no GPU); combine accepts
    only bf16 and fp32."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("host without a GPU only")
    for dt, h in ((0, 7168), (1, 7168), (2, 7168), (3, 3584), (2, 16), (1, 4)):
        assert _dispatch(cfg(dtype=dt, hiddenDim=h), 8) == -7, (dt, h, epdc.epdc_last_error())
    for dt in (0, 1):
        for odt in (0, 1):  # either row type into either output type
            assert _combine(cfg(dtype=dt), 8, outDtype=odt) == -7
            assert _reduce(cfg(dtype=dt), 8, outDtype=odt) == -7
    # scales: any scaleDim in range with both pointers
    for S in (1, 56, 64, 65, 1024):
        assert _dispatch(cfg(scaleDim=S), 8) == -7, (S, epdc.epdc_last_error())
    assert _dispatch(cfg(scaleDim=0), 8, scales=None, recvScales=None) == -7


def test_zero_tokens_needs_only_recvcount_without_gpu():
    import torch
    if torch.cuda.is_available():
        pytest.skip("host without a GPU only")
    n = dict(x=None, expertIds=None, weights=None, recvX=None, recvTokIdx=None, recvExpertIds=None,
             recvWeights=None, sendMap=None, scratch=None, scratchBytes=0)
    assert _dispatch(cfg(), 0, **n) == -7  # passes the checks, then no device
    assert _combine(cfg(), 0, y=None, expertIds=None, weights=None, sendMap=None, out=None) == 0


def test_prepared_calls_check_like_direct_calls():
    """A prepared call returns what the direct call returns: the host checks'
    codes for bad arguments, and (on a host with no GPU) EPDC_ERR_HIP for
    good ones."""
    import torch
    if torch.cuda.is_available():
        pytest.skip("host without a GPU only")
    ptrs = [P16] * 12
    bad = epdc.prepare_dispatch(cfg(), 4097, *ptrs, scratchBytes=1 << 20)
    assert bad(stream=0, check=False) == -3
    mis = epdc.prepare_dispatch(cfg(), 8, P16 + 8, *ptrs[1:], scratchBytes=1 << 20)
    assert mis(stream=0, check=False) == -4
    with pytest.raises(epdc.EpdcError):
        mis(stream=0)
    assert epdc.prepare_dispatch(cfg(), 8, *ptrs, scratchBytes=1 << 20)(stream=0, check=False) == -7
    assert epdc.prepare_combine(cfg(dtype=2), 8, *[P16] * 5)(stream=0, check=False) == -2
    assert epdc.prepare_combine(cfg(), 8, *[P16] * 5)(stream=0, check=False) == -7
    assert epdc.prepare_combine_push(cfg(), 8, *[P16] * 6)(stream=0, check=False) == -7
    assert epdc.prepare_combine_reduce(cfg(), 8, *[P16] * 5)(stream=0, check=False) == -7
    assert epdc.prepare_combine_reduce(cfg(), 8, P16, None, P16, P16, P16)(stream=0, check=False) == -5
    assert epdc.prepare_combine(cfg(), 8, *[P16] * 5, outDtype=2)(stream=0, check=False) == -2
    assert epdc.prepare_combine(cfg(dtype=1), 8, *[P16] * 5, outDtype=0)(stream=0, check=False) == -7


class _FakeDeviceTensor:
    """Reports a device placement and a layout like a torch tensor would."""

    def __init__(self, contiguous):
        self.is_cuda = True
        self._c = contiguous
        self.shape, self.device = (4, 4), "cuda:0"

    def is_contiguous(self):
        return self._c

    def stride(self):
        return (1, 4)

    def data_ptr(self):
        return P16


def test_binding_refuses_host_and_strided_tensors_before_any_call():
    import torch
    host = torch.zeros(64, dtype=torch.int32)
    ptrs = [P16] * 12
    with pytest.raises(ValueError, match="device tensor"):
        epdc.epdc_dispatch(cfg(), 8, host, *ptrs[1:], scratchBytes=1 << 20, stream=0)
    with pytest.raises(ValueError, match="contiguous"):
        epdc.epdc_combine(cfg(), 8, _FakeDeviceTensor(False), P16, P16, P16, P16, stream=0)
    with pytest.raises(ValueError, match="device tensor"):
        epdc.prepare_combine_reduce(cfg(), 8, P16, None, P16, host, P16)
    # a contiguous device tensor passes the binding (the library then runs its own checks)
    assert epdc.epdc_combine(cfg(dtype=2), 8, _FakeDeviceTensor(True), P16, P16, P16, P16, stream=0,
                             check=False) == -2


class _FakeSized(_FakeDeviceTensor):
    """A contiguous device tensor of a given byte size."""

    def __init__(self, nbytes):
        super().__init__(True)
        self._n = nbytes

    def numel(self):
        return self._n

    def element_size(self):
        return 1


def test_binding_refuses_short_buffers_before_any_call():
    """A tensor smaller than the call needs would be read or written past its
    end on the device: the binding refuses it, naming it, before the launch."""
    c = cfg(maxTokPerRank=64, scaleDim=4)  # W 8, H 7168 bf16, K 8, 8 tokens
    T, W, M, K, rb = 8, 8, 64, 8, 7168 * 2
    ok = dict(x=T * rb, expertIds=T * K * 4, weights=T * K * 4, scales=T * 4 * 4, recvX=W * M * rb,
              recvTokIdx=W * M * 4, recvExpertIds=W * M * K * 4, recvWeights=W * M * K * 4, recvScales=W * M * 4 * 4,
              recvCount=W * 4, sendMap=T * K * 4)
    names = list(ok)
    for short in names:
        args = [_FakeSized(ok[n] - (4 if n == short else 0)) for n in names]
        with pytest.raises(ValueError, match=f"^{short} holds"):
            epdc.epdc_dispatch(c, T, *args, P16, scratchBytes=1 << 20, stream=0)
        with pytest.raises(ValueError, match=f"^{short} holds"):
            epdc.prepare_dispatch(c, T, *args, P16, scratchBytes=1 << 20)
    cc = cfg(maxTokPerRank=64)
    full = dict(y=W * M * rb, expertIds=T * K * 4, weights=T * K * 4, sendMap=T * K * 4, out=T * 7168 * 4)
    for short in full:
        args = [_FakeSized(full[n] - (4 if n == short else 0)) for n in full]
        with pytest.raises(ValueError, match=f"^{short} holds"):
            epdc.epdc_combine(cc, T, *args, epdc.EPDC_FP32, stream=0)
    # an fp32 output needs twice the bytes of a bf16 one
    args = [_FakeSized(full[n] if n != "out" else T * 7168 * 2) for n in full]
    with pytest.raises(ValueError, match="^out holds"):
        epdc.epdc_combine(cc, T, *args, epdc.EPDC_FP32, stream=0)
    R = T * 8
    land = dict(landing=R * rb, landScale=R * 4, recvCount=W * 4, sendMap=T * K * 4, out=T * rb)
    for short in land:
        args = [_FakeSized(land[n] - (4 if n == short else 0)) for n in land]
        with pytest.raises(ValueError, match=f"^{short} holds"):
            epdc.epdc_combine_reduce(cc, T, *args, stream=0)
    push = dict(y=W * M * rb, recvExpertIds=W * M * K * 4, recvWeights=W * M * K * 4, recvCount=W * 4,
                landing=R * rb, landScale=R * 4)
    for short in push:
        args = [_FakeSized(push[n] - (4 if n == short else 0)) for n in push]
        with pytest.raises(ValueError, match=f"^{short} holds"):
            epdc.epdc_combine_push(cc, T, *args, stream=0)


def test_status_constants_match_the_header():
    """The binding's status-word constants are the header's (the library
    checks the header against its kernels' own at compile time)."""
    src = open(HEADER).read()
    for name in ("EPDC_STATUS_WORD", "EPDC_STATUS_WAIT_TIMEOUT", "EPDC_STATUS_ROW_OUTSIDE", "EPDC_MAX_SCALE_DIM"):
        m = re.search(rf"#define {name} (\d+)", src)
        assert m and int(m.group(1)) == getattr(epdc, name), name
    api = open(os.path.join(ROOT, "combine_count_amd", "csrc", "epdc_api.cpp")).read()
    assert "static_assert(EPDC_STATUS_WORD == epdc::kScratchError" in api


def test_dispatch_status_reads_the_status_word():
    import torch
    s = torch.zeros(1100, dtype=torch.int32)
    assert epdc.dispatch_status(s) == 0
    s[epdc.EPDC_STATUS_WORD] = epdc.EPDC_STATUS_WAIT_TIMEOUT
    assert epdc.dispatch_status(s) == 1
    assert epdc.dispatch_status(s.view(torch.uint8)) == 1
