"""ctypes binding of libepdc.so (include/epdc.h), same entry-point names.

Argument marshalling only: tensors become their device pointers (after a
check that each is on the device, contiguous and at least as large as the
call needs), the stream defaults to torch's current stream, and a negative
return code becomes an ``EpdcError``.  Every step of dispatch and combine runs in the HIP kernels of
libepdc.so; there is no other code path.  If the library is not built this
module raises on first use.
"""
from __future__ import annotations

import ctypes
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libepdc.so")

EPDC_BF16, EPDC_FP32, EPDC_FP8, EPDC_FP4X2 = 0, 1, 2, 3
ERRORS = {
    -1: "EPDC_ERR_INVALID_ARG",
    -2: "EPDC_ERR_UNSUPPORTED",
    -3: "EPDC_ERR_CAPACITY",
    -4: "EPDC_ERR_ALIGN",
    -5: "EPDC_ERR_NULLPTR",
    -6: "EPDC_ERR_SCRATCH",
    -7: "EPDC_ERR_HIP",
}
EXPORTS = ("epdc_dispatch_scratch_bytes", "epdc_dispatch", "epdc_dispatch_noalloc", "epdc_combine",
           "epdc_landing_rows", "epdc_combine_push", "epdc_combine_reduce", "epdc_last_error")
# include/epdc.h: the dispatch scratch's status word (index in 32-bit words) and its values
EPDC_STATUS_WORD = 2
EPDC_STATUS_WAIT_TIMEOUT = 1
EPDC_STATUS_ROW_OUTSIDE = 2
EPDC_MAX_SCALE_DIM = 1024


class EpdcError(RuntimeError):
    def __init__(self, code: int, message: str):
        super().__init__(f"{ERRORS.get(code, code)}: {message}")
        self.code = code


class EpCfg(ctypes.Structure):
    """epdc_cfg: field names as in the pages' EpCfg."""
    _fields_ = [
        ("worldSize", ctypes.c_int32),
        ("hiddenDim", ctypes.c_int32),
        ("maxTokPerRank", ctypes.c_int32),
        ("numExpertPerRank", ctypes.c_int32),
        ("numExpertPerToken", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("useWeights", ctypes.c_int32),
        ("scaleDim", ctypes.c_int32),
    ]

    def __repr__(self):
        return "EpCfg(" + ", ".join(f"{n}={getattr(self, n)}" for n, _ in self._fields_) + ")"


_lib = None


def load_library() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built: run __graft_entry__.build() "
                           "(hipcc --offload-arch=gfx950); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    p, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    cfgp = ctypes.POINTER(EpCfg)
    lib.epdc_dispatch_scratch_bytes.restype = sz
    lib.epdc_dispatch_scratch_bytes.argtypes = [cfgp]
    lib.epdc_dispatch.restype = ctypes.c_int
    lib.epdc_dispatch.argtypes = [cfgp, i32] + [p] * 12 + [sz, p]
    lib.epdc_dispatch_noalloc.restype = ctypes.c_int
    lib.epdc_dispatch_noalloc.argtypes = [cfgp, i32] + [p] * 11 + [p]
    lib.epdc_combine.restype = ctypes.c_int
    lib.epdc_combine.argtypes = [cfgp, i32] + [p] * 5 + [i32, p]
    lib.epdc_landing_rows.restype = i32
    lib.epdc_landing_rows.argtypes = [cfgp, i32]
    lib.epdc_combine_push.restype = ctypes.c_int
    lib.epdc_combine_push.argtypes = [cfgp, i32] + [p] * 6 + [p]
    lib.epdc_combine_reduce.restype = ctypes.c_int
    lib.epdc_combine_reduce.argtypes = [cfgp, i32] + [p] * 5 + [i32, p]
    lib.epdc_last_error.restype = ctypes.c_char_p
    lib.epdc_last_error.argtypes = []
    _lib = lib
    return lib


def _ptr(a):
    """Device address of a buffer argument: None, a raw address (int), or a
    contiguous device tensor (anything else is refused before any launch: a
    host pointer would fault the GPU, a strided view would be read densely)."""
    if a is None:
        return None
    if isinstance(a, int):
        return a
    if not a.is_cuda:
        raise ValueError(f"expected a device tensor, got one on {a.device}")
    if not a.is_contiguous():
        raise ValueError(f"expected a contiguous tensor, got strides {tuple(a.stride())} for shape {tuple(a.shape)}")
    return a.data_ptr()


_ELEM = {EPDC_BF16: 2, EPDC_FP32: 4, EPDC_FP8: 1, EPDC_FP4X2: 1}


def _need(a, nbytes: int, name: str):
    """A tensor argument must hold at least the bytes include/epdc.h states
    for it (a short buffer would be read or written past its end on the
    device).  Raw addresses and None pass through unchecked."""
    if a is None or isinstance(a, int):
        return
    _ptr(a)  # device and layout first
    if not hasattr(a, "element_size"):
        return
    have = a.numel() * a.element_size()
    if have < nbytes:
        raise ValueError(f"{name} holds {have} bytes, the call needs {nbytes}")


def _sizes_dispatch(cfg, T, x, expertIds, weights, scales, recvX, recvTokIdx, recvExpertIds, recvWeights,
                    recvScales, recvCount, sendMap):
    W, M, H, K, S = cfg.worldSize, cfg.maxTokPerRank, cfg.hiddenDim, cfg.numExpertPerToken, cfg.scaleDim
    eb = _ELEM.get(cfg.dtype)
    if eb is None or T <= 0 or min(W, M, H, K) < 1 or S < 0:
        return  # the library rejects it, or nothing token-sized is touched
    rb = H * eb
    for a, n, name in ((x, T * rb, "x"), (expertIds, T * K * 4, "expertIds"), (recvX, W * M * rb, "recvX"),
                       (recvTokIdx, W * M * 4, "recvTokIdx"), (recvExpertIds, W * M * K * 4, "recvExpertIds"),
                       (recvCount, W * 4, "recvCount"), (sendMap, T * K * 4, "sendMap"),
                       (weights, T * K * 4 if cfg.useWeights else 0, "weights"),
                       (recvWeights, W * M * K * 4 if cfg.useWeights else 0, "recvWeights"),
                       (scales, T * S * 4, "scales"), (recvScales, W * M * S * 4, "recvScales")):
        _need(a, n, name)


def _sizes_combine(cfg, T, outDtype, y, expertIds, weights, sendMap, out, landing=False):
    W, M, H, K = cfg.worldSize, cfg.maxTokPerRank, cfg.hiddenDim, cfg.numExpertPerToken
    eb, ob = {EPDC_BF16: 2, EPDC_FP32: 4}.get(cfg.dtype), {EPDC_BF16: 2, EPDC_FP32: 4}.get(outDtype)
    if eb is None or ob is None or T <= 0 or min(W, M, H, K) < 1:
        return
    rows = T * min(W, K) if landing else W * M
    _need(y, rows * H * eb, "landing" if landing else "y")
    _need(sendMap, T * K * 4, "sendMap")
    _need(out, T * H * ob, "out")
    if cfg.useWeights:
        _need(weights, (rows if landing else T * K) * 4, "landScale" if landing else "weights")
        if not landing:
            _need(expertIds, T * K * 4, "expertIds")


def _sizes_push(cfg, T, y, recvExpertIds, recvWeights, recvCount, landing, landScale):
    W, M, H, K = cfg.worldSize, cfg.maxTokPerRank, cfg.hiddenDim, cfg.numExpertPerToken
    eb = {EPDC_BF16: 2, EPDC_FP32: 4}.get(cfg.dtype)
    if eb is None or T <= 0 or min(W, M, H, K) < 1:
        return
    R = T * min(W, K)
    _need(y, W * M * H * eb, "y")
    _need(recvCount, W * 4, "recvCount")
    _need(landing, R * H * eb, "landing")
    if cfg.useWeights:
        _need(recvExpertIds, W * M * K * 4, "recvExpertIds")
        _need(recvWeights, W * M * K * 4, "recvWeights")
        _need(landScale, R * 4, "landScale")


_current_stream = None


def _stream(s):
    """hipStream_t of `s`: an int passes through, a torch stream gives its
    handle, None gives torch's current stream on the current device (through
    torch's raw-handle query when it has one: no Stream object per call)."""
    global _current_stream
    if s is None:
        if _current_stream is None:
            import torch
            raw = getattr(torch._C, "_cuda_getCurrentRawStream", None)
            dev = getattr(torch._C, "_cuda_getDevice", None)
            if raw is not None and dev is not None:
                _current_stream = lambda: raw(dev())
            else:
                _current_stream = lambda: torch.cuda.current_stream().cuda_stream
        return _current_stream()
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _check(rc: int, check: bool) -> int:
    if rc != 0 and check:
        raise EpdcError(rc, epdc_last_error())
    return rc


def epdc_last_error() -> str:
    return load_library().epdc_last_error().decode()


def epdc_dispatch_scratch_bytes(cfg: EpCfg) -> int:
    return load_library().epdc_dispatch_scratch_bytes(ctypes.byref(cfg))


def epdc_dispatch(cfg: EpCfg, numTokens: int, x, expertIds, weights, scales, recvX, recvTokIdx, recvExpertIds,
                  recvWeights, recvScales, recvCount, sendMap, scratch, scratchBytes: int | None = None,
                  stream=None, check: bool = True) -> int:
    if scratchBytes is None:
        scratchBytes = 0 if scratch is None or isinstance(scratch, int) else scratch.numel() * scratch.element_size()
    _sizes_dispatch(cfg, numTokens, x, expertIds, weights, scales, recvX, recvTokIdx, recvExpertIds, recvWeights,
                    recvScales, recvCount, sendMap)
    rc = (_lib or load_library()).epdc_dispatch(
        ctypes.byref(cfg), int(numTokens), _ptr(x), _ptr(expertIds), _ptr(weights), _ptr(scales), _ptr(recvX),
        _ptr(recvTokIdx), _ptr(recvExpertIds), _ptr(recvWeights), _ptr(recvScales), _ptr(recvCount),
        _ptr(sendMap), _ptr(scratch), int(scratchBytes), _stream(stream))
    return _check(rc, check)


def epdc_dispatch_noalloc(cfg: EpCfg, numTokens: int, x, expertIds, weights, scales, recvX, recvTokIdx,
                          recvExpertIds, recvWeights, recvScales, recvCount, sendMap, stream=None,
                          check: bool = True) -> int:
    _sizes_dispatch(cfg, numTokens, x, expertIds, weights, scales, recvX, recvTokIdx, recvExpertIds, recvWeights,
                    recvScales, recvCount, sendMap)
    rc = (_lib or load_library()).epdc_dispatch_noalloc(
        ctypes.byref(cfg), int(numTokens), _ptr(x), _ptr(expertIds), _ptr(weights), _ptr(scales), _ptr(recvX),
        _ptr(recvTokIdx), _ptr(recvExpertIds), _ptr(recvWeights), _ptr(recvScales), _ptr(recvCount),
        _ptr(sendMap), _stream(stream))
    return _check(rc, check)


def _out_dtype(cfg: EpCfg, outDtype) -> int:
    """outDtype of a combine or reduce; None means the rows' own type."""
    return cfg.dtype if outDtype is None else int(outDtype)


def epdc_combine(cfg: EpCfg, numTokens: int, y, expertIds, weights, sendMap, out, outDtype=None, stream=None,
                 check: bool = True) -> int:
    _sizes_combine(cfg, numTokens, _out_dtype(cfg, outDtype), y, expertIds, weights, sendMap, out)
    rc = (_lib or load_library()).epdc_combine(
        ctypes.byref(cfg), int(numTokens), _ptr(y), _ptr(expertIds), _ptr(weights), _ptr(sendMap),
        _ptr(out), _out_dtype(cfg, outDtype), _stream(stream))
    return _check(rc, check)


def epdc_landing_rows(cfg: EpCfg, numTokens: int) -> int:
    return load_library().epdc_landing_rows(ctypes.byref(cfg), int(numTokens))


def epdc_combine_push(cfg: EpCfg, numTokens: int, y, recvExpertIds, recvWeights, recvCount, landing, landScale,
                      stream=None, check: bool = True) -> int:
    _sizes_push(cfg, numTokens, y, recvExpertIds, recvWeights, recvCount, landing, landScale)
    rc = (_lib or load_library()).epdc_combine_push(
        ctypes.byref(cfg), int(numTokens), _ptr(y), _ptr(recvExpertIds), _ptr(recvWeights), _ptr(recvCount),
        _ptr(landing), _ptr(landScale), _stream(stream))
    return _check(rc, check)


def epdc_combine_reduce(cfg: EpCfg, numTokens: int, landing, landScale, recvCount, sendMap, out, outDtype=None,
                        stream=None, check: bool = True) -> int:
    _sizes_combine(cfg, numTokens, _out_dtype(cfg, outDtype), landing, None, landScale, sendMap, out, landing=True)
    _need(recvCount, cfg.worldSize * 4, "recvCount")
    rc = (_lib or load_library()).epdc_combine_reduce(
        ctypes.byref(cfg), int(numTokens), _ptr(landing), _ptr(landScale), _ptr(recvCount), _ptr(sendMap),
        _ptr(out), _out_dtype(cfg, outDtype), _stream(stream))
    return _check(rc, check)


def dispatch_status(scratch) -> int:
    """The status word of a dispatch scratch buffer (a device tensor), read
    after the caller's own synchronisation: 0, EPDC_STATUS_WAIT_TIMEOUT or
    EPDC_STATUS_ROW_OUTSIDE (include/epdc.h).  One 4-byte copy to the host."""
    import torch
    words = scratch.view(torch.int32) if scratch.element_size() != 4 or scratch.dtype != torch.int32 else scratch
    return int(words.reshape(-1)[EPDC_STATUS_WORD].item())


class PreparedCall:
    """One entry point with every argument but the stream marshalled once.

    For launch loops that reuse the same buffers (a serving step, a
    benchmark): the device pointers and sizes are fixed at preparation, so a
    call costs one ctypes call.  The buffers must stay alive and in place as
    long as the prepared call is used; `keep` holds references to them."""

    def __init__(self, fn, args, keep):
        self._fn = fn
        self._args = tuple(args)
        self._keep = keep

    def __call__(self, stream=None, check: bool = True) -> int:
        rc = self._fn(*self._args, _stream(stream))
        if rc != 0 and check:
            raise EpdcError(rc, epdc_last_error())
        return rc


def _vp(a):
    p = _ptr(a)
    return ctypes.c_void_p(p) if p is not None else None


def prepare_dispatch(cfg: EpCfg, numTokens: int, x, expertIds, weights, scales, recvX, recvTokIdx, recvExpertIds,
                     recvWeights, recvScales, recvCount, sendMap, scratch,
                     scratchBytes: int | None = None) -> PreparedCall:
    if scratchBytes is None:
        scratchBytes = 0 if scratch is None or isinstance(scratch, int) else scratch.numel() * scratch.element_size()
    _sizes_dispatch(cfg, numTokens, x, expertIds, weights, scales, recvX, recvTokIdx, recvExpertIds, recvWeights,
                    recvScales, recvCount, sendMap)
    bufs = (x, expertIds, weights, scales, recvX, recvTokIdx, recvExpertIds, recvWeights, recvScales, recvCount,
            sendMap, scratch)
    args = [ctypes.byref(cfg), ctypes.c_int32(int(numTokens)), *(_vp(b) for b in bufs),
            ctypes.c_size_t(int(scratchBytes))]
    return PreparedCall((_lib or load_library()).epdc_dispatch, args, (cfg, bufs))


def prepare_combine(cfg: EpCfg, numTokens: int, y, expertIds, weights, sendMap, out, outDtype=None) -> PreparedCall:
    _sizes_combine(cfg, numTokens, _out_dtype(cfg, outDtype), y, expertIds, weights, sendMap, out)
    bufs = (y, expertIds, weights, sendMap, out)
    args = [ctypes.byref(cfg), ctypes.c_int32(int(numTokens)), *(_vp(b) for b in bufs),
            ctypes.c_int32(_out_dtype(cfg, outDtype))]
    return PreparedCall((_lib or load_library()).epdc_combine, args, (cfg, bufs))


def prepare_combine_push(cfg: EpCfg, numTokens: int, y, recvExpertIds, recvWeights, recvCount, landing,
                         landScale) -> PreparedCall:
    _sizes_push(cfg, numTokens, y, recvExpertIds, recvWeights, recvCount, landing, landScale)
    bufs = (y, recvExpertIds, recvWeights, recvCount, landing, landScale)
    args = [ctypes.byref(cfg), ctypes.c_int32(int(numTokens)), *(_vp(b) for b in bufs)]
    return PreparedCall((_lib or load_library()).epdc_combine_push, args, (cfg, bufs))


def prepare_combine_reduce(cfg: EpCfg, numTokens: int, landing, landScale, recvCount, sendMap, out,
                           outDtype=None) -> PreparedCall:
    _sizes_combine(cfg, numTokens, _out_dtype(cfg, outDtype), landing, None, landScale, sendMap, out, landing=True)
    _need(recvCount, cfg.worldSize * 4, "recvCount")
    bufs = (landing, landScale, recvCount, sendMap, out)
    args = [ctypes.byref(cfg), ctypes.c_int32(int(numTokens)), *(_vp(b) for b in bufs),
            ctypes.c_int32(_out_dtype(cfg, outDtype))]
    return PreparedCall((_lib or load_library()).epdc_combine_reduce, args, (cfg, bufs))
