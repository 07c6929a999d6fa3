"""CPU oracle for MoE expert-parallel dispatch + combine (ctypes over plain C).

TEST INFRASTRUCTURE ONLY: only ``tests/``, ``__graft_entry__.smoke()`` and
``bench.py``'s ``cpu_baseline`` leg may import or call this package.  The
product library (``combine_count_amd``) never touches it and shares no code
with it.

The arithmetic lives in ``epdc_oracle.c`` (sequential, single-threaded,
``-O2 -ffp-contract=off``); this module only builds it with gcc when no
library is built yet and marshals numpy arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "epdc_oracle.c")
LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared"]


def build(src: str = SRC, out: str = LIB, extra: tuple = ()) -> str:
    """Compile the oracle with gcc; returns the library path."""
    tmp = out + f".tmp{os.getpid()}"
    subprocess.run(["gcc", *CFLAGS, *extra, "-o", tmp, src, "-lm"], check=True)
    os.replace(tmp, out)
    return out


_lib_cache: dict[str, ctypes.CDLL] = {}


def load(path: str | None = None) -> ctypes.CDLL:
    path = path or LIB
    if path in _lib_cache:
        return _lib_cache[path]
    if path == LIB and (not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC)):
        build()
    lib = ctypes.CDLL(path)
    i32, p = ctypes.c_int32, ctypes.c_void_p
    lib.oracle_dispatch.restype = i32
    lib.oracle_dispatch.argtypes = [i32] * 9 + [p] * 11
    lib.oracle_combine.restype = i32
    lib.oracle_combine.argtypes = [i32] * 9 + [p] * 5 + [i32, p, p]
    lib.oracle_combine_push.restype = i32
    lib.oracle_combine_push.argtypes = [i32] * 8 + [p] * 6
    lib.oracle_combine_reduce.restype = i32
    lib.oracle_combine_reduce.argtypes = [i32] * 9 + [p] * 5 + [i32, p, p]
    _lib_cache[path] = lib
    return lib


def _ptr(a):
    if a is None:
        return None
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data


class DispatchOut:
    def __init__(self, recvX, recvTokIdx, recvExpertIds, recvWeights, recvCount, sendMap, recvScales=None):
        self.recvX = recvX
        self.recvTokIdx = recvTokIdx
        self.recvExpertIds = recvExpertIds
        self.recvWeights = recvWeights
        self.recvCount = recvCount
        self.sendMap = sendMap
        self.recvScales = recvScales


def dispatch(W, H, M, Epr, K, useWeights, x, expertIds, weights, scales=None, *, fill=None, lib=None):
    """Run the oracle dispatch on numpy inputs.

    ``x``: [T][H] rows of any 1-, 2- or 4-byte element type (bf16 as uint16
    bits, fp32, fp8 / fp4x2 as uint8); ``expertIds``: int32 [T][K];
    ``weights``: float32 [T][K] or None; ``scales``: float32 [T][S] per-token
    scales forwarded with each row, or None (S = 0).  recvX has x's dtype.
    Windows are pre-filled with ``fill`` (a dict of sentinel values; recvX's
    is a byte, repeated) so that untouched rows stay recognisable.
    """
    lib = lib or load()
    T = x.shape[0]
    fill = fill or {}
    eb = x.dtype.itemsize
    recvX = np.empty((W, M, H), dtype=x.dtype)
    recvX.view(np.uint8)[...] = fill.get("recvX_byte", 0xAD)
    recvTokIdx = np.full((W, M), fill.get("recvTokIdx", 0), dtype=np.int32)
    recvExpertIds = np.full((W, M, K), fill.get("recvExpertIds", 0), dtype=np.int32)
    recvWeights = np.full((W, M, K), fill.get("recvWeights", 0), dtype=np.float32)
    recvCount = np.full((W,), -7, dtype=np.int32)
    sendMap = np.full((T, K), -99, dtype=np.int32)
    x = np.ascontiguousarray(x)
    expertIds = np.ascontiguousarray(expertIds, dtype=np.int32)
    if weights is not None:
        weights = np.ascontiguousarray(weights, dtype=np.float32)
    S = 0
    recvScales = None
    if scales is not None:
        scales = np.ascontiguousarray(scales, dtype=np.float32)
        assert scales.ndim == 2 and scales.shape[0] == T
        S = scales.shape[1]
        recvScales = np.full((W, M, S), fill.get("recvScales", 0), dtype=np.float32)
    rc = lib.oracle_dispatch(W, H, M, Epr, K, int(useWeights), T, eb, S,
                             _ptr(x), _ptr(expertIds), _ptr(weights), _ptr(scales),
                             _ptr(recvX), _ptr(recvTokIdx), _ptr(recvExpertIds),
                             _ptr(recvWeights), _ptr(recvScales), _ptr(recvCount), _ptr(sendMap))
    if rc != 0:
        raise ValueError(f"oracle_dispatch rejected its arguments ({rc})")
    return DispatchOut(recvX, recvTokIdx, recvExpertIds, recvWeights, recvCount, sendMap, recvScales)


def combine(W, H, M, Epr, K, useWeights, y, expertIds, weights, sendMap, tokens=None, out_fp32=None, lib=None):
    """Run the oracle combine.  ``y``: [W][M][H] bf16 bits (uint16) or
    float32; returns float32 rows if ``out_fp32`` else bf16 bits (uint16);
    by default the output type is y's.

    With ``tokens`` (an int sequence) only those tokens are combined, in that
    order; otherwise every token of ``sendMap``.
    """
    lib = lib or load()
    T = sendMap.shape[0]
    fp32 = y.dtype == np.float32
    ofp32 = fp32 if out_fp32 is None else bool(out_fp32)
    y = np.ascontiguousarray(y, dtype=np.float32 if fp32 else np.uint16)
    assert y.shape == (W, M, H)
    expertIds = np.ascontiguousarray(expertIds, dtype=np.int32)
    sendMap = np.ascontiguousarray(sendMap, dtype=np.int32)
    if weights is not None:
        weights = np.ascontiguousarray(weights, dtype=np.float32)
    tok = None
    n = T
    if tokens is not None:
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        n = tok.shape[0]
    out = np.empty((n, H), dtype=np.float32 if ofp32 else np.uint16)
    acc = np.empty((H,), dtype=np.float32)
    rc = lib.oracle_combine(W, H, M, Epr, K, int(useWeights), T, int(fp32), int(ofp32),
                            _ptr(y), _ptr(expertIds), _ptr(weights), _ptr(sendMap),
                            _ptr(tok), n, _ptr(acc), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_combine rejected its arguments ({rc})")
    return out


def landing_rows(W, K, T):
    """Landing capacity of the scatter combine: one row per (token, PE), at
    most min(W, K) PEs per token."""
    return T * min(W, K)


def combine_push(W, H, M, Epr, K, useWeights, T, y, recvExpertIds, recvWeights, recvCount, *,
                 fill_byte=0xA5, scale_fill=-3.25, lib=None):
    """Run the oracle push half of the scatter combine.  ``y``: [W][M][H]
    bf16 bits (uint16) or float32.  Returns (landing [T*min(W,K)][H] of y's
    dtype, landScale [T*min(W,K)] float32); rows not landed keep the fill."""
    lib = lib or load()
    fp32 = y.dtype == np.float32
    y = np.ascontiguousarray(y, dtype=np.float32 if fp32 else np.uint16)
    assert y.shape == (W, M, H)
    cap = landing_rows(W, K, T)
    landing = np.empty((cap, H), dtype=y.dtype)
    landing.view(np.uint8)[...] = fill_byte
    landScale = np.full((cap,), scale_fill, dtype=np.float32)
    recvExpertIds = np.ascontiguousarray(recvExpertIds, dtype=np.int32)
    recvCount = np.ascontiguousarray(recvCount, dtype=np.int32)
    if useWeights:
        recvWeights = np.ascontiguousarray(recvWeights, dtype=np.float32)
    rc = lib.oracle_combine_push(W, H, M, Epr, K, int(useWeights), T, int(fp32), _ptr(y), _ptr(recvExpertIds),
                                 _ptr(recvWeights) if useWeights else None, _ptr(recvCount),
                                 _ptr(landing), _ptr(landScale))
    if rc != 0:
        raise ValueError(f"oracle_combine_push rejected its arguments ({rc})")
    return landing, landScale


def combine_reduce(W, H, M, Epr, K, useWeights, landing, landScale, recvCount, sendMap, tokens=None,
                   out_fp32=None, lib=None):
    """Run the oracle reduce half of the scatter combine over the landing rows
    (bf16 bits or float32); returns one row per token (or per entry of
    ``tokens``), float32 if ``out_fp32`` else bf16 bits, by default the
    landing rows' type."""
    lib = lib or load()
    T = sendMap.shape[0]
    fp32 = landing.dtype == np.float32
    ofp32 = fp32 if out_fp32 is None else bool(out_fp32)
    landing = np.ascontiguousarray(landing, dtype=np.float32 if fp32 else np.uint16)
    assert landing.shape == (landing_rows(W, K, T), H)
    landScale = np.ascontiguousarray(landScale, dtype=np.float32)
    recvCount = np.ascontiguousarray(recvCount, dtype=np.int32)
    sendMap = np.ascontiguousarray(sendMap, dtype=np.int32)
    tok = None
    n = T
    if tokens is not None:
        tok = np.ascontiguousarray(np.asarray(tokens, dtype=np.int32))
        n = tok.shape[0]
    out = np.empty((n, H), dtype=np.float32 if ofp32 else np.uint16)
    acc = np.empty((H,), dtype=np.float32)
    rc = lib.oracle_combine_reduce(W, H, M, Epr, K, int(useWeights), T, int(fp32), int(ofp32), _ptr(landing),
                                   _ptr(landScale), _ptr(recvCount), _ptr(sendMap), _ptr(tok), n,
                                   _ptr(acc), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle_combine_reduce rejected its arguments ({rc})")
    return out


def timed_step(W, M, Epr, K, useWeights, x, expertIds, weights, y, push=False, scales=None, out_fp32=None,
               lib=None):
    """A callable running one oracle dispatch + combine into preallocated
    buffers (allocation kept out of the timed call), for bench.py's CPU
    baseline; with ``push`` the combine is the scatter combine's push then
    reduce.  x: [T][Hd] rows of any 1/2/4-byte type; y: [W][M][Hc] bf16 bits
    (uint16) or float32; scales: float32 [T][S] or None; out_fp32: output
    type of the combine (default: y's).  Returns (step, outputs)."""
    lib = lib or load()
    T, Hd = x.shape
    Hc = y.shape[2]
    fp32 = y.dtype == np.float32
    ofp32 = fp32 if out_fp32 is None else bool(out_fp32)
    S = 0 if scales is None else scales.shape[1]
    outs = dict(
        recvX=np.empty((W, M, Hd), x.dtype), recvTokIdx=np.empty((W, M), np.int32),
        recvExpertIds=np.empty((W, M, K), np.int32), recvWeights=np.empty((W, M, K), np.float32),
        recvScales=np.empty((W, M, S), np.float32),
        recvCount=np.empty((W,), np.int32), sendMap=np.empty((T, K), np.int32),
        out=np.empty((T, Hc), np.float32 if ofp32 else np.uint16), acc=np.empty((Hc,), np.float32),
        landing=np.empty((landing_rows(W, K, T) if push else 0, Hc), y.dtype),
        landScale=np.empty((landing_rows(W, K, T) if push else 0,), np.float32))
    x = np.ascontiguousarray(x)
    expertIds = np.ascontiguousarray(expertIds, dtype=np.int32)
    weights = np.ascontiguousarray(weights, dtype=np.float32) if useWeights else None
    scales = np.ascontiguousarray(scales, dtype=np.float32) if S else None
    y = np.ascontiguousarray(y)
    o = outs

    def step():
        rc = lib.oracle_dispatch(W, Hd, M, Epr, K, int(useWeights), T, x.itemsize, S, _ptr(x), _ptr(expertIds),
                                 _ptr(weights), _ptr(scales), _ptr(o["recvX"]), _ptr(o["recvTokIdx"]),
                                 _ptr(o["recvExpertIds"]), _ptr(o["recvWeights"]), _ptr(o["recvScales"]),
                                 _ptr(o["recvCount"]), _ptr(o["sendMap"]))
        if push:
            rc |= lib.oracle_combine_push(W, Hc, M, Epr, K, int(useWeights), T, int(fp32), _ptr(y),
                                          _ptr(o["recvExpertIds"]), _ptr(o["recvWeights"]), _ptr(o["recvCount"]),
                                          _ptr(o["landing"]), _ptr(o["landScale"]))
            rc |= lib.oracle_combine_reduce(W, Hc, M, Epr, K, int(useWeights), T, int(fp32), int(ofp32),
                                            _ptr(o["landing"]), _ptr(o["landScale"]), _ptr(o["recvCount"]),
                                            _ptr(o["sendMap"]), None, T, _ptr(o["acc"]), _ptr(o["out"]))
        else:
            rc |= lib.oracle_combine(W, Hc, M, Epr, K, int(useWeights), T, int(fp32), int(ofp32), _ptr(y),
                                     _ptr(expertIds), _ptr(weights), _ptr(o["sendMap"]), None, T, _ptr(o["acc"]),
                                     _ptr(o["out"]))
        if rc:
            raise RuntimeError("oracle step failed")

    return step, outs
