"""Device buffers for the calls of include/epdc.h, allocated with torch.

A convenience for callers: every tensor has the extent and element type
include/epdc.h states for its argument.  PyTorch only allocates; the library
never does.  Row buffers take the cfg's dtype: bf16 and fp32 rows as
torch.bfloat16 / torch.float32, the one-byte fp8 and fp4x2 rows as uint8
(the library moves their bytes without reading them; for fp4x2 hiddenDim
counts bytes).
"""
from __future__ import annotations

import torch

from .binding import (EPDC_BF16, EPDC_FP4X2, EPDC_FP8, EPDC_FP32, EpCfg, EpdcError, epdc_dispatch_scratch_bytes,
                      epdc_landing_rows, epdc_last_error)

ROW_DTYPE = {EPDC_BF16: torch.bfloat16, EPDC_FP32: torch.float32, EPDC_FP8: torch.uint8, EPDC_FP4X2: torch.uint8}


def row_dtype(cfg: EpCfg) -> torch.dtype:
    if cfg.dtype not in ROW_DTYPE:
        raise ValueError(f"dtype {cfg.dtype} is not an EPDC dtype")
    return ROW_DTYPE[cfg.dtype]


class DispatchBuffers:
    """Outputs and scratch of epdc_dispatch for up to maxTokPerRank tokens
    (sendMap has maxTokPerRank rows; a call with T tokens writes the first
    T).  The scratch is zero-filled here, as its first use requires."""

    def __init__(self, cfg: EpCfg, device="cuda"):
        W, M, H, K = cfg.worldSize, cfg.maxTokPerRank, cfg.hiddenDim, cfg.numExpertPerToken
        nbytes = epdc_dispatch_scratch_bytes(cfg)
        if nbytes == 0:
            raise EpdcError(-1, epdc_last_error() or "invalid cfg")
        self.recvX = torch.empty((W, M, H), dtype=row_dtype(cfg), device=device)
        self.recvTokIdx = torch.empty((W, M), dtype=torch.int32, device=device)
        self.recvExpertIds = torch.empty((W, M, K), dtype=torch.int32, device=device)
        self.recvWeights = (torch.empty((W, M, K), dtype=torch.float32, device=device)
                            if cfg.useWeights else None)
        self.recvScales = (torch.empty((W, M, cfg.scaleDim), dtype=torch.float32, device=device)
                           if cfg.scaleDim > 0 else None)
        self.recvCount = torch.empty((W,), dtype=torch.int32, device=device)
        self.sendMap = torch.empty((M, K), dtype=torch.int32, device=device)
        self.scratch = torch.zeros((nbytes + 3) // 4, dtype=torch.int32, device=device)


class LandingBuffers:
    """Landing rows and forwarded scales of the scatter combine for numTokens
    tokens: epdc_landing_rows(cfg, numTokens) rows of the cfg's (bf16 or
    fp32) row type; landScale only when cfg.useWeights."""

    def __init__(self, cfg: EpCfg, numTokens: int, device="cuda"):
        rows = epdc_landing_rows(cfg, numTokens)
        if rows < 0:
            raise EpdcError(-1, "invalid cfg or numTokens for the scatter combine (bf16/fp32 rows, "
                                "0 <= numTokens <= maxTokPerRank)")
        self.landing = torch.empty((rows, cfg.hiddenDim), dtype=row_dtype(cfg), device=device)
        self.landScale = torch.empty((rows,), dtype=torch.float32, device=device) if cfg.useWeights else None
