"""Device buffers for one dispatch/combine pair, allocated with torch.

A convenience for callers and tests: every tensor has the extent and dtype
include/epdc.h states for its argument.  PyTorch only allocates; the
library never does.
"""
from __future__ import annotations

import torch

from .binding import EpCfg, epdc_dispatch_scratch_bytes


class DispatchBuffers:
    def __init__(self, cfg: EpCfg, device="cuda"):
        W, M, H, K = cfg.worldSize, cfg.maxTokPerRank, cfg.hiddenDim, cfg.numExpertPerToken
        self.recvX = torch.empty((W, M, H), dtype=torch.bfloat16, device=device)
        self.recvTokIdx = torch.empty((W, M), dtype=torch.int32, device=device)
        self.recvExpertIds = torch.empty((W, M, K), dtype=torch.int32, device=device)
        self.recvWeights = (torch.empty((W, M, K), dtype=torch.float32, device=device)
                            if cfg.useWeights else None)
        self.recvCount = torch.empty((W,), dtype=torch.int32, device=device)
        self.sendMap = torch.empty((M, K), dtype=torch.int32, device=device)
        nbytes = epdc_dispatch_scratch_bytes(cfg)
        self.scratch = torch.zeros((max(nbytes, 4) + 3) // 4, dtype=torch.int32, device=device)
