"""Seeded synthetic inputs for the MoE dispatch/combine path.

This module is shared by the oracle tests, the GPU parity tests, ``smoke()``
and ``bench.py``.  It holds none of the method's arithmetic: it draws expert
ids, softmax routing weights and bf16 token rows from a numpy ``PCG64``
stream and hands the same bits to both sides.

Workload shapes follow the configurations the pages measure:

* MORI JIT v2 design doc, §3.2 (the ``EpCfg`` defaults: worldSize 8,
  hiddenDim 7168, maxTokPerRank 128, numExpertPerRank 8, numExpertPerToken 8,
  bf16, useWeights) and §8 (EP8, hidden 7168, topk 8, 128..4096 tokens per
  rank; EP4 64..16384 tokens per rank);
* mori PR #599 "Perf/ep disp 1250 ship", summary (ct=512, topk=6, EP4).

Draw order for one seed (fixed, so that any consumer regenerates the same
bits): expert ids, then routing logits, then ``x`` row by row, then ``y``
destination by destination.
"""
from __future__ import annotations

import dataclasses
import functools

import numpy as np
import torch


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic configuration; field names follow the pages' EpCfg."""
    name: str
    worldSize: int
    numExpertPerRank: int
    maxTokPerRank: int
    numTokens: int
    numExpertPerToken: int
    hiddenDim: int
    routing: str          # "uniform" or "zipf"
    useWeights: int
    zipf_s: float = 1.1
    wire: str = "bf16"          # dispatch row type: bf16, fp32, fp8 or fp4x2
    combineDtype: str = "bf16"  # combine row type: bf16 or fp32
    outDtype: str = ""          # combine output type: bf16 or fp32 ("" = combineDtype)
    scaleDim: int = 0           # fp32 scales per token forwarded by the dispatch

    @property
    def outType(self) -> str:
        return self.outDtype or self.combineDtype

    @property
    def numExperts(self) -> int:
        return self.worldSize * self.numExpertPerRank

    @property
    def dispatchHidden(self) -> int:
        """hiddenDim of the dispatch call: fp4x2 packs two values per byte and
        counts bytes (MORI JIT v2 design doc, §3.7)."""
        return self.hiddenDim // 2 if self.wire == "fp4x2" else self.hiddenDim

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five configurations (plus the two edge runs and both useWeights
# variants of the large prefill).  maxTokPerRank = numTokens unless stated.
CONFIGS: dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny", 4, 4, 8, 8, 2, 128, "uniform", 1),
        Workload("pr_scale", 4, 32, 512, 512, 6, 7168, "uniform", 1),
        Workload("epcfg_defaults", 8, 8, 128, 128, 8, 7168, "uniform", 1),
        Workload("gen_zipf_h2048", 8, 32, 4096, 4096, 8, 2048, "zipf", 1),
        Workload("gen_zipf_h7168", 8, 32, 4096, 4096, 8, 7168, "zipf", 1),
        Workload("gen_edge_t1", 8, 32, 4096, 1, 6, 7168, "zipf", 1),
        Workload("gen_edge_t8", 8, 32, 4096, 8, 6, 7168, "zipf", 1),
        Workload("large_unweighted", 8, 32, 16384, 16384, 8, 7168, "uniform", 0),
        Workload("large_weighted", 8, 32, 16384, 16384, 8, 7168, "uniform", 1),
    ]
}


def expert_logp(w: Workload) -> np.ndarray:
    """Log popularity of each expert id (unnormalised).

    uniform: all equal.  zipf: P(e) proportional to (e+1)^-s, the expert id
    being its popularity rank (no permutation).
    """
    E = w.numExperts
    if w.routing == "uniform":
        return np.zeros(E, dtype=np.float64)
    if w.routing == "zipf":
        return -w.zipf_s * np.log(np.arange(1, E + 1, dtype=np.float64))
    raise ValueError(f"unknown routing {w.routing!r}")


def draw_expert_ids(rng: np.random.Generator, w: Workload) -> np.ndarray:
    """K distinct expert ids per token, in draw order.

    Sequential draws without replacement from the popularity distribution,
    done as Gumbel-top-k: perturb each log-probability with an independent
    Gumbel variate and take the K largest, largest first.  Slot order is the
    draw order, so slots that share a PE need not be adjacent.
    """
    T, E, K = w.numTokens, w.numExperts, w.numExpertPerToken
    if K > E:
        raise ValueError("numExpertPerToken > number of experts")
    logp = expert_logp(w)
    out = np.empty((T, K), dtype=np.int32)
    step = 2048  # bounded temporary memory at 16384 x 256
    for t0 in range(0, T, step):
        n = min(step, T - t0)
        u = rng.random((n, E))
        keys = logp[None, :] - np.log(-np.log(u))
        top = np.argpartition(-keys, K - 1, axis=1)[:, :K]
        order = np.argsort(-np.take_along_axis(keys, top, axis=1), axis=1, kind="stable")
        out[t0:t0 + n] = np.take_along_axis(top, order, axis=1).astype(np.int32)
    return out


def softmax_weights(rng: np.random.Generator, w: Workload) -> np.ndarray:
    """Routing weights: fp32 softmax of N(0,1) logits over the K slots."""
    logits = rng.standard_normal((w.numTokens, w.numExpertPerToken), dtype=np.float32)
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    return (z / z.sum(axis=1, keepdims=True)).astype(np.float32)


WIRE_BYTES = {"bf16": 2, "fp32": 4, "fp8": 1, "fp4x2": 1}
EPDC_DTYPE = {"bf16": 0, "fp32": 1, "fp8": 2, "fp4x2": 3}

# e2m1 magnitudes of the 3-bit codes 0..7 (bit 3 is the sign)
_E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def rows_of(rng: np.random.Generator, shape, kind: str) -> np.ndarray:
    """N(0,1) rows in one of the row types.  bf16 -> uint16 bits; fp32 ->
    float32; fp8 -> uint8 e4m3 codes (torch's cast); fp4x2 -> uint8, two e2m1
    codes per byte (nearest magnitude, low nibble first), shape[-1] halved."""
    if kind == "bf16":
        return bf16_normal_bits(rng, shape)
    f = rng.standard_normal(shape, dtype=np.float32)
    if kind == "fp32":
        return f
    if kind == "fp8":
        return torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    if kind == "fp4x2":
        mag = np.abs(f)[..., None]
        code = np.argmin(np.abs(mag - _E2M1), axis=-1).astype(np.uint8) | (np.signbit(f).astype(np.uint8) << 3)
        return (code[..., 0::2] | (code[..., 1::2] << 4)).astype(np.uint8)
    raise ValueError(kind)


def bf16_normal_bits(rng: np.random.Generator, shape) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0,1) samples.

    The float32 draw is converted by torch's own float32->bfloat16 cast.
    """
    f = rng.standard_normal(shape, dtype=np.float32)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


@dataclasses.dataclass
class Inputs:
    w: Workload
    seed: int
    x: np.ndarray          # [T][dispatchHidden] token rows of the wire type
    expertIds: np.ndarray  # int32  [T][K]
    weights: np.ndarray    # fp32   [T][K]
    y: np.ndarray | None   # [W][M][H] returned rows of the combine type
    scales: np.ndarray | None = None  # fp32 [T][scaleDim], None when scaleDim == 0


def make_inputs(w: Workload, seed: int, with_y: bool = True) -> Inputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    ids = draw_expert_ids(rng, w)
    weights = softmax_weights(rng, w)
    x = rows_of(rng, (w.numTokens, w.hiddenDim), w.wire)
    y = None
    if with_y:
        ydt = np.uint16 if w.combineDtype == "bf16" else np.float32
        y = np.empty((w.worldSize, w.maxTokPerRank, w.hiddenDim), dtype=ydt)
        for p in range(w.worldSize):
            y[p] = rows_of(rng, (w.maxTokPerRank, w.hiddenDim), w.combineDtype)
    scales = token_scales(w, seed, w.scaleDim) if w.scaleDim else None
    return Inputs(w, seed, x, ids, weights, y, scales)


def token_scales(w: Workload, seed: int, scaleDim: int) -> np.ndarray:
    """Per-token quantisation scales forwarded by the dispatch: float32
    [T][scaleDim], drawn from their own PCG64 stream (the seed and a fixed
    tag), so that adding them changes no other input.  Values in the range
    of fp8 e4m3 block scales of N(0,1) rows (block max magnitude / 448)."""
    rng = np.random.Generator(np.random.PCG64([seed, 0x5CA1E]))
    return rng.uniform(0.004, 0.012, size=(w.numTokens, scaleDim)).astype(np.float32)


@functools.lru_cache(maxsize=4)
def cached_inputs(name: str, seed: int, with_y: bool = True) -> Inputs:
    return make_inputs(CONFIGS[name], seed, with_y)


def as_bf16_tensor(bits: np.ndarray) -> torch.Tensor:
    """View uint16 bf16 bits as a CPU torch.bfloat16 tensor (no copy)."""
    return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
