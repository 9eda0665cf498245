"""Seeded synthetic inputs for the lightning indexer.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no scores, no visibility rule, no selection).  Both the
GPU tests/bench and the CPU oracle take their inputs from here.

Workloads mirror the pages' prefill and decode shapes: the last 2048-token
chunk of a cold 8k / 32k / 64k-context prefill at compression ratio 4 with
64 index heads of dim 128 and top-512 ("How I made DeepSeek 12x faster on a
Mac Studio", section "1: the kernels", cold-prefill table; the 2048-token
prefill step of "How I turned one oversized DeepSeek optimization into three
merged oMLX PRs", section "Independent upstream reproduction"), a single
decode token at the 1M-token window, and a tiny case for exhaustive checks.

Draw order for one workload, from numpy.random.default_rng(seed): q, then k,
then w (for power-of-two weights: the signs, then the exponents).
  * "int":   q, k integers uniform on {-4..4}, stored exactly in fp16;
             w = (+1 or -1) * 2^-n with n uniform on {0,1,2,3}, float32.
  * "gauss": q, k = N(0,1) / sqrt(128) drawn in float64, rounded to nearest
             even into float32 and then into the storage type (fp16 or
             bf16); w uniform on [0, 1) drawn as float32.
Positions are consecutive: pos = p0, p0+1, ..., p0+T-1 (int32).
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int          # query tokens
    p0: int         # position of the first query token
    N: int          # compressed rows present in K
    H: int          # index heads
    D: int          # head dim
    topk: int
    ratio: int
    dtype: str      # "f16" | "bf16"
    dist: str       # "int" | "gauss"
    seed: int = 0

    @property
    def positions(self) -> np.ndarray:
        return np.arange(self.p0, self.p0 + self.T, dtype=np.int32)


WORKLOADS = {
    "tiny": Workload("tiny", T=256, p0=0, N=64, H=4, D=32, topk=48, ratio=4,
                     dtype="f16", dist="int"),
    "prefill8k": Workload("prefill8k", T=2048, p0=6144, N=2048, H=64, D=128, topk=512,
                          ratio=4, dtype="f16", dist="int"),
    "prefill32k": Workload("prefill32k", T=2048, p0=30720, N=8192, H=64, D=128, topk=512,
                           ratio=4, dtype="f16", dist="int"),
    "prefill64k": Workload("prefill64k", T=2048, p0=63488, N=16384, H=64, D=128, topk=512,
                           ratio=4, dtype="bf16", dist="gauss"),
    "decode1m": Workload("decode1m", T=1, p0=1048575, N=262144, H=64, D=128, topk=512,
                         ratio=4, dtype="f16", dist="gauss"),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to nearest-even bfloat16; return the raw uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to nearest-even float32, then into fp16 / bf16 storage;
    return the raw uint16 bits."""
    x32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    if dtype == "f16":
        return x32.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def draw(T: int, N: int, H: int, D: int, dtype: str, dist: str, seed: int = 0,
         int_range: int = 4):
    """Draw (q_bits [T,H,D] u16, k_bits [N,D] u16, w [T,H] f32) for one workload."""
    rng = np.random.default_rng(seed)
    if dist == "int":
        q = rng.integers(-int_range, int_range + 1, size=(T, H, D)).astype(np.float64)
        k = rng.integers(-int_range, int_range + 1, size=(N, D)).astype(np.float64)
        sign = rng.integers(0, 2, size=(T, H)) * 2 - 1
        expo = rng.integers(0, 4, size=(T, H))
        w = (sign * np.ldexp(1.0, -expo)).astype(np.float32)
    elif dist == "gauss":
        q = rng.standard_normal(size=(T, H, D)) / math.sqrt(128.0)
        k = rng.standard_normal(size=(N, D)) / math.sqrt(128.0)
        w = rng.random(size=(T, H), dtype=np.float32)
    else:
        raise ValueError(dist)
    return to_bits(q, dtype), to_bits(k, dtype), w


def make(wl: Workload | str):
    """Inputs of a named workload: dict with q, k (uint16 bits), w, pos and the shape."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    q, k, w = draw(wl.T, wl.N, wl.H, wl.D, wl.dtype, wl.dist, wl.seed)
    return {"q": q, "k": k, "w": w, "pos": wl.positions, "wl": wl}
