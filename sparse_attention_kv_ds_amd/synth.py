"""Seeded synthetic inputs for the lightning indexer and for the sparse
attention that consumes its selection.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no scores, no visibility rule, no selection).  Both the
GPU tests/bench and the CPU oracle take their inputs from here.

Workloads mirror the pages' prefill and decode shapes: the last 2048-token
chunk of a cold 8k / 32k / 64k-context prefill at compression ratio 4 with
64 index heads of dim 128 and top-512 ("How I made DeepSeek 12x faster on a
Mac Studio", section "1: the kernels", cold-prefill table; the 2048-token
prefill step of "How I turned one oversized DeepSeek optimization into three
merged oMLX PRs", section "Independent upstream reproduction"), a single
decode token at the 1M-token window, a tiny case for exhaustive checks, and
the first 2048-token chunk of a prompt (every row fits in the top-512).

Draw order for one workload, from numpy.random.default_rng(seed): q, then k,
then w (for power-of-two weights: the signs, then the exponents).
  * "int":   q, k integers uniform on {-4..4}, stored exactly in fp16;
             w = (+1 or -1) * 2^-n with n uniform on {0,1,2,3}, float32.
  * "gauss": q, k = N(0,1) / sqrt(128) drawn in float64 and rounded once, to
             nearest even, into the storage type (fp16 or bf16); w uniform on
             [0, 1) drawn as float32.
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
    # the first 2048-token chunk of any prompt: 512 rows, all of them fit in top-512
    "prefill2k": Workload("prefill2k", T=2048, p0=0, N=512, H=64, D=128, topk=512, ratio=4,
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


# query projection ahead of the indexer: the 32k chunk's shape (2048 tokens at
# 30720..32767, 8192 rows, 64 x 128 heads, top-512) with a query input of
# d_in features per token and projection weights [H*D][d_in], all Gaussian in
# bf16: x = N(0,1), wq = N(0,1) / sqrt(128 d_in) (so q ~ N(0,1)/sqrt(128) as in
# the Gaussian workloads), k = N(0,1)/sqrt(128), w uniform [0,1).  Draw order
# from default_rng(seed): x, wq, k, w.
PROJ_WORKLOADS = {"qproj32k": ("prefill32k", 1536, "bf16", 7)}


def make_projection(name: str):
    base, din, dtype, seed = PROJ_WORKLOADS[name]
    wl = WORKLOADS[base]
    rng = np.random.default_rng(seed)
    x = to_bits(rng.standard_normal((wl.T, din)), dtype)
    wq = to_bits(rng.standard_normal((wl.H * wl.D, din)) / math.sqrt(128.0 * din), dtype)
    k = to_bits(rng.standard_normal((wl.N, wl.D)) / math.sqrt(128.0), dtype)
    w = rng.random((wl.T, wl.H), dtype=np.float32)
    return {"x": x, "wq": wq, "k": k, "w": w, "pos": wl.positions, "wl": wl, "din": din,
            "dtype": dtype}


# batched decode: B sequences, each drawn like the single-token workload with
# seed + b (sequence b's q, k, w in that order), all at the same position
DECODE_BATCHES = {"decode1m_b8": ("decode1m", 8)}


def make_decode_batch(name: str):
    """Inputs of a batched decode workload: q [B,H,D], k [B,N,D] (uint16 bits),
    w [B,H], pos [B] and the per-sequence workload."""
    base, B = DECODE_BATCHES[name]
    wl = WORKLOADS[base]
    qs, ks, ws = [], [], []
    for b in range(B):
        q, k, w = draw(wl.T, wl.N, wl.H, wl.D, wl.dtype, wl.dist, wl.seed + b)
        qs.append(q[0]); ks.append(k); ws.append(w[0])
    pos = np.full(B, wl.p0, dtype=np.int32)
    return {"q": np.stack(qs), "k": np.stack(ks), "w": np.stack(ws), "pos": pos, "wl": wl, "B": B}


# significand bits (with the leading one), least normal exponent and largest
# finite value of the two storage types
_FORMATS = {"f16": (11, -14, 65504.0), "bf16": (8, -126, 3.3895313892515355e38)}


def to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest fp16 / bf16 value (ties to even, one
    rounding, overflow to infinity); return the raw uint16 bits."""
    if dtype not in _FORMATS:
        raise ValueError(dtype)
    p, emin, fmax = _FORMATS[dtype]
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        _, e2 = np.frexp(x)                          # |x| = m 2^e2, m in [0.5, 1)
        e = np.maximum(e2.astype(np.int64) - 1, emin)  # exponent of x's binade (subnormals: emin)
        ulp = np.ldexp(1.0, (e - (p - 1)).astype(np.int32))
        r = np.rint(x / ulp) * ulp                   # exact: scaling by powers of two
        r = np.where(np.abs(r) > fmax, np.copysign(np.inf, x), r)
        r = np.where(np.isfinite(x), r, x)
    if dtype == "f16":
        return r.astype(np.float16).view(np.uint16)  # exact: r is an fp16 value
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


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


# --- sparse attention over the selected rows ---------------------------------
#
# The attention consumes, per token, a list of pooled rows (in the full path,
# the indexer's selection).  Its inputs here are drawn independently of any
# indexer run: the list of token t holds m_t distinct pooled rows drawn
# uniformly from 0..N-1, ascending, padded with -1, with m_t = topk except
# for every `short_every`-th token, whose list is cut to a random length (the
# attention itself does not require the rows to be causally visible; that is
# the indexer's guarantee).  The query heads, pooled keys and values, and raw
# (local) keys and values are N(0,1) draws (queries and keys scaled by
# 1/sqrt(DK)), rounded to the storage type.  Draw order from
# default_rng(seed): q, kp, vp, kl, vl, then the index lists token by token.

@dataclasses.dataclass(frozen=True)
class AttnWorkload:
    name: str
    T: int          # query tokens
    p0: int         # position of the first query token
    N: int          # pooled (compressed) rows
    L: int          # raw rows kept, indexed by absolute position
    HA: int         # attention heads
    DK: int
    DV: int
    topk: int
    window: int     # local rows per token (the causal sliding window)
    dtype: str
    short_every: int = 0  # every n-th token gets a shorter index list (0: none)
    seed: int = 0
    ratio: int = 0  # > 0: no index list; every pooled row a token can see (all-visible form)

    @property
    def positions(self) -> np.ndarray:
        return np.arange(self.p0, self.p0 + self.T, dtype=np.int32)

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.DK)


ATTN_WORKLOADS = {
    "attn_tiny": AttnWorkload("attn_tiny", T=96, p0=100, N=49, L=196, HA=32, DK=64, DV=64,
                              topk=16, window=8, dtype="f16", short_every=5),
    # the consumer of the 32k prefill chunk's indices
    "attn32k": AttnWorkload("attn32k", T=2048, p0=30720, N=8192, L=32768, HA=64, DK=128, DV=128,
                            topk=512, window=128, dtype="bf16"),
    # the same chunk in a ratio-128 layer: every visible pooled row (240..256 of
    # 256), no indexer
    "attn32k_r128": AttnWorkload("attn32k_r128", T=2048, p0=30720, N=256, L=32768, HA=64, DK=128,
                                 DV=128, topk=0, window=128, dtype="bf16", ratio=128),
}


def draw_index_lists(rng, T: int, N: int, topk: int, short_every: int = 0) -> np.ndarray:
    """Per token: an ascending set of distinct rows of 0..N-1, -1 padded to topk
    entries -- the rows holding the m smallest of N uniform draws, with
    m = min(N, topk), or a uniform count in 0..m for every short_every-th token
    (those counts are drawn after all the uniforms)."""
    idx = np.full((T, topk), -1, dtype=np.int32)
    full = min(N, topk)
    if T == 0 or full == 0:
        return idx
    keys = rng.random((T, N), dtype=np.float32)
    part = np.argpartition(keys, full - 1, axis=1)[:, :full] if full < N else \
        np.broadcast_to(np.arange(N), (T, N)).copy()
    order = np.argsort(np.take_along_axis(keys, part, axis=1), axis=1, kind="stable")
    part = np.take_along_axis(part, order, axis=1)  # by increasing draw
    m = np.full(T, full, dtype=np.int64)
    if short_every:
        sel = np.arange(T) % short_every == short_every - 1
        m[sel] = rng.integers(0, full + 1, size=int(sel.sum()))
    for t in range(T):
        if m[t]:
            idx[t, :m[t]] = np.sort(part[t, :m[t]])
    return idx


def make_attention(wl: AttnWorkload | str):
    """Inputs of a named attention workload (raw uint16 bits for the 16-bit tensors)."""
    if isinstance(wl, str):
        wl = ATTN_WORKLOADS[wl]
    rng = np.random.default_rng(wl.seed)
    sk = 1.0 / math.sqrt(wl.DK)
    q = to_bits(rng.standard_normal(size=(wl.T, wl.HA, wl.DK)) * sk, wl.dtype)
    kp = to_bits(rng.standard_normal(size=(wl.N, wl.DK)) * sk, wl.dtype)
    vp = to_bits(rng.standard_normal(size=(wl.N, wl.DV)), wl.dtype)
    kl = to_bits(rng.standard_normal(size=(wl.L, wl.DK)) * sk, wl.dtype)
    vl = to_bits(rng.standard_normal(size=(wl.L, wl.DV)), wl.dtype)
    pos = wl.positions
    idx = draw_index_lists(rng, wl.T, wl.N, wl.topk, wl.short_every) if wl.ratio == 0 else \
        np.full((wl.T, 0), -1, dtype=np.int32)
    return {"q": q, "kp": kp, "vp": vp, "kl": kl, "vl": vl, "idx": idx, "pos": pos, "wl": wl}
