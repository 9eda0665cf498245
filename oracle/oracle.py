"""ctypes front end of the CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the package smoke check and the
benchmark's CPU-baseline leg are the only callers.  The GPU product path never
imports this module.

The oracle computes, for each query token, the lightning-indexer score of
every causally visible compressed row in double precision, sorts all of them
by (score descending, row ascending), keeps the first min(n_t, topk), and
returns those rows in ascending order padded with -1; the sparse attention of
each token over its local raw rows plus its selected pooled rows; and the
query projection ahead of the indexer (the definitions are written out in
oracle.c, with their sources).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle.c")
LIB = os.path.join(HERE, "liboracle.so")

DTYPES = {"f16": 1, "bf16": 2}
STATUS = {0: "ok", -1: "invalid argument", -2: "non-finite input", -3: "out of memory"}


class OracleError(RuntimeError):
    pass


def build(out: str = LIB, src: str = SRC) -> str:
    """Compile oracle.c into a shared library with the system C compiler."""
    cmd = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-shared", "-fPIC", "-pthread",
           "-o", out, src, "-lm"]
    subprocess.run(cmd, check=True)
    return out


class Oracle:
    """One loaded copy of the oracle library (the tests also load mutated copies)."""

    def __init__(self, path: str = LIB):
        if not os.path.exists(path):
            raise OracleError(f"oracle library {path} is not built; run __graft_entry__.build()")
        self.path = path
        lib = ctypes.CDLL(path)
        lib.oracle_half_to_double.restype = ctypes.c_double
        lib.oracle_half_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_bf16_to_double.restype = ctypes.c_double
        lib.oracle_bf16_to_double.argtypes = [ctypes.c_uint16]
        lib.oracle_visible_rows.restype = ctypes.c_int64
        lib.oracle_visible_rows.argtypes = [ctypes.c_int64, ctypes.c_int64, ctypes.c_int64]
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        I = ctypes.c_int
        lib.oracle_score_topk.restype = I
        lib.oracle_score_topk.argtypes = [P, P, P, P, I64, I64, I, I, I, I, I, P, I64, P, P, I]
        lib.oracle_sparse_attention.restype = I
        lib.oracle_sparse_attention.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I, I, I, I, I,
                                                ctypes.c_double, I, P, I64, P, I]
        lib.oracle_double_to_half.restype = ctypes.c_uint16
        lib.oracle_double_to_half.argtypes = [ctypes.c_double]
        lib.oracle_double_to_bf16.restype = ctypes.c_uint16
        lib.oracle_double_to_bf16.argtypes = [ctypes.c_double]
        lib.oracle_project_q.restype = I
        lib.oracle_project_q.argtypes = [P, P, I64, I64, I64, I, P, I]
        lib.oracle_sparse_attention_all.restype = I
        lib.oracle_sparse_attention_all.argtypes = [P, P, P, P, P, P, I64, I64, I64, I, I, I, I, I,
                                                    ctypes.c_double, I, P, I64, P, I]
        self.lib = lib

    def half_to_double(self, bits: int) -> float:
        return self.lib.oracle_half_to_double(int(bits))

    def bf16_to_double(self, bits: int) -> float:
        return self.lib.oracle_bf16_to_double(int(bits))

    def visible_rows(self, pos: int, ratio: int, n_rows: int) -> int:
        return self.lib.oracle_visible_rows(int(pos), int(ratio), int(n_rows))

    def score_topk(self, q_bits, k_bits, w, pos, *, H: int, D: int, dtype: str, ratio: int,
                   topk: int, tokens=None, want_scores: bool = False, threads: int = 1):
        """Run the oracle on host arrays.

        q_bits  uint16 [T, H, D] (raw fp16/bf16 bits)
        k_bits  uint16 [N, D]
        w       float32 [T, H]
        pos     int32 [T]
        tokens  optional int64 list of token indices to compute (default: all)

        Returns out int32 [n_out, topk] (and scores float64 [n_out, N] with -inf
        where a row is not visible, when want_scores).
        """
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        k_bits = np.ascontiguousarray(k_bits, dtype=np.uint16)
        w = np.ascontiguousarray(w, dtype=np.float32)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        T = int(pos.shape[0])
        N = int(k_bits.shape[0]) if k_bits.ndim == 2 else 0
        if q_bits.size != T * H * D or w.size != T * H or (N and k_bits.shape[1] != D):
            raise OracleError("oracle: inconsistent shapes")
        if tokens is None:
            tok = None
            n_out = T
        else:
            tok = np.ascontiguousarray(tokens, dtype=np.int64)
            n_out = int(tok.shape[0])
        out = np.empty((n_out, topk), dtype=np.int32)
        scores = np.empty((n_out, N), dtype=np.float64) if want_scores else None

        def ptr(a):
            return None if a is None else a.ctypes.data_as(ctypes.c_void_p)

        st = self.lib.oracle_score_topk(ptr(q_bits), ptr(k_bits) if N else None, ptr(w), ptr(pos),
                                        T, N, H, D, DTYPES[dtype], ratio, topk, ptr(tok), n_out,
                                        ptr(out), ptr(scores), int(threads))
        if st != 0:
            raise OracleError(f"oracle_score_topk: {STATUS.get(st, st)}")
        return (out, scores) if want_scores else out


    def sparse_attention(self, q_bits, kp_bits, vp_bits, kl_bits, vl_bits, idx, pos, *,
                         dtype: str, window: int, scale: float, tokens=None, threads: int = 1):
        """Attention of each token's heads over its local window of raw rows plus
        the pooled rows its index list names (definition in oracle.c).

        q_bits  uint16 [T, HA, DK]; kp_bits [N, DK], vp_bits [N, DV] (pooled rows);
        kl_bits [L, DK], vl_bits [L, DV] (raw rows by absolute position);
        idx     int32 [T, topk] (-1 = padding); pos int32 [T].
        Returns float64 [n_out, HA, DV].
        """
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        kp_bits = np.ascontiguousarray(kp_bits, dtype=np.uint16)
        vp_bits = np.ascontiguousarray(vp_bits, dtype=np.uint16)
        kl_bits = np.ascontiguousarray(kl_bits, dtype=np.uint16)
        vl_bits = np.ascontiguousarray(vl_bits, dtype=np.uint16)
        idx = np.ascontiguousarray(idx, dtype=np.int32)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        T, HA, DK = q_bits.shape
        N, L = kp_bits.shape[0], kl_bits.shape[0]
        DV = vp_bits.shape[1] if vp_bits.ndim == 2 else vl_bits.shape[1]
        topk = idx.shape[1] if idx.ndim == 2 else 0
        if (pos.shape != (T,) or (N and (kp_bits.shape[1] != DK or vp_bits.shape != (N, DV)))
                or (L and (kl_bits.shape[1] != DK or vl_bits.shape != (L, DV)))
                or (topk and idx.shape[0] != T)):
            raise OracleError("oracle: inconsistent shapes")
        if tokens is None:
            tok, n_out = None, T
        else:
            tok = np.ascontiguousarray(tokens, dtype=np.int64)
            n_out = int(tok.shape[0])
        out = np.empty((n_out, HA, DV), dtype=np.float64)

        def ptr(a):
            return None if a is None or a.size == 0 else a.ctypes.data_as(ctypes.c_void_p)

        st = self.lib.oracle_sparse_attention(ptr(q_bits), ptr(kp_bits), ptr(vp_bits), ptr(kl_bits),
                                              ptr(vl_bits), ptr(idx), ptr(pos), T, N, L, HA, DK, DV,
                                              topk, int(window), float(scale), DTYPES[dtype], ptr(tok),
                                              n_out, ptr(out), int(threads))
        if st != 0:
            raise OracleError(f"oracle_sparse_attention: {STATUS.get(st, st)}")
        return out


    def double_to_half(self, v: float) -> int:
        return self.lib.oracle_double_to_half(float(v))

    def double_to_bf16(self, v: float) -> int:
        return self.lib.oracle_double_to_bf16(float(v))

    def project_q(self, x_bits, wq_bits, *, dtype: str, threads: int = 1):
        """The query projection: q = round_dtype(x . wq^T) (definition in oracle.c).
        x_bits uint16 [T, d_in], wq_bits uint16 [O, d_in]; returns uint16 [T, O]."""
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        wq_bits = np.ascontiguousarray(wq_bits, dtype=np.uint16)
        T, din = x_bits.shape
        O = wq_bits.shape[0]
        if wq_bits.shape[1] != din:
            raise OracleError("oracle: inconsistent shapes")
        q = np.empty((T, O), dtype=np.uint16)
        st = self.lib.oracle_project_q(x_bits.ctypes.data_as(ctypes.c_void_p),
                                       wq_bits.ctypes.data_as(ctypes.c_void_p), T, din, O,
                                       DTYPES[dtype], q.ctypes.data_as(ctypes.c_void_p),
                                       int(threads))
        if st != 0:
            raise OracleError(f"oracle_project_q: {STATUS.get(st, st)}")
        return q

    def project_score_topk(self, x_bits, wq_bits, k_bits, w, pos, *, H: int, D: int, dtype: str,
                           ratio: int, topk: int, tokens=None, want_scores: bool = False,
                           threads: int = 1):
        """The projection followed by the indexer: q = project_q(x, wq) reshaped to
        [T, H, D], then score_topk on it (tokens: the rows of x projected and scored)."""
        x_bits = np.ascontiguousarray(x_bits, dtype=np.uint16)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        w = np.ascontiguousarray(w, dtype=np.float32)
        if tokens is not None:
            tok = np.ascontiguousarray(tokens, dtype=np.int64)
            x_bits, pos, w = x_bits[tok], pos[tok], w[tok]
        q = self.project_q(x_bits, wq_bits, dtype=dtype, threads=threads)
        return self.score_topk(q.reshape(len(pos), H, D), k_bits, w, pos, H=H, D=D, dtype=dtype,
                               ratio=ratio, topk=topk, want_scores=want_scores, threads=threads)

    def sparse_attention_all(self, q_bits, kp_bits, vp_bits, kl_bits, vl_bits, pos, *, dtype: str,
                             ratio: int, window: int, scale: float, tokens=None, threads: int = 1):
        """The all-visible form: each token attends to its local window plus
        every pooled row it can see, rows 0 .. n_t-1 (definition in oracle.c).
        Arrays as in sparse_attention, without idx.  Returns float64 [n_out, HA, DV]."""
        q_bits = np.ascontiguousarray(q_bits, dtype=np.uint16)
        kp_bits = np.ascontiguousarray(kp_bits, dtype=np.uint16)
        vp_bits = np.ascontiguousarray(vp_bits, dtype=np.uint16)
        kl_bits = np.ascontiguousarray(kl_bits, dtype=np.uint16)
        vl_bits = np.ascontiguousarray(vl_bits, dtype=np.uint16)
        pos = np.ascontiguousarray(pos, dtype=np.int32)
        T, HA, DK = q_bits.shape
        N, L = kp_bits.shape[0], kl_bits.shape[0]
        DV = vp_bits.shape[1] if vp_bits.ndim == 2 else vl_bits.shape[1]
        if (pos.shape != (T,) or (N and (kp_bits.shape[1] != DK or vp_bits.shape != (N, DV)))
                or (L and (kl_bits.shape[1] != DK or vl_bits.shape != (L, DV)))):
            raise OracleError("oracle: inconsistent shapes")
        if tokens is None:
            tok, n_out = None, T
        else:
            tok = np.ascontiguousarray(tokens, dtype=np.int64)
            n_out = int(tok.shape[0])
        out = np.empty((n_out, HA, DV), dtype=np.float64)

        def ptr(a):
            return None if a is None or a.size == 0 else a.ctypes.data_as(ctypes.c_void_p)

        st = self.lib.oracle_sparse_attention_all(ptr(q_bits), ptr(kp_bits), ptr(vp_bits),
                                                  ptr(kl_bits), ptr(vl_bits), ptr(pos), T, N, L,
                                                  HA, DK, DV, int(ratio), int(window), float(scale),
                                                  DTYPES[dtype], ptr(tok), n_out, ptr(out),
                                                  int(threads))
        if st != 0:
            raise OracleError(f"oracle_sparse_attention_all: {STATUS.get(st, st)}")
        return out


_default = None


def load() -> Oracle:
    """The oracle built from oracle.c (loaded once per process)."""
    global _default
    if _default is None:
        _default = Oracle(LIB)
    return _default
