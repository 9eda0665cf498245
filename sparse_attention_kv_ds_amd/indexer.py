"""Thin Python binding of libds_indexer.so (the C ABI in include/ds_indexer.h).

Argument marshalling only: every step of the indexer (scoring, skip path,
selection) runs in the library's HIP kernels.  torch supplies device memory
and the current stream.  There is no fallback: if the library is not built,
importing this module raises.

Functions with the C names take raw integers (device pointers, a stream
handle); the ``Indexer`` class wraps them for torch tensors.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
# DS_INDEXER_LIB selects another build of the same library (the timestamped
# libds_indexer_stamps.so for phase breakdowns); default: the product build
LIB_PATH = os.environ.get("DS_INDEXER_LIB") or os.path.join(HERE, "libds_indexer.so")

DS_F16 = 1
DS_BF16 = 2
DS_OK = 0
DS_ERR_INVALID_ARG = -1
DS_ERR_UNSUPPORTED = -2
DS_ERR_CAPACITY = -3
DS_ERR_HIP = -4
DS_ERR_OOM = -5
DS_KERNEL_SCORE = 0
DS_KERNEL_SELECT = 1
DS_KERNEL_DECODE_SCORE = 2
DS_KERNEL_DECODE_SELECT = 3
DS_KERNEL_PROJECT = 4
DS_KERNEL_CLASSES = 5
KERNEL_CLASS_NAMES = ("score", "select", "decode_score", "decode_select", "project")

EXPORTS = ("ds_indexer_create", "ds_indexer_score_topk", "ds_indexer_destroy",
           "ds_indexer_scores", "ds_indexer_status_str", "ds_indexer_timing",
           "ds_indexer_timing_read", "ds_sparse_attention", "ds_sparse_attention_all",
           "ds_indexer_score_topk_batch", "ds_indexer_project_q", "ds_indexer_project_score_topk",
           "ds_indexer_score_topk_noalloc", "ds_indexer_stamps_read",
           "ds_indexed_sparse_attention")
DS_STAMPS_DECODE_SCORE = 0
DS_STAMPS_TOPK = 1
DS_STAMPS_MERGE = 2
DS_STAMPS_ATTENTION = 3


class IndexerError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        super().__init__(f"{what}: {ds_indexer_status_str(status)} ({status})" if what
                         else ds_indexer_status_str(status))


def _load() -> ctypes.CDLL:
    # torch first: its HIP runtime must be the one the library binds to, so that
    # torch's device pointers and stream handles are valid in the library's calls
    # (loaded the other way round, the process can end up with two runtimes)
    import torch  # noqa: F401
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built (run __graft_entry__.build()); "
                          "the indexer has no non-HIP implementation")
    lib = ctypes.CDLL(LIB_PATH)
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    lib.ds_indexer_create.restype = I
    lib.ds_indexer_create.argtypes = [ctypes.POINTER(P), I, I, I, I, I, I64, I64]
    lib.ds_indexer_score_topk.restype = I
    lib.ds_indexer_score_topk.argtypes = [P, P, P, P, P, I64, I64, I, I, P, P]
    lib.ds_indexer_project_q.restype = I
    lib.ds_indexer_project_q.argtypes = [P, P, P, I64, I64, P, P]
    lib.ds_indexer_project_score_topk.restype = I
    lib.ds_indexer_project_score_topk.argtypes = [P, P, P, P, P, P, I64, I64, I64, I, I, P, P]
    lib.ds_indexer_score_topk_noalloc.restype = I
    lib.ds_indexer_score_topk_noalloc.argtypes = [P, P, P, P, I64, I64, I, I, I, I, I, P, P]
    lib.ds_indexer_score_topk_batch.restype = I
    lib.ds_indexer_score_topk_batch.argtypes = [P, P, P, P, P, I64, I64, I, I, P, P]
    lib.ds_indexer_destroy.restype = None
    lib.ds_indexer_destroy.argtypes = [P]
    lib.ds_indexer_scores.restype = I
    lib.ds_indexer_scores.argtypes = [P, P, P, P, P, I64, I64, I, P, P]
    lib.ds_indexer_status_str.restype = ctypes.c_char_p
    lib.ds_indexer_status_str.argtypes = [I]
    lib.ds_indexer_timing.restype = I
    lib.ds_indexer_timing.argtypes = [P, I]
    lib.ds_indexer_timing_read.restype = I
    lib.ds_indexer_timing_read.argtypes = [P, P, P]
    lib.ds_sparse_attention.restype = I
    lib.ds_sparse_attention.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I, I, I, I, I,
                                        ctypes.c_float, P, P]
    lib.ds_indexer_stamps_read.restype = I
    lib.ds_indexer_stamps_read.argtypes = [I, P, I64]
    lib.ds_sparse_attention_all.restype = I
    lib.ds_sparse_attention_all.argtypes = [P, P, P, P, P, P, I64, I64, I64, I, I, I, I, I,
                                            ctypes.c_float, P, P]
    lib.ds_indexed_sparse_attention.restype = I
    lib.ds_indexed_sparse_attention.argtypes = [P, P, P, P, P, I64, I64, I, I, P, P, P, P, I64,
                                                P, P, I64, I, I, I, ctypes.c_float, P, P]
    return lib


_lib = _load()


def library() -> ctypes.CDLL:
    return _lib


# --- the C entry points, same names --------------------------------------------------

def ds_indexer_create(device: int, n_heads: int, head_dim: int, dtype: int, max_topk: int,
                      max_tokens: int, max_rows: int):
    """Returns (status, handle); handle is None unless status == DS_OK."""
    h = ctypes.c_void_p()
    st = _lib.ds_indexer_create(ctypes.byref(h), device, n_heads, head_dim, dtype, max_topk,
                                max_tokens, max_rows)
    return st, (h.value if st == DS_OK else None)


def ds_indexer_score_topk(handle, q, k, w, pos, T, N, ratio, topk, out, stream) -> int:
    return _lib.ds_indexer_score_topk(handle, q, k, w, pos, T, N, ratio, topk, out, stream)


def ds_indexer_stamps_read(unit, host, nbytes) -> int:
    return _lib.ds_indexer_stamps_read(unit, host, nbytes)


def ds_indexer_score_topk_noalloc(q, k, w, pos, T, N, n_heads, head_dim, dtype, ratio, topk,
                                  out, stream) -> int:
    return _lib.ds_indexer_score_topk_noalloc(q, k, w, pos, T, N, n_heads, head_dim, dtype,
                                              ratio, topk, out, stream)


def ds_indexer_project_q(handle, x, wq, T, d_in, q, stream) -> int:
    return _lib.ds_indexer_project_q(handle, x, wq, T, d_in, q, stream)


def ds_indexer_project_score_topk(handle, x, wq, k, w, pos, T, N, d_in, ratio, topk, out,
                                  stream) -> int:
    return _lib.ds_indexer_project_score_topk(handle, x, wq, k, w, pos, T, N, d_in, ratio, topk,
                                              out, stream)


def ds_indexer_score_topk_batch(handle, q, k, w, pos, B, N, ratio, topk, out, stream) -> int:
    return _lib.ds_indexer_score_topk_batch(handle, q, k, w, pos, B, N, ratio, topk, out, stream)


def ds_indexer_destroy(handle) -> None:
    _lib.ds_indexer_destroy(handle)


def ds_indexer_scores(handle, q, k, w, pos, T, N, ratio, scores, stream) -> int:
    return _lib.ds_indexer_scores(handle, q, k, w, pos, T, N, ratio, scores, stream)


def ds_indexer_status_str(status: int) -> str:
    return _lib.ds_indexer_status_str(status).decode()


def ds_indexer_timing(handle, enable: int) -> int:
    return _lib.ds_indexer_timing(handle, enable)


def ds_indexer_timing_read(handle):
    """Returns (status, ms[4], launches[4]) per kernel class."""
    ms = (ctypes.c_double * DS_KERNEL_CLASSES)()
    n = (ctypes.c_int64 * DS_KERNEL_CLASSES)()
    st = _lib.ds_indexer_timing_read(handle, ms, n)
    return st, list(ms), list(n)


def ds_sparse_attention(q, k_pool, v_pool, k_local, v_local, idx, pos, T, N, L, n_heads,
                        head_dim, dtype, topk, window, scale, out, stream) -> int:
    return _lib.ds_sparse_attention(q, k_pool, v_pool, k_local, v_local, idx, pos, T, N, L,
                                    n_heads, head_dim, dtype, topk, window, scale, out, stream)


def ds_indexed_sparse_attention(handle, q_index, k_index, w, pos, T, n_index_rows, ratio, topk,
                                idx, q, k_pool, v_pool, n_pool_rows, k_local, v_local, L,
                                n_heads, head_dim, window, scale, out, stream) -> int:
    return _lib.ds_indexed_sparse_attention(handle, q_index, k_index, w, pos, T, n_index_rows,
                                            ratio, topk, idx, q, k_pool, v_pool, n_pool_rows,
                                            k_local, v_local, L, n_heads, head_dim, window, scale,
                                            out, stream)


# --- torch-facing wrapper -------------------------------------------------------------

def _dtype_code(dtype) -> int:
    import torch
    if dtype in ("f16", torch.float16, DS_F16):
        return DS_F16
    if dtype in ("bf16", torch.bfloat16, DS_BF16):
        return DS_BF16
    raise ValueError(f"unsupported dtype {dtype!r}")


class Indexer:
    """One library handle on one device.

    q: [T, H, D] fp16/bf16 (or the raw bits as int16/uint16), k: [N, D] same,
    w: [T, H] float32, pos: [T] int32, all contiguous on the handle's device.
    Work is enqueued on torch's current stream of that device.
    """

    def __init__(self, n_heads: int, head_dim: int, dtype, max_topk: int, max_tokens: int,
                 max_rows: int, device: int = 0):
        self.H, self.D = n_heads, head_dim
        self.dtype = _dtype_code(dtype)
        self.device = device
        st, h = ds_indexer_create(device, n_heads, head_dim, self.dtype, max_topk, max_tokens,
                                  max_rows)
        if st != DS_OK:
            raise IndexerError(st, "ds_indexer_create")
        self.handle = h

    def close(self) -> None:
        if self.handle is not None:
            ds_indexer_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()

    def _check(self, q, k, w, pos):
        import torch
        dev = torch.device("cuda", self.device)
        T = pos.shape[0]
        N = k.shape[0]
        elem = (torch.float16, torch.bfloat16, torch.int16, torch.uint16)
        for name, t in (("q", q), ("k", k), ("w", w), ("pos", pos)):
            if t.device != dev or not t.is_contiguous():
                raise ValueError(f"{name} must be a contiguous tensor on {dev}")
        if q.dtype not in elem or k.dtype not in elem or q.element_size() != 2:
            raise ValueError("q and k must hold 16-bit elements")
        if tuple(q.shape) != (T, self.H, self.D) or tuple(k.shape[1:]) != (self.D,):
            raise ValueError(f"shapes: q {tuple(q.shape)}, k {tuple(k.shape)}")
        if w.dtype != torch.float32 or tuple(w.shape) != (T, self.H):
            raise ValueError("w must be float32 [T, H]")
        if pos.dtype != torch.int32:
            raise ValueError("pos must be int32 [T]")
        return T, N, torch.cuda.current_stream(dev).cuda_stream

    def score_topk(self, q, k, w, pos, ratio: int, topk: int, out=None):
        import torch
        T, N, stream = self._check(q, k, w, pos)
        if out is None:
            out = torch.empty((T, topk), dtype=torch.int32, device=q.device)
        elif (out.dtype != torch.int32 or tuple(out.shape) != (T, topk) or not out.is_contiguous()
              or out.device != q.device):
            raise ValueError("out must be a contiguous int32 [T, topk] tensor on q's device")
        st = ds_indexer_score_topk(self.handle, q.data_ptr(), k.data_ptr(), w.data_ptr(),
                                   pos.data_ptr(), T, N, ratio, topk, out.data_ptr(), stream)
        if st != DS_OK:
            raise IndexerError(st, "ds_indexer_score_topk")
        return out

    def _check_proj(self, x, wq):
        import torch
        dev = torch.device("cuda", self.device)
        for name, t in (("x", x), ("wq", wq)):
            if t.device != dev or not t.is_contiguous() or t.element_size() != 2 or t.dim() != 2:
                raise ValueError(f"{name} must be a contiguous 2-D 16-bit tensor on {dev}")
        if wq.shape[0] != self.H * self.D or wq.shape[1] != x.shape[1]:
            raise ValueError(f"wq must be [H*D, d_in]; got {tuple(wq.shape)}, x {tuple(x.shape)}")
        return x.shape[0], x.shape[1], torch.cuda.current_stream(dev).cuda_stream

    def project_q(self, x, wq, out=None):
        """The query projection (ds_indexer_project_q): x [T, d_in], wq [H*D, d_in]
        (16-bit, the handle's dtype); returns q [T, H, D] as int16 bits."""
        import torch
        T, din, stream = self._check_proj(x, wq)
        if out is None:
            out = torch.empty((T, self.H, self.D), dtype=torch.int16, device=x.device)
        st = ds_indexer_project_q(self.handle, x.data_ptr(), wq.data_ptr(), T, din,
                                  out.data_ptr(), stream)
        if st != DS_OK:
            raise IndexerError(st, "ds_indexer_project_q")
        return out

    def project_score_topk(self, x, wq, k, w, pos, ratio: int, topk: int, out=None):
        """Projection then score + top-k in one call (ds_indexer_project_score_topk)."""
        import torch
        T, din, stream = self._check_proj(x, wq)
        if out is None:
            out = torch.empty((T, topk), dtype=torch.int32, device=x.device)
        st = ds_indexer_project_score_topk(self.handle, x.data_ptr(), wq.data_ptr(), k.data_ptr(),
                                           w.data_ptr(), pos.data_ptr(), T, k.shape[0], din,
                                           ratio, topk, out.data_ptr(), stream)
        if st != DS_OK:
            raise IndexerError(st, "ds_indexer_project_score_topk")
        return out

    def score_topk_batch(self, q, k, w, pos, ratio: int, topk: int, out=None):
        """Batched decode (ds_indexer_score_topk_batch): q [B, H, D], k [B, N, D],
        w [B, H], pos [B]; returns out [B, topk]."""
        import torch
        dev = torch.device("cuda", self.device)
        B = pos.shape[0]
        if k.dim() != 3 or k.shape[0] != B:
            raise ValueError(f"k must be [B, N, D]; got {tuple(k.shape)}")
        N = k.shape[1]
        _, _, stream = self._check(q, k[0] if B else k.reshape(0, self.D), w, pos)
        if not k.is_contiguous() or k.device != dev:
            raise ValueError(f"k must be a contiguous tensor on {dev}")
        if out is None:
            out = torch.empty((B, topk), dtype=torch.int32, device=dev)
        elif (out.dtype != torch.int32 or tuple(out.shape) != (B, topk) or not out.is_contiguous()
              or out.device != dev):
            raise ValueError("out must be a contiguous int32 [B, topk] tensor on the device")
        st = ds_indexer_score_topk_batch(self.handle, q.data_ptr(), k.data_ptr(), w.data_ptr(),
                                         pos.data_ptr(), B, N, ratio, topk, out.data_ptr(), stream)
        if st != DS_OK:
            raise IndexerError(st, "ds_indexer_score_topk_batch")
        return out

    def indexed_sparse_attention(self, q_index, k_index, w, pos, ratio: int, topk: int, q,
                                 k_pool, v_pool, k_local, v_local, *, window: int, scale: float,
                                 idx=None, out=None):
        """The selection and the attention over it in one call
        (ds_indexed_sparse_attention): q_index, k_index, w, pos as score_topk;
        q, k_pool, v_pool, k_local, v_local as sparse_attention, in the
        handle's dtype.  k_index and k_pool must hold the same number of rows
        (the library refuses the call otherwise).  Returns (idx [T, topk] int32,
        out [T, HA, D] float32)."""
        import torch
        T, N, stream = self._check(q_index, k_index, w, pos)
        if idx is None:
            idx = torch.empty((T, topk), dtype=torch.int32, device=q_index.device)
        elif (idx.dtype != torch.int32 or tuple(idx.shape) != (T, topk) or not idx.is_contiguous()
              or idx.device != q_index.device):
            raise ValueError("idx must be a contiguous int32 [T, topk] tensor on q's device")
        _, HA, D, _, out, _ = _attention_args(q, k_pool, v_pool, k_local, v_local, idx, pos,
                                              self.dtype, out)
        st = ds_indexed_sparse_attention(
            self.handle, q_index.data_ptr(), _ptr(k_index), w.data_ptr(), pos.data_ptr(), T, N,
            ratio, topk, idx.data_ptr(), _ptr(q), _ptr(k_pool), _ptr(v_pool), k_pool.shape[0],
            _ptr(k_local), _ptr(v_local), k_local.shape[0], HA, D, window, float(scale),
            out.data_ptr(), stream)
        if st != DS_OK:
            raise IndexerError(st, "ds_indexed_sparse_attention")
        return idx, out

    def timing(self, enable: bool) -> None:
        st = ds_indexer_timing(self.handle, 1 if enable else 0)
        if st != DS_OK:
            raise IndexerError(st, "ds_indexer_timing")

    def timing_read(self):
        """{class name: (total ms, launches)} since the last read."""
        st, ms, n = ds_indexer_timing_read(self.handle)
        if st != DS_OK:
            raise IndexerError(st, "ds_indexer_timing_read")
        return {name: (ms[i], n[i]) for i, name in enumerate(KERNEL_CLASS_NAMES)}

    def scores(self, q, k, w, pos, ratio: int, out=None):
        import torch
        T, N, stream = self._check(q, k, w, pos)
        if out is None:
            out = torch.empty((T, N), dtype=torch.float32, device=q.device)
        st = ds_indexer_scores(self.handle, q.data_ptr(), k.data_ptr(), w.data_ptr(),
                               pos.data_ptr(), T, N, ratio, out.data_ptr(), stream)
        if st != DS_OK:
            raise IndexerError(st, "ds_indexer_scores")
        return out


def ds_sparse_attention_all(q, k_pool, v_pool, k_local, v_local, pos, T, N, L, n_heads, head_dim,
                            dtype, ratio, window, scale, out, stream) -> int:
    return _lib.ds_sparse_attention_all(q, k_pool, v_pool, k_local, v_local, pos, T, N, L, n_heads,
                                        head_dim, dtype, ratio, window, scale, out, stream)


def _attention_args(q, k_pool, v_pool, k_local, v_local, idx, pos, dtype, out):
    import torch
    dev = q.device
    T, HA, D = q.shape
    if dtype is None:
        dtype = q.dtype
    code = _dtype_code(dtype)
    tensors = [("q", q), ("k_pool", k_pool), ("v_pool", v_pool), ("k_local", k_local),
               ("v_local", v_local), ("pos", pos)] + ([("idx", idx)] if idx is not None else [])
    for name, t_ in tensors:
        if t_.device != dev or not t_.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor on {dev}")
    for name, t_ in (("k_pool", k_pool), ("v_pool", v_pool), ("k_local", k_local),
                     ("v_local", v_local)):
        if t_.element_size() != 2 or (t_.numel() and tuple(t_.shape[1:]) != (D,)):
            raise ValueError(f"{name} must be [rows, {D}] with 16-bit elements")
    if pos.dtype != torch.int32 or tuple(pos.shape) != (T,) or (
            idx is not None and idx.dtype != torch.int32):
        raise ValueError("idx [T, topk] and pos [T] must be int32")
    if out is None:
        out = torch.empty((T, HA, D), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev).cuda_stream
    return T, HA, D, code, out, stream


def _ptr(t_):
    return t_.data_ptr() if t_.numel() else None


def sparse_attention_all(q, k_pool, v_pool, k_local, v_local, pos, *, ratio: int, window: int,
                         scale: float, dtype=None, out=None):
    """Attention of each token's heads over its local raw rows plus every pooled
    row it can see (ds_sparse_attention_all); arguments as sparse_attention,
    with the compression ratio instead of an index list."""
    T, HA, D, code, out, stream = _attention_args(q, k_pool, v_pool, k_local, v_local, None, pos,
                                                  dtype, out)
    st = ds_sparse_attention_all(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_local),
                                 _ptr(v_local), pos.data_ptr(), T, k_pool.shape[0],
                                 k_local.shape[0], HA, D, code, int(ratio), window, float(scale),
                                 out.data_ptr(), stream)
    if st != DS_OK:
        raise IndexerError(st, "ds_sparse_attention_all")
    return out


def sparse_attention(q, k_pool, v_pool, k_local, v_local, idx, pos, *, window: int,
                     scale: float, dtype=None, out=None):
    """Attention of each token's heads over its local raw rows plus the pooled
    rows listed in idx (ds_sparse_attention).  q [T, HA, D], k_pool/v_pool
    [N, D], k_local/v_local [L, D] (fp16/bf16 or their raw bits), idx [T, topk]
    int32, pos [T] int32, all contiguous on one device; returns out [T, HA, D]
    float32.  Work is enqueued on torch's current stream of that device."""
    T, HA, D, code, out, stream = _attention_args(q, k_pool, v_pool, k_local, v_local, idx, pos,
                                                  dtype, out)
    topk = idx.shape[1] if idx.dim() == 2 else 0
    st = ds_sparse_attention(_ptr(q), _ptr(k_pool), _ptr(v_pool), _ptr(k_local), _ptr(v_local),
                             _ptr(idx), pos.data_ptr(), T, k_pool.shape[0], k_local.shape[0], HA,
                             D, code, topk, window, float(scale), out.data_ptr(), stream)
    if st != DS_OK:
        raise IndexerError(st, "ds_sparse_attention")
    return out
