"""The timestamped build (libds_indexer_stamps.so: the same sources compiled
with DSI_STAMPS) on the GPU: it computes the same bytes as the product build,
and its phase records are ordered in time.  It is loaded beside the product
library in this process (ctypes keeps the two apart)."""
import ctypes
import dataclasses
import os

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def libs():
    from sparse_attention_kv_ds_amd import indexer
    path = os.path.join(os.path.dirname(indexer.__file__), "libds_indexer_stamps.so")
    if not os.path.exists(path):
        pytest.fail("libds_indexer_stamps.so is not built (build() builds it)")
    st = ctypes.CDLL(path)
    st.ds_indexer_create.argtypes = [ctypes.POINTER(P), I, I, I, I, I, I64, I64]
    st.ds_indexer_score_topk.argtypes = [P, P, P, P, P, I64, I64, I, I, P, P]
    st.ds_indexer_destroy.argtypes = [P]
    st.ds_indexer_stamps_read.argtypes = [I, P, I64]
    st.ds_sparse_attention.argtypes = [P, P, P, P, P, P, P, I64, I64, I64, I, I, I, I, I,
                                       ctypes.c_float, P, P]
    return indexer, st


def stamps(st, unit):
    buf = np.zeros(4096 * 8, dtype=np.uint64)
    assert st.ds_indexer_stamps_read(unit, buf.ctypes.data, buf.nbytes) == 0
    return buf.reshape(4096, 8).astype(np.int64)


def run_stamped(st, d, wl):
    q = torch.from_numpy(d["q"].view(np.int16)).to(DEV)
    k = torch.from_numpy(d["k"].view(np.int16)).to(DEV)
    w = torch.from_numpy(d["w"]).to(DEV)
    pos = torch.from_numpy(d["pos"]).to(DEV)
    out = torch.empty((wl.T, wl.topk), dtype=torch.int32, device=DEV)
    h = P()
    dt = 1 if wl.dtype == "f16" else 2
    assert st.ds_indexer_create(ctypes.byref(h), 0, wl.H, wl.D, dt, wl.topk, wl.T, wl.N) == 0
    try:
        s = torch.cuda.current_stream(DEV).cuda_stream
        assert st.ds_indexer_score_topk(h, q.data_ptr(), k.data_ptr(), w.data_ptr(), pos.data_ptr(),
                                        wl.T, wl.N, wl.ratio, wl.topk, out.data_ptr(), s) == 0
        torch.cuda.synchronize(DEV)
    finally:
        st.ds_indexer_destroy(h)
    return out.cpu().numpy(), (q, k, w, pos)


def test_stamps_build_same_results_and_ordered_phases(libs):
    from sparse_attention_kv_ds_amd import synth
    ix, st = libs
    say("stamps build: prefill8k (every token selects)")
    d = synth.make("prefill8k")
    wl = d["wl"]
    got, (q, k, w, pos) = run_stamped(st, d, wl)
    with ix.Indexer(wl.H, wl.D, wl.dtype, wl.topk, wl.T, wl.N) as h:
        want = h.score_topk(q, k, w, pos, wl.ratio, wl.topk).cpu().numpy()
    assert np.array_equal(got, want)
    r = stamps(st, ix.DS_STAMPS_TOPK)[:wl.T]
    assert (np.diff(r[:, :5], axis=1) >= 0).all(), "top-k phases out of order"
    say("stamps build: decode at 65536 rows")
    d = synth.make("decode1m")
    wl = d["wl"]
    n = 65536
    d = dict(d, k=np.ascontiguousarray(d["k"][:n]), pos=np.array([4 * n - 1], np.int32))
    wl = dataclasses.replace(wl, N=n)
    got, (q, k, w, pos) = run_stamped(st, d, wl)
    with ix.Indexer(wl.H, wl.D, wl.dtype, wl.topk, wl.T, wl.N) as h:
        want = h.score_topk(q, k, w, pos, wl.ratio, wl.topk).cpu().numpy()
    assert np.array_equal(got, want)
    r = stamps(st, ix.DS_STAMPS_DECODE_SCORE)[:n // 512]
    assert (r[:, 1] >= r[:, 0]).all() and (r[:, 2:6].min(axis=1) >= r[:, 1]).all()
    assert (r[:, 6] >= r[:, 2:6].max(axis=1)).all(), "decode phases out of order"
    # (at 65536 rows the 128 partitions' 8-key lists often miss a row of the
    # top 512 and the merge ends with the exact re-stream: entry 5 instead of
    # 4, the other keeping an older launch's value)
    m = stamps(st, ix.DS_STAMPS_MERGE)[0]
    assert m[0] >= r[:, 6].max() and (np.diff(m[:4]) >= 0).all(), "merge phases out of order"
    assert max(m[4], m[5]) >= m[3], "merge end before its exactness check"
