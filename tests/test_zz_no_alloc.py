"""ds_indexer_score_topk_noalloc (no handle, nothing allocated, scratch in one
fixed device array per GPU) against ds_indexer_score_topk on the same inputs:
the outputs must be identical, on two calls in a row with the second smaller
(the array keeps the first call's contents), for the prefill kernels and for
the single-token kernels."""
import numpy as np
import pytest
import torch

from sparse_attention_kv_ds_amd import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


def say(msg):
    print(msg, flush=True)


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from sparse_attention_kv_ds_amd import indexer
    return indexer


def upload(q, k, w, pos):
    return (torch.from_numpy(np.ascontiguousarray(q).view(np.int16)).to(DEV),
            torch.from_numpy(np.ascontiguousarray(k).view(np.int16)).to(DEV),
            torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(DEV),
            torch.from_numpy(np.ascontiguousarray(pos, dtype=np.int32)).to(DEV))


def both(lib, q, k, w, pos, H, D, dtype, ratio, topk):
    """(no-alloc output, handle output) for one problem."""
    T, N = len(pos), k.shape[0]
    tq, tk, tw, tp = upload(q, k, w, pos)
    code = lib.DS_F16 if dtype == "f16" else lib.DS_BF16
    out = torch.full((T, topk), -7, dtype=torch.int32, device=DEV)
    st = lib.ds_indexer_score_topk_noalloc(tq.data_ptr(), tk.data_ptr(), tw.data_ptr(),
                                           tp.data_ptr(), T, N, H, D, code, ratio, topk,
                                           out.data_ptr(), torch.cuda.current_stream(DEV).cuda_stream)
    assert st == lib.DS_OK, lib.ds_indexer_status_str(st)
    torch.cuda.synchronize(DEV)
    got = out.cpu().numpy()
    with lib.Indexer(H, D, dtype, topk, T, N, device=0) as ix:
        want = ix.score_topk(tq, tk, tw, tp, ratio, topk)
        torch.cuda.synchronize(DEV)
    return got, want.cpu().numpy()


def check_same(got, want, where):
    bad = np.nonzero((got != want).any(axis=1))[0]
    assert bad.size == 0, (f"{where}: {bad.size} tokens differ; token {bad[0]} got "
                           f"{got[bad[0]].tolist()[:12]} want {want[bad[0]].tolist()[:12]}")


def test_noalloc_prefill_two_calls(lib):
    """The full 32k chunk (2048 x 8192: exactly the array's 2^24 score entries),
    then a smaller ragged call on other data."""
    say("no-alloc prefill: 2048 tokens x 8192 rows")
    d = synth.make("prefill32k")
    wl = d["wl"]
    got, want = both(lib, d["q"], d["k"], d["w"], d["pos"], wl.H, wl.D, wl.dtype, wl.ratio,
                     wl.topk)
    check_same(got, want, "32k chunk")
    say("no-alloc prefill: 300 tokens x 3000 rows (bf16 gaussian), second call")
    rng = np.random.default_rng(5)
    T, N, H, D = 300, 3000, 64, 128
    q = synth.to_bits(rng.standard_normal((T, H, D)) / np.sqrt(128.0), "bf16")
    k = synth.to_bits(rng.standard_normal((N, D)) / np.sqrt(128.0), "bf16")
    w = rng.random((T, H), dtype=np.float32)
    pos = np.sort(rng.integers(-5, 4 * N + 9, size=T)).astype(np.int32)
    got, want = both(lib, q, k, w, pos, H, D, "bf16", 4, 512)
    check_same(got, want, "second, smaller call")
    assert (got >= -1).all() and (got[:, 0] >= -1).all()


def test_noalloc_decode_two_calls(lib):
    """The 1M-token decode (262144 rows) then a 5000-row decode."""
    say("no-alloc decode: 262144 rows")
    d = synth.make("decode1m")
    wl = d["wl"]
    got, want = both(lib, d["q"], d["k"], d["w"], d["pos"], wl.H, wl.D, wl.dtype, wl.ratio,
                     wl.topk)
    check_same(got, want, "decode1m")
    say("no-alloc decode: 5000 rows, integer inputs, second call")
    rng = np.random.default_rng(6)
    q = synth.to_bits(rng.integers(-4, 5, size=(1, 64, 128)), "f16")
    k = synth.to_bits(rng.integers(-4, 5, size=(5000, 128)), "f16")
    w = np.ldexp(1.0, -rng.integers(0, 4, size=(1, 64))).astype(np.float32)
    got, want = both(lib, q, k, w, np.array([4 * 5000 - 1], np.int32), 64, 128, "f16", 4, 512)
    check_same(got, want, "second, smaller decode")


def test_noalloc_rejects_beyond_its_array(lib):
    """Beyond the fixed array: a clear capacity error, nothing launched, the
    output untouched."""
    q = torch.zeros(2049 * 64 * 128, dtype=torch.int16, device=DEV)
    k = torch.zeros(8193 * 128, dtype=torch.int16, device=DEV)
    w = torch.zeros(2049 * 64, dtype=torch.float32, device=DEV)
    pos = torch.zeros(2049, dtype=torch.int32, device=DEV)
    out = torch.full((2049 * 512,), -7, dtype=torch.int32, device=DEV)
    s = torch.cuda.current_stream(DEV).cuda_stream
    for T, N in ((2049, 8192), (2048, 8193)):
        st = lib.ds_indexer_score_topk_noalloc(q.data_ptr(), k.data_ptr(), w.data_ptr(),
                                               pos.data_ptr(), T, N, 64, 128, lib.DS_F16, 4, 512,
                                               out.data_ptr(), s)
        assert st == lib.DS_ERR_CAPACITY
    torch.cuda.synchronize(DEV)
    assert bool((out == -7).all())
