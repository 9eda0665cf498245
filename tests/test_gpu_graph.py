"""The entry points under HIP graph capture.  A call enqueues kernels only (no
allocation, copy, memset or synchronisation on the way), so a captured call
replays to the eager result.  Each graph is replayed three times; before every
replay the output is overwritten and other eager work runs, with
synchronisations in between, and every replay must equal the eager call bit
for bit (the kernels are deterministic)."""
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


def bits(a):
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV)


def dev32(a, dtype):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=dtype)).to(DEV)


def replays_match(call, out, fill, label):
    """Eager result of call() (which writes out), then the same call captured
    and replayed three times, each replay checked against the eager result."""
    out.fill_(fill)
    call()
    torch.cuda.synchronize(DEV)
    want = out.cpu().clone()
    # a first call on a side stream before the capture, as torch advises
    side = torch.cuda.Stream(DEV)
    side.wait_stream(torch.cuda.current_stream(DEV))
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream(DEV).wait_stream(side)
    torch.cuda.synchronize(DEV)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    torch.cuda.synchronize(DEV)
    junk = torch.empty(1 << 22, dtype=torch.float32, device=DEV)
    for r in range(3):
        out.fill_(fill)
        junk.normal_()
        s = float(junk.sum())  # other eager work, synchronised
        assert np.isfinite(s)
        torch.cuda.synchronize(DEV)
        g.replay()
        torch.cuda.synchronize(DEV)
        got = out.cpu()
        assert torch.equal(got, want), f"{label}: replay {r} differs from the eager call"
    say(f"{label}: three replays equal the eager call")
    return want


def test_prefill_score_topk_in_a_graph(lib):
    """The 8k chunk (2048 tokens x 2048 rows, the prefill scorer and top-k)."""
    d = synth.make("prefill8k")
    wl = d["wl"]
    q, k = bits(d["q"]), bits(d["k"])
    w, pos = dev32(d["w"], np.float32), dev32(d["pos"], np.int32)
    out = torch.empty((wl.T, wl.topk), dtype=torch.int32, device=DEV)
    with lib.Indexer(wl.H, wl.D, wl.dtype, wl.topk, wl.T, wl.N, device=0) as ix:
        want = replays_match(lambda: ix.score_topk(q, k, w, pos, wl.ratio, wl.topk, out=out),
                             out, -7, "prefill8k")
    assert (want >= -1).all()


def test_decode_score_topk_in_a_graph(lib):
    """One token over 40000 rows (the decode scorer with its partition lists,
    then the merge)."""
    rng = np.random.default_rng(11)
    N, H, D, topk = 40000, 64, 128, 512
    q = bits(synth.to_bits(rng.standard_normal((1, H, D)) / np.sqrt(128.0), "f16"))
    k = bits(synth.to_bits(rng.standard_normal((N, D)) / np.sqrt(128.0), "f16"))
    w = dev32(rng.random((1, H), dtype=np.float32), np.float32)
    pos = dev32([4 * N - 1], np.int32)
    out = torch.empty((1, topk), dtype=torch.int32, device=DEV)
    with lib.Indexer(H, D, "f16", topk, 1, N, device=0) as ix:
        want = replays_match(lambda: ix.score_topk(q, k, w, pos, 4, topk, out=out), out, -7,
                             "decode, 40000 rows")
    row = want[0].numpy()
    assert (np.diff(row) > 0).all() and row[0] >= 0 and row[-1] < N


def test_noalloc_entry_in_a_graph(lib):
    """The allocation-free entry point (no handle), on the 8k chunk."""
    d = synth.make("prefill8k")
    wl = d["wl"]
    q, k = bits(d["q"]), bits(d["k"])
    w, pos = dev32(d["w"], np.float32), dev32(d["pos"], np.int32)
    out = torch.empty((wl.T, wl.topk), dtype=torch.int32, device=DEV)
    code = lib.DS_F16 if wl.dtype == "f16" else lib.DS_BF16

    def call():
        st = lib.ds_indexer_score_topk_noalloc(
            q.data_ptr(), k.data_ptr(), w.data_ptr(), pos.data_ptr(), wl.T, wl.N, wl.H, wl.D,
            code, wl.ratio, wl.topk, out.data_ptr(), torch.cuda.current_stream(DEV).cuda_stream)
        assert st == lib.DS_OK, lib.ds_indexer_status_str(st)

    replays_match(call, out, -7, "no-alloc prefill8k")


def test_sparse_attention_in_a_graph(lib):
    """The sparse attention over listed pooled rows (300 tokens, 64 heads of 128)."""
    rng = np.random.default_rng(12)
    T, N, L, HA, D, topk, window = 300, 4000, 4000, 64, 128, 512, 128

    def g16(*shape):
        return bits(synth.to_bits(rng.standard_normal(shape) / np.sqrt(128.0), "bf16"))

    q, kp, vp, kl, vl = g16(T, HA, D), g16(N, D), g16(N, D), g16(L, D), g16(L, D)
    idx_np = rng.integers(0, N, size=(T, topk)).astype(np.int32)
    idx_np[:, -20:] = -1  # empty slots
    idx = dev32(idx_np, np.int32)
    pos = dev32(np.sort(rng.integers(3000, L, size=T)), np.int32)
    out = torch.empty((T, HA, D), dtype=torch.float32, device=DEV)
    want = replays_match(
        lambda: lib.sparse_attention(q, kp, vp, kl, vl, idx, pos, window=window,
                                     scale=1.0 / np.sqrt(D), dtype="bf16", out=out),
        out, float("nan"), "sparse attention")
    assert torch.isfinite(want).all()
