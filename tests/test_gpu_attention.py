"""GPU parity of the sparse attention (ds_sparse_attention) against the CPU oracle.

Tolerance, from the arithmetic of the kernel: scores and softmax run in
float32; each weight p is rounded to the value type (unit roundoff u = 2^-8
for bf16, 2^-11 for fp16) before the value product; sums are float32.  So
|o_gpu - o_exact| <= u * max |value| over the token's rows, plus float32
rounding of order 1e-6.  The tests allow twice that.  Inputs are seeded and
synthetic (sparse_attention_kv_ds_amd.synth); the index lists are drawn
independently of any indexer run.
"""
import numpy as np
import pytest

from sparse_attention_kv_ds_amd import synth

pytestmark = pytest.mark.gpu

U = {"f16": 2.0 ** -11, "bf16": 2.0 ** -8}


@pytest.fixture(scope="module")
def ix():
    from sparse_attention_kv_ds_amd import indexer
    return indexer


@pytest.fixture(scope="module")
def orc():
    from oracle import oracle
    return oracle.load()


def to_dev(d):
    import torch
    dev = torch.device("cuda", 0)
    t = {k: torch.from_numpy(np.ascontiguousarray(d[k]).view(np.int16)).to(dev)
         for k in ("q", "kp", "vp", "kl", "vl")}
    t["idx"] = torch.from_numpy(np.ascontiguousarray(d["idx"])).to(dev)
    t["pos"] = torch.from_numpy(np.ascontiguousarray(d["pos"])).to(dev)
    return t


def run_gpu(ix, d, dtype, window, scale):
    import torch
    t = to_dev(d)
    out = ix.sparse_attention(t["q"], t["kp"], t["vp"], t["kl"], t["vl"], t["idx"], t["pos"],
                              window=window, scale=scale, dtype=dtype)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


def vmax(d, dtype):
    def dec(b):
        b = np.asarray(b, dtype=np.uint16)
        if dtype == "f16":
            return b.view(np.float16).astype(np.float64)
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    m = 0.0
    for k in ("vp", "vl"):
        if d[k].size:
            m = max(m, float(np.abs(dec(d[k])).max()))
    return m


def check(got, want, d, dtype, where=""):
    tol = 2 * U[dtype] * vmax(d, dtype) + 1e-5
    err = np.abs(got - want)
    bad = np.argwhere(err > tol)
    assert bad.size == 0, (f"{where}: {len(bad)} outputs beyond {tol:.3g}; worst {err.max():.3g} "
                           f"at {tuple(bad[0])}: got {got[tuple(bad[0])]}, want {want[tuple(bad[0])]}")


def test_tiny_workload(ix, orc):
    d = synth.make_attention("attn_tiny")
    wl = d["wl"]
    got = run_gpu(ix, d, wl.dtype, wl.window, wl.scale)
    want = orc.sparse_attention(d["q"], d["kp"], d["vp"], d["kl"], d["vl"], d["idx"], d["pos"],
                                dtype=wl.dtype, window=wl.window, scale=wl.scale)
    check(got, want, d, wl.dtype, "attn_tiny")


def random_case(seed, T, N, L, HA, D, topk, dtype, pos_lo, pos_hi, dup=False):
    rng = np.random.default_rng(seed)
    sk = 1.0 / np.sqrt(D)
    d = {"q": synth.to_bits(rng.standard_normal((T, HA, D)) * sk * 2, dtype),
         "kp": synth.to_bits(rng.standard_normal((N, D)) * sk, dtype),
         "vp": synth.to_bits(rng.standard_normal((N, D)), dtype),
         "kl": synth.to_bits(rng.standard_normal((L, D)) * sk, dtype),
         "vl": synth.to_bits(rng.standard_normal((L, D)), dtype),
         "pos": rng.integers(pos_lo, pos_hi + 1, size=T).astype(np.int32)}
    idx = np.full((T, topk), -1, dtype=np.int32)
    for t in range(T):
        if topk == 0 or N == 0:
            continue
        m = int(rng.integers(0, min(N, topk) + 1))
        rows = rng.choice(N, size=m, replace=False)
        if dup and m >= 2:
            rows[1] = rows[0]
        slots = np.sort(rng.choice(topk, size=m, replace=False)) if t % 3 == 0 else np.arange(m)
        idx[t, slots] = np.sort(rows)
    d["idx"] = idx
    return d


SHAPES = [
    # (HA, D, dtype, T, N, L, topk, window, pos range)
    (32, 64, "f16", 40, 100, 300, 16, 8, (-3, 320)),
    (32, 128, "bf16", 33, 700, 900, 100, 0, (0, 900)),
    (64, 64, "bf16", 20, 64, 100, 64, 40, (-1, 120)),
    (64, 128, "f16", 25, 3000, 5000, 512, 128, (4000, 4999)),
    (64, 128, "bf16", 17, 2000, 4000, 512, 128, (100, 4100)),
    (128, 64, "f16", 9, 300, 600, 200, 33, (0, 599)),
    (128, 128, "bf16", 7, 5000, 9000, 512, 64, (8000, 8999)),
    (64, 128, "bf16", 12, 40, 60, 0, 50, (-2, 70)),      # local rows only
    (64, 128, "f16", 12, 800, 10, 33, 1, (-2, 20)),      # one local row, pooled rows
    (32, 64, "bf16", 30, 5, 5, 7, 5, (-10, 10)),         # tiny pools
    (64, 128, "bf16", 10, 4096, 4200, 2048, 200, (4000, 4199)),  # largest index list
]


@pytest.mark.parametrize("HA,D,dtype,T,N,L,topk,window,prange", SHAPES)
def test_shapes(ix, orc, HA, D, dtype, T, N, L, topk, window, prange):
    d = random_case(HA * 7 + D + T, T, N, L, HA, D, topk, dtype, *prange)
    scale = 1.0 / np.sqrt(D)
    got = run_gpu(ix, d, dtype, window, scale)
    want = orc.sparse_attention(d["q"], d["kp"], d["vp"], d["kl"], d["vl"], d["idx"], d["pos"],
                                dtype=dtype, window=window, scale=scale, threads=8)
    check(got, want, d, dtype, f"HA={HA} D={D} {dtype}")


def test_duplicate_rows_count_twice(ix, orc):
    d = random_case(3, 16, 300, 400, 64, 128, 64, "bf16", 100, 399, dup=True)
    got = run_gpu(ix, d, "bf16", 16, 0.09)
    want = orc.sparse_attention(d["q"], d["kp"], d["vp"], d["kl"], d["vl"], d["idx"], d["pos"],
                                dtype="bf16", window=16, scale=0.09)
    check(got, want, d, "bf16", "duplicates")


def test_empty_sets_are_zero(ix):
    d = random_case(5, 8, 50, 60, 64, 128, 16, "f16", -5, -1)
    d["idx"][:] = -1
    got = run_gpu(ix, d, "f16", 4, 0.1)
    assert not got.any()


def test_attn32k_every_token(ix, orc):
    """The full 2048-token workload in one launch (the benchmark's launch
    configuration); every token checked against the oracle."""
    d = synth.make_attention("attn32k")
    wl = d["wl"]
    got = run_gpu(ix, d, wl.dtype, wl.window, wl.scale)
    want = orc.sparse_attention(d["q"], d["kp"], d["vp"], d["kl"], d["vl"], d["idx"], d["pos"],
                                dtype=wl.dtype, window=wl.window, scale=wl.scale, threads=16)
    check(got, want, d, wl.dtype, "attn32k")


def run_gpu_all(ix, d, dtype, ratio, window, scale):
    import torch
    t = to_dev(d)
    out = ix.sparse_attention_all(t["q"], t["kp"], t["vp"], t["kl"], t["vl"], t["pos"],
                                  ratio=ratio, window=window, scale=scale, dtype=dtype)
    torch.cuda.synchronize()
    return out.cpu().numpy().astype(np.float64)


ALL_SHAPES = [
    # (HA, D, dtype, T, N, L, ratio, window, pos range): the all-visible form
    (64, 128, "bf16", 30, 256, 32768, 128, 128, (30700, 32767)),
    (32, 64, "f16", 40, 70, 300, 4, 8, (-3, 290)),
    (128, 128, "f16", 9, 2048, 2100, 1, 16, (1000, 2099)),   # every raw row pooled, 2048 rows
    (64, 64, "bf16", 21, 33, 4300, 128, 0, (0, 4299)),       # pooled rows only
    (64, 128, "bf16", 12, 0, 60, 128, 20, (-2, 70)),         # empty pool
    (32, 128, "bf16", 17, 100, 5000, 16, 64, (1500, 1700)),  # positions past the pool's end
]


@pytest.mark.parametrize("HA,D,dtype,T,N,L,ratio,window,prange", ALL_SHAPES)
def test_all_visible_shapes(ix, orc, HA, D, dtype, T, N, L, ratio, window, prange):
    d = random_case(HA * 5 + D + T + ratio, T, N, L, HA, D, 0, dtype, *prange)
    scale = 1.0 / np.sqrt(D)
    got = run_gpu_all(ix, d, dtype, ratio, window, scale)
    want = orc.sparse_attention_all(d["q"], d["kp"], d["vp"], d["kl"], d["vl"], d["pos"],
                                    dtype=dtype, ratio=ratio, window=window, scale=scale,
                                    threads=8)
    check(got, want, d, dtype, f"all-visible HA={HA} D={D} {dtype} ratio={ratio}")


def test_all_visible_equals_the_sequential_lists(ix):
    """The all-visible form and the list form with each token's lists 0 .. n_t-1
    process the same rows in the same order: bit-identical outputs."""
    T, N, L, ratio = 24, 256, 33000, 128
    d = random_case(77, T, N, L, 64, 128, 0, "bf16", 30000, 32999)
    n = np.clip((d["pos"].astype(np.int64) + 1) // ratio, 0, N)
    d["idx"] = np.where(np.arange(N)[None, :] < n[:, None], np.arange(N)[None, :], -1).astype(np.int32)
    a = run_gpu_all(ix, d, "bf16", ratio, 128, 0.088)
    b = run_gpu(ix, d, "bf16", 128, 0.088)
    assert np.array_equal(a, b)


def test_attn32k_r128_every_token(ix, orc):
    """The ratio-128 form of the 32k chunk in one launch; every token checked
    against the oracle."""
    d = synth.make_attention("attn32k_r128")
    wl = d["wl"]
    got = run_gpu_all(ix, d, wl.dtype, wl.ratio, wl.window, wl.scale)
    want = orc.sparse_attention_all(d["q"], d["kp"], d["vp"], d["kl"], d["vl"], d["pos"],
                                    dtype=wl.dtype, ratio=wl.ratio, window=wl.window,
                                    scale=wl.scale, threads=16)
    check(got, want, d, wl.dtype, "attn32k_r128")


def test_deterministic(ix):
    d = random_case(9, 24, 1000, 1500, 64, 128, 256, "bf16", 1000, 1499)
    a = run_gpu(ix, d, "bf16", 64, 0.088)
    b = run_gpu(ix, d, "bf16", 64, 0.088)
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# the selection and the attention in one call (ds_indexed_sparse_attention)
# ---------------------------------------------------------------------------

def indexed_case(seed, T, N, p_lo, p_hi, topk, L, window, H=8, D=64, HA=32, dtype="f16"):
    """Integer-valued indexer inputs (every fp32 sum exact) at ratio 4 and
    Gaussian attention inputs over the same N pooled rows."""
    rng = np.random.default_rng(seed)
    q_idx, k_idx, w = synth.draw(T, N, H, D, dtype, "int", seed=seed)
    sk = 1.0 / np.sqrt(D)
    d = {"q": synth.to_bits(rng.standard_normal((T, HA, D)) * sk * 2, dtype),
         "kp": synth.to_bits(rng.standard_normal((N, D)) * sk, dtype),
         "vp": synth.to_bits(rng.standard_normal((N, D)), dtype),
         "kl": synth.to_bits(rng.standard_normal((L, D)) * sk, dtype),
         "vl": synth.to_bits(rng.standard_normal((L, D)), dtype),
         "pos": np.sort(rng.integers(p_lo, p_hi + 1, size=T)).astype(np.int32)}
    return q_idx, k_idx, w, d


def run_indexed(ix, h, q_idx, k_idx, w, d, *, topk, window, scale, extra_pool_rows=0):
    import torch
    dev = torch.device("cuda", 0)
    t = to_dev({**d, "idx": np.zeros((1, 1), dtype=np.int32)})
    if extra_pool_rows:
        pad = torch.zeros((extra_pool_rows, t["kp"].shape[1]), dtype=t["kp"].dtype, device=dev)
        t["kp"] = torch.cat([t["kp"], pad]).contiguous()
        t["vp"] = torch.cat([t["vp"], pad]).contiguous()
    qi = torch.from_numpy(q_idx.view(np.int16)).to(dev)
    ki = torch.from_numpy(k_idx.view(np.int16)).to(dev)
    wt = torch.from_numpy(w).to(dev)
    T = d["pos"].shape[0]
    idx = torch.full((T, topk), -7, dtype=torch.int32, device=dev)
    out = torch.full((T, t["q"].shape[1], t["q"].shape[2]), 3.0, dtype=torch.float32, device=dev)
    try:
        h.indexed_sparse_attention(qi, ki, wt, t["pos"], 4, topk, t["q"], t["kp"], t["vp"],
                                   t["kl"], t["vl"], window=window, scale=scale, idx=idx, out=out)
        err = None
    except ix.IndexerError as e:
        err = e
    torch.cuda.synchronize()
    return err, idx.cpu().numpy(), out.cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("seed,T,N,p_lo,p_hi,topk", [
    (1, 70, 250, 700, 999, 64),      # selection for most tokens, all-fit for the earliest
    (2, 33, 600, 2000, 2399, 100),   # selection everywhere
    (3, 40, 50, -3, 300, 64),        # every pooled row fits: no scoring at all
    (4, 1, 3000, 11999, 11999, 512), # one token: the single-token decode path, then attention
])
def test_indexed_attention_against_oracle(ix, orc, seed, T, N, p_lo, p_hi, topk):
    """idx bit-exact against the indexer oracle, out against the attention
    oracle over the oracle's own selection."""
    H, D, HA, dtype, window = 8, 64, 32, "f16", 48
    L = max(2500, p_hi + 1)  # raw rows up to the last position
    scale = 1.0 / np.sqrt(D)
    q_idx, k_idx, w, d = indexed_case(seed, T, N, p_lo, p_hi, topk, L, window, H=H, D=D, HA=HA,
                                      dtype=dtype)
    h = ix.Indexer(H, D, dtype, max_topk=topk, max_tokens=T, max_rows=N)
    try:
        err, idx, out = run_indexed(ix, h, q_idx, k_idx, w, d, topk=topk, window=window,
                                    scale=scale)
    finally:
        h.close()
    assert err is None, err
    want_idx = orc.score_topk(q_idx, k_idx, w, d["pos"], H=H, D=D, dtype=dtype, ratio=4,
                              topk=topk, threads=8)
    np.testing.assert_array_equal(idx, want_idx)
    want = orc.sparse_attention(d["q"], d["kp"], d["vp"], d["kl"], d["vl"], want_idx, d["pos"],
                                dtype=dtype, window=window, scale=scale, threads=8)
    check(out, want, d, dtype, f"indexed seed {seed}")


def test_indexed_attention_refuses_diverged_pool_counts(ix):
    """Pooled-row counts that differ between the indexer's and the attention's
    rows: DS_ERR_INVALID_ARG, and neither idx nor out is written."""
    H, D, HA, dtype, T, N, topk = 8, 64, 32, "f16", 20, 300, 64
    q_idx, k_idx, w, d = indexed_case(9, T, N, 800, 1100, topk, 1200, 16, H=H, D=D, HA=HA,
                                      dtype=dtype)
    h = ix.Indexer(H, D, dtype, max_topk=topk, max_tokens=T, max_rows=N + 1)
    try:
        err, idx, out = run_indexed(ix, h, q_idx, k_idx, w, d, topk=topk, window=16,
                                    scale=0.125, extra_pool_rows=1)
    finally:
        h.close()
    assert err is not None and err.status == ix.DS_ERR_INVALID_ARG
    assert (idx == -7).all() and (out == 3.0).all()
