"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Integer-valued inputs (q, k integers, w = +-2^-n) make every fp32 sum exact in
any order, so indices AND scores must match the oracle bit for bit.  Gaussian
inputs must match scores within 1e-3 relative, and the selected set must agree
except inside the tie margin around the oracle's k-th best score.  Full-size
workloads are compared with the oracle on every token (indices and scores),
and also checked through properties that hold at any size (ascending, unique,
causal, all-fit sequential, and dominance of the selected rows under the
GPU's own scores).
"""
import sys

import numpy as np
import pytest
import torch

from oracle import oracle as oracle_mod
from oracle_pins import check_output_row, rand_int_case
from sparse_attention_kv_ds_amd import synth

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
REL = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def orc():
    return oracle_mod.load()


@pytest.fixture(scope="module")
def lib():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a GPU")
    from sparse_attention_kv_ds_amd import indexer
    return indexer


def dev_inputs(q, k, w, pos):
    return (torch.from_numpy(np.ascontiguousarray(q).view(np.int16)).to(DEV),
            torch.from_numpy(np.ascontiguousarray(k).view(np.int16)).to(DEV),
            torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).to(DEV),
            torch.from_numpy(np.ascontiguousarray(pos, dtype=np.int32)).to(DEV))


def gpu_run(lib, q, k, w, pos, *, H, D, dtype, ratio, topk, scores=False, ix=None):
    T, N = len(pos), k.shape[0]
    own = ix is None
    if own:
        ix = lib.Indexer(H, D, dtype, max(topk, 1), max(T, 1), max(N, 1), device=0)
    try:
        tq, tk, tw, tp = dev_inputs(q, k, w, pos)
        out = ix.score_topk(tq, tk, tw, tp, ratio, topk)
        sc = ix.scores(tq, tk, tw, tp, ratio) if scores else None
        torch.cuda.synchronize(DEV)
        res = out.cpu().numpy()
        return (res, sc.cpu().numpy()) if scores else res
    finally:
        if own:
            ix.close()


def visible(pos, ratio, N):
    p = np.asarray(pos, dtype=np.int64)
    return np.clip(np.where(p < 0, 0, (p + 1) // ratio), 0, N)


def ordered_keys(scores_f32, rows):
    """The unique selection key of (score, row) as uint64, computed on the host."""
    b = np.ascontiguousarray(scores_f32, dtype=np.float32).view(np.uint32).copy()
    b[b == 0x80000000] = 0
    neg = (b & 0x80000000) != 0
    o = np.where(neg, ~b, b | 0x80000000).astype(np.uint64)
    return (o << np.uint64(32)) | (np.uint64(0xFFFFFFFF) - rows.astype(np.uint64))


def check_all_tokens(out, gscores, pos, ratio, N, topk, where):
    """Invariants on every token, plus dominance under the GPU's own scores."""
    ns = visible(pos, ratio, N)
    for t in range(len(pos)):
        n = int(ns[t])
        sel = check_output_row(out[t], n, topk, f"{where} token {t}")
        if gscores is not None and n > topk:
            rows = np.arange(n)
            keys = ordered_keys(gscores[t, :n], rows)
            mask = np.zeros(n, dtype=bool)
            mask[sel] = True
            assert keys[mask].min() > keys[~mask].max(), f"{where} token {t}: dominance"


def check_tolerant(out_row, g_row, o_row, n, topk, where):
    """Scores within REL relative; set agreement outside the tie margin."""
    m = min(n, topk)
    sel = check_output_row(out_row, n, topk, where)
    if n == 0:
        return
    g = g_row[:n].astype(np.float64)
    o = o_row[:n]
    err = np.abs(g - o)
    bad = np.nonzero(err > REL * np.abs(o))[0]
    assert bad.size == 0, f"{where}: score row {bad[0]} gpu {g[bad[0]]} oracle {o[bad[0]]}"
    if n <= topk:
        return
    order = np.lexsort((np.arange(n), -o))
    tau = o[order[m - 1]]
    delta = REL * abs(tau)
    chosen = np.zeros(n, dtype=bool)
    chosen[sel] = True
    must = o > tau + delta
    must_not = o < tau - delta
    assert chosen[must].all(), f"{where}: a row clearly above the k-th score was dropped"
    assert not chosen[must_not].any(), f"{where}: a row clearly below the k-th score was kept"
    assert len(sel) == m


def exact_case(lib, orc, q, k, w, pos, *, H, D, dtype, ratio, topk, where, ix=None):
    out, sc = gpu_run(lib, q, k, w, pos, H=H, D=D, dtype=dtype, ratio=ratio, topk=topk,
                      scores=True, ix=ix)
    want, osc = orc.score_topk(q, k, w, pos, H=H, D=D, dtype=dtype, ratio=ratio, topk=topk,
                               want_scores=True, threads=8)
    diff = np.argwhere(out != want)
    assert diff.size == 0, (f"{where}: token {diff[0][0]} got {out[diff[0][0]].tolist()} "
                            f"want {want[diff[0][0]].tolist()}")
    np.testing.assert_array_equal(sc.astype(np.float64), osc, err_msg=f"{where}: scores")


# ---------------------------------------------------------------------------
# small and medium shapes, bit-exact
# ---------------------------------------------------------------------------

def test_tiny_workload_bit_exact(lib, orc):
    d = synth.make("tiny")
    wl = d["wl"]
    say("tiny workload T=256 N=64 H=4 D=32 k=48")
    exact_case(lib, orc, d["q"], d["k"], d["w"], d["pos"], H=wl.H, D=wl.D, dtype=wl.dtype,
               ratio=wl.ratio, topk=wl.topk, where="tiny")
    n = visible(d["pos"], wl.ratio, wl.N)
    assert (n <= wl.topk).sum() == 195 and (n == 0).sum() == 3  # skip-path tokens


SHAPES = [
    # H, D, dtype, topk, T, N, ratio
    (4, 32, "f16", 48, 300, 257, 4),
    (4, 64, "bf16", 5, 77, 1100, 1),
    (8, 32, "f16", 48, 130, 700, 4),
    (8, 128, "bf16", 100, 64, 1500, 2),
    (16, 64, "f16", 1, 45, 2100, 3),
    (16, 128, "f16", 512, 40, 3000, 1),
    (32, 32, "bf16", 48, 70, 1500, 4),
    (32, 128, "f16", 512, 33, 2500, 1),
    (64, 32, "f16", 48, 20, 1025, 1),
    (64, 64, "bf16", 200, 17, 1999, 1),
    (64, 128, "f16", 512, 24, 2600, 1),
    (64, 128, "bf16", 512, 9, 4100, 1),
    (64, 128, "f16", 1, 10, 3000, 1),
    (64, 128, "f16", 2048, 12, 5000, 1),
]


@pytest.mark.parametrize("H,D,dtype,topk,T,N,ratio", SHAPES)
def test_shapes_bit_exact(lib, orc, H, D, dtype, topk, T, N, ratio):
    say(f"shape H={H} D={D} {dtype} k={topk} T={T} N={N} r={ratio}")
    rng = np.random.default_rng(1000 + H * 7 + D + T)
    q, k, w, _ = rand_int_case(rng, T, N, H, D, -4, 4, ratio, 1, dtype)
    # positions sweep from "nothing visible" through "all fit" to "all rows"
    pos = np.sort(rng.integers(-3, ratio * (N + 40), size=T)).astype(np.int32)
    pos[-1] = ratio * N + 5
    exact_case(lib, orc, q, k, w, pos, H=H, D=D, dtype=dtype, ratio=ratio, topk=topk,
               where=f"H{H}D{D}{dtype}k{topk}")


def test_frontier_sweep_bit_exact(lib, orc):
    """32 chunk start positions straddling n = 0 and n = topk, as consecutive chunks."""
    H, D, topk, ratio, N, T = 8, 64, 48, 4, 300, 40
    starts = sorted(set([-45, -39, -2, 0, 1, 3, 150, 170, 180, 185, 188, 189, 190, 191, 192, 193,
                         194, 195, 196, 200, 230, 300, 500, 640, 700, 1000, 1150, 1160, 1170,
                         1180, 1195, 1300]))
    assert len(starts) == 32
    rng = np.random.default_rng(7)
    q, k, w, _ = rand_int_case(rng, T, N, H, D, -4, 4, ratio, 1, "f16")
    lib_ix = lib.Indexer(H, D, "f16", topk, T, N, device=0)
    try:
        for p0 in starts:
            say(f"frontier p0={p0}")
            pos = np.arange(p0, p0 + T, dtype=np.int32)
            exact_case(lib, orc, q, k, w, pos, H=H, D=D, dtype="f16", ratio=ratio, topk=topk,
                       where=f"frontier {p0}", ix=lib_ix)
    finally:
        lib_ix.close()


def test_edge_cases(lib, orc):
    rng = np.random.default_rng(9)
    H, D = 64, 128
    q, k, w, _ = rand_int_case(rng, 6, 600, H, D, -4, 4, 4, 1, "f16")
    ix = lib.Indexer(H, D, "f16", 512, 6, 600, device=0)
    try:
        say("edge: N = 0")
        out = gpu_run(lib, q, k[:0], w, np.array([5, 9, 100, 0, -1, 3], np.int32), H=H, D=D,
                      dtype="f16", ratio=4, topk=7, ix=ix)
        assert (out == -1).all()
        say("edge: T = 0")
        out = gpu_run(lib, q[:0], k, w[:0], np.zeros(0, np.int32), H=H, D=D, dtype="f16",
                      ratio=4, topk=7, ix=ix)
        assert out.shape == (0, 7)
        say("edge: every token all-fit / empty / negative / beyond N")
        for pos, ratio, topk in (([0, 1, 2, 3, 4, 2047], 4, 512),
                                 ([-100, -1, 2, 2**31 - 1, 599, 600], 1, 512),
                                 ([-100, -1, 2, 2**31 - 1, 599, 600], 1, 3),
                                 ([127, 128 * 5 - 1, 128 * 600, 10**6, 255, 0], 128, 2),
                                 ([6, 5, 4, 3, 2, 1], 1, 1)):
            pos = np.array(pos, dtype=np.int32)
            exact_case(lib, orc, q, k, w, pos, H=H, D=D, dtype="f16", ratio=ratio, topk=topk,
                       where=f"edge pos={pos.tolist()} r={ratio} k={topk}", ix=ix)
        say("edge: all scores equal (ties broken by row)")
        qz = np.zeros_like(q)
        exact_case(lib, orc, qz, k, w, np.array([599, 2000, 2399, 9999, 100, 40], np.int32),
                   H=H, D=D, dtype="f16", ratio=4, topk=17, where="all ties", ix=ix)
    finally:
        ix.close()


def test_deterministic(lib):
    d = synth.make("tiny")
    wl = d["wl"]
    a = gpu_run(lib, d["q"], d["k"], d["w"], d["pos"], H=wl.H, D=wl.D, dtype=wl.dtype,
                ratio=wl.ratio, topk=wl.topk, scores=True)
    b = gpu_run(lib, d["q"], d["k"], d["w"], d["pos"], H=wl.H, D=wl.D, dtype=wl.dtype,
                ratio=wl.ratio, topk=wl.topk, scores=True)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


# ---------------------------------------------------------------------------
# single-token decode path
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("N,topk,dtype", [(100, 48, "f16"), (700, 512, "f16"), (1025, 512, "bf16"),
                                          (5000, 512, "f16"), (70000, 512, "f16"),
                                          (33000, 2048, "bf16"), (20000, 1, "f16")])
def test_decode_integer_bit_exact(lib, orc, N, topk, dtype):
    say(f"decode int N={N} k={topk} {dtype}")
    rng = np.random.default_rng(N + topk)
    q, k, w, _ = rand_int_case(rng, 1, N, 64, 128, -4, 4, 4, 1, dtype)
    for p in (4 * N - 1, 4 * N + 100, 4 * (N // 2) + 1):
        exact_case(lib, orc, q, k, w, np.array([p], np.int32), H=64, D=128, dtype=dtype, ratio=4,
                   topk=topk, where=f"decode N={N} pos={p}")


def batch_run(lib, q, k, w, pos, *, H, D, dtype, ratio, topk):
    """ds_indexer_score_topk_batch on host arrays: q [B,H,D], k [B,N,D], w [B,H], pos [B]."""
    B, N = len(pos), k.shape[1]
    ix = lib.Indexer(H, D, dtype, max(topk, 1), max(B, 1), max(N, 1), device=0)
    try:
        tq, tk, tw, tp = dev_inputs(q, k, w, pos)
        out = ix.score_topk_batch(tq, tk, tw, tp, ratio, topk)
        torch.cuda.synchronize(DEV)
        return out.cpu().numpy()
    finally:
        ix.close()


@pytest.mark.parametrize("B,N,topk,dtype", [(5, 5000, 512, "f16"), (3, 700, 512, "bf16"),
                                            (9, 1100, 48, "f16"), (2, 300, 512, "f16"),
                                            (64, 3000, 512, "bf16")])
def test_decode_batch_integer_bit_exact(lib, orc, B, N, topk, dtype):
    """Each sequence of a batched decode call equals the oracle on that sequence
    alone; positions differ per sequence (all rows, half the rows, all-fit, none)."""
    say(f"batched decode int B={B} N={N} k={topk} {dtype}")
    rng = np.random.default_rng(B * 1000 + N)
    H, D = 64, 128
    qs, ks, ws = [], [], []
    for b in range(B):
        q, k, w, _ = rand_int_case(rng, 1, N, H, D, -4, 4, 4, 1, dtype)
        qs.append(q[0]); ks.append(k); ws.append(w[0])
    choices = [4 * N - 1, 4 * N + 77, 2 * N + 1, 4 * min(topk, N) - 1, -3, 4 * (N // 3)]
    pos = np.array([choices[b % len(choices)] for b in range(B)], np.int32)
    q, k, w = np.stack(qs), np.stack(ks), np.stack(ws)
    out = batch_run(lib, q, k, w, pos, H=H, D=D, dtype=dtype, ratio=4, topk=topk)
    for b in range(B):
        want = orc.score_topk(q[b:b + 1], k[b], w[b:b + 1], pos[b:b + 1], H=H, D=D, dtype=dtype,
                              ratio=4, topk=topk, threads=8)
        assert np.array_equal(out[b], want[0]), f"sequence {b} (pos {pos[b]}) differs"


def test_decode_batch_equals_single_calls(lib):
    """Gaussian sequences: the batched call gives every sequence bit for bit what a
    single-token call gives it, including a sequence whose rows all fit."""
    say("batched decode vs single calls (gaussian)")
    rng = np.random.default_rng(8)
    B, N, H, D, topk = 6, 70000, 64, 128, 512
    q = synth.to_bits(rng.standard_normal((B, H, D)) / np.sqrt(128.0), "bf16")
    k = synth.to_bits(rng.standard_normal((B, N, D)) / np.sqrt(128.0), "bf16")
    w = rng.random((B, H), dtype=np.float32)
    pos = np.array([4 * N - 1, 4 * N - 1, 3 * N, 1000, 4 * N - 1, 4 * N + 5], np.int32)
    out = batch_run(lib, q, k, w, pos, H=H, D=D, dtype="bf16", ratio=4, topk=topk)
    for b in range(B):
        one = gpu_run(lib, q[b:b + 1], k[b], w[b:b + 1], pos[b:b + 1], H=H, D=D, dtype="bf16",
                      ratio=4, topk=topk)
        assert np.array_equal(out[b], one[0]), f"sequence {b} differs from its single call"
    check_all_tokens(out, None, pos, 4, N, topk, "batched decode")


def test_decode1m_batch_full_size(lib, orc):
    """Eight 1M-token sequences (fp16 Gaussian, 262144 rows each) in one call: two of
    them against the oracle (tolerance and tie margin), all eight against single calls."""
    say("full-size batched decode, 8 x 262144 rows")
    d = synth.make_decode_batch("decode1m_b8")
    wl, B = d["wl"], d["B"]
    out = batch_run(lib, d["q"], d["k"], d["w"], d["pos"], H=wl.H, D=wl.D, dtype=wl.dtype,
                    ratio=wl.ratio, topk=wl.topk)
    for b in range(B):
        one, sc = gpu_run(lib, d["q"][b:b + 1], d["k"][b], d["w"][b:b + 1], d["pos"][b:b + 1],
                          H=wl.H, D=wl.D, dtype=wl.dtype, ratio=wl.ratio, topk=wl.topk,
                          scores=True)
        assert np.array_equal(out[b], one[0]), f"sequence {b} differs from its single call"
        if b in (0, B - 1):
            _, osc = orc.score_topk(d["q"][b:b + 1], d["k"][b], d["w"][b:b + 1],
                                    d["pos"][b:b + 1], H=wl.H, D=wl.D, dtype=wl.dtype,
                                    ratio=wl.ratio, topk=wl.topk, want_scores=True, threads=16)
            n = int(visible(d["pos"][b:b + 1], wl.ratio, wl.N)[0])
            check_tolerant(out[b], sc[0], osc[0], n, wl.topk, f"decode1m_b8 sequence {b}")


def proj_run(lib, x, wq, H, D, dtype, topk=None, k=None, w=None, pos=None, ratio=4):
    """ds_indexer_project_q (topk None) or ds_indexer_project_score_topk on host arrays."""
    T, din = x.shape
    N = k.shape[0] if k is not None else 1
    ix = lib.Indexer(H, D, dtype, max(topk or 1, 1), max(T, 1), max(N, 1), device=0)
    try:
        tx = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).to(DEV)
        tw = torch.from_numpy(np.ascontiguousarray(wq).view(np.int16)).to(DEV)
        if topk is None:
            q = ix.project_q(tx, tw)
            torch.cuda.synchronize(DEV)
            return q.cpu().numpy().view(np.uint16).reshape(T, H * D)
        _, tk, tww, tp = dev_inputs(np.zeros((1, H, D), np.uint16), k, w, pos)
        out = ix.project_score_topk(tx, tw, tk, tww, tp, ratio, topk)
        torch.cuda.synchronize(DEV)
        return out.cpu().numpy()
    finally:
        ix.close()


def ulp_distance(a_bits, b_bits):
    """Distance in representable steps between two arrays of 16-bit float bits."""
    def ordered(b):
        b = b.astype(np.int32)
        return np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(ordered(a_bits) - ordered(b_bits))


@pytest.mark.parametrize("T,din,H,D,dtype", [(37, 64, 4, 32, "f16"), (300, 200, 64, 128, "bf16"),
                                             (129, 1536, 64, 128, "f16"), (8, 24, 8, 64, "bf16"),
                                             (256, 1536, 32, 128, "bf16"), (70, 136, 16, 64, "f16"),
                                             (520, 320, 8, 128, "bf16"), (300, 72, 4, 32, "bf16")])
def test_project_q_against_oracle(lib, orc, T, din, H, D, dtype):
    """Gaussian operands: the GPU sums in fp32 and rounds once, the oracle sums
    in double and rounds once.  So each GPU value lies within one step of the
    storage type plus the fp32 summation bound d_in * 2^-24 * sum_i |x_i w_i| of
    the exact sum (that bound matters only where the terms cancel), and all but
    a small fraction of the values are identical to the oracle's.  Integer operands (exact sums):
    bit-exact."""
    say(f"projection T={T} d_in={din} O={H * D} {dtype}")
    rng = np.random.default_rng(T + din)
    x = synth.to_bits(rng.standard_normal((T, din)), dtype)
    wq = synth.to_bits(rng.standard_normal((H * D, din)) / np.sqrt(din), dtype)
    got = proj_run(lib, x, wq, H, D, dtype)
    want = orc.project_q(x, wq, dtype=dtype, threads=16)
    d = ulp_distance(got, want)
    # a rounding decision differs only where the exact sum lies within the fp32
    # error of a midpoint: rare (about sqrt(d_in) 2^-24 / 2^-11 at most, fp16)
    assert (d > 0).mean() < 1e-2, f"{(d > 0).mean():.2e} of q not identical"

    def dec(b):
        b = np.asarray(b, dtype=np.uint16)
        if dtype == "f16":
            return b.view(np.float16).astype(np.float64)
        return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    xd, wd = dec(x), dec(wq)
    exact = xd @ wd.T
    bound = din * 2.0 ** -24 * (np.abs(xd) @ np.abs(wd).T)
    step = np.abs(dec(want) - dec(want ^ np.uint16(1)))  # one step of the type at the oracle's value
    err = np.abs(dec(got) - exact)
    bad = np.argwhere(err > step + bound)
    assert bad.size == 0, f"{len(bad)} values beyond one step plus the fp32 bound, e.g. {tuple(bad[0])}"
    xi = synth.to_bits(rng.integers(-3, 4, size=(T, din)), dtype)
    wi = synth.to_bits(rng.integers(-2, 3, size=(H * D, din)), dtype)
    assert np.array_equal(proj_run(lib, xi, wi, H, D, dtype), orc.project_q(xi, wi, dtype=dtype,
                                                                            threads=16))


def test_project_score_topk_integer_exact(lib, orc):
    """Projection then score + top-k in one call, integer inputs kept small enough
    that every fp32 sum is exact (|q| <= 128, |q . k| <= 2^16, 64 heads): bit-exact
    against the oracle's projection then score + top-k.  A pool that fits in top-k
    skips the projection and the scoring."""
    say("projection + indexer, integer, bit-exact")
    rng = np.random.default_rng(12)
    T, din, H, D, N, topk = 70, 64, 64, 128, 900, 100
    x = synth.to_bits(rng.integers(-2, 3, size=(T, din)), "f16")
    wq = synth.to_bits(rng.integers(-1, 2, size=(H * D, din)), "f16")
    k = synth.to_bits(rng.integers(-4, 5, size=(N, D)), "f16")
    w = ((rng.integers(0, 2, size=(T, H)) * 2 - 1) * np.ldexp(1.0, -rng.integers(0, 4, size=(T, H)))
         ).astype(np.float32)
    pos = rng.integers(-2, 4 * N + 3, size=T).astype(np.int32)
    got = proj_run(lib, x, wq, H, D, "f16", topk=topk, k=k, w=w, pos=pos)
    want = orc.project_score_topk(x, wq, k, w, pos, H=H, D=D, dtype="f16", ratio=4, topk=topk,
                                  threads=16)
    assert np.array_equal(got, want)
    got = proj_run(lib, x, wq, H, D, "f16", topk=N, k=k, w=w, pos=pos)
    want = orc.project_score_topk(x, wq, k, w, pos, H=H, D=D, dtype="f16", ratio=4, topk=N,
                                  threads=16)
    assert np.array_equal(got, want)


def test_qproj32k_full_size(lib, orc):
    """The full 32k-chunk projection (2048 x 1536 -> 64 x 128, bf16 Gaussian) fused
    ahead of the indexer: every token within score tolerance and tie margin of
    the oracle's projection then scores, and every token's output valid."""
    say("full-size qproj32k")
    d = synth.make_projection("qproj32k")
    wl = d["wl"]
    out = proj_run(lib, d["x"], d["wq"], wl.H, wl.D, d["dtype"], topk=wl.topk, k=d["k"],
                   w=d["w"], pos=d["pos"], ratio=wl.ratio)
    q_gpu = proj_run(lib, d["x"], d["wq"], wl.H, wl.D, d["dtype"]).reshape(wl.T, wl.H, wl.D)
    _, sc = gpu_run(lib, q_gpu, d["k"], d["w"], d["pos"], H=wl.H, D=wl.D, dtype=d["dtype"],
                    ratio=wl.ratio, topk=wl.topk, scores=True)
    say(f"full-size qproj32k: oracle projection and scores on all {wl.T} tokens")
    _, osc = orc.project_score_topk(d["x"], d["wq"], d["k"], d["w"], d["pos"], H=wl.H, D=wl.D,
                                    dtype=d["dtype"], ratio=wl.ratio, topk=wl.topk,
                                    want_scores=True, threads=16)
    n = visible(d["pos"], wl.ratio, wl.N)
    for t in range(wl.T):
        check_tolerant(out[t], sc[t], osc[t], int(n[t]), wl.topk, f"qproj32k token {t}")
    check_all_tokens(out, sc, d["pos"], wl.ratio, wl.N, wl.topk, "qproj32k")


@pytest.mark.parametrize("N", [40000, 70000])
def test_decode_fallback_paths_exact(lib, orc, N):
    """Scores rising with the row concentrate the best rows in the last partitions
    (their short candidate lists cannot be trusted), and all-equal scores make
    every partition's list a pure tie-break; both must stay exact.  At 40000 rows
    the partitions list 16 keys each (selected by the threshold search), at 70000
    rows 8 (selected by ranking)."""
    D, H = 128, 64
    rng = np.random.default_rng(3)
    kf = np.zeros((N, D))
    kf[:, 0] = np.floor(np.arange(N) / 40)  # non-decreasing, exact in fp16 up to 2048
    kf[:, 1:] = rng.integers(-1, 2, size=(N, D - 1))
    k = synth.to_bits(kf, "f16")
    qf = np.zeros((1, H, D))
    qf[0, :, 0] = 1
    w = np.ones((1, H), np.float32)
    q = synth.to_bits(qf, "f16")
    for topk in (512, 100):
        say(f"decode rising scores N={N} k={topk}")
        exact_case(lib, orc, q, k, w, np.array([4 * N - 1], np.int32), H=H, D=D, dtype="f16",
                   ratio=4, topk=topk, where="decode rising")
    say(f"decode all ties N={N}")
    exact_case(lib, orc, np.zeros_like(q), k, w, np.array([4 * N - 1], np.int32), H=H, D=D,
               dtype="f16", ratio=4, topk=512, where="decode ties")


# ---------------------------------------------------------------------------
# full-size workloads (the launch configuration the benchmark times)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["prefill2k", "prefill8k", "prefill32k"])
def test_integer_workloads_full_size(lib, orc, name):
    """Every token of the full integer workload, in the launch configuration the
    benchmark times: indices and scores bit-exact against the oracle."""
    say(f"full-size {name}")
    d = synth.make(name)
    wl = d["wl"]
    out, sc = gpu_run(lib, d["q"], d["k"], d["w"], d["pos"], H=wl.H, D=wl.D, dtype=wl.dtype,
                      ratio=wl.ratio, topk=wl.topk, scores=True)
    say(f"full-size {name}: oracle on all {wl.T} tokens")
    want, osc = orc.score_topk(d["q"], d["k"], d["w"], d["pos"], H=wl.H, D=wl.D, dtype=wl.dtype,
                               ratio=wl.ratio, topk=wl.topk, want_scores=True, threads=16)
    bad = np.nonzero((out != want).any(axis=1))[0]
    assert bad.size == 0, (f"{name}: {bad.size} of {wl.T} tokens differ; token {bad[0]} got "
                           f"{out[bad[0]].tolist()} want {want[bad[0]].tolist()}")
    # every score (-inf where a row is not visible), bit for bit
    sbad = np.nonzero((sc.astype(np.float64) != osc).any(axis=1))[0]
    assert sbad.size == 0, f"{name}: scores of {sbad.size} tokens differ, first token {sbad[0]}"
    check_all_tokens(out, sc, d["pos"], wl.ratio, wl.N, wl.topk, name)


def test_gaussian_prefill64k_full_size(lib, orc):
    """Every token of the full 64k workload (bf16 Gaussian): scores within 1e-3
    relative of the oracle on every visible pair, and the selected set equal
    outside the tie margin."""
    say("full-size prefill64k (bf16 gaussian)")
    d = synth.make("prefill64k")
    wl = d["wl"]
    out, sc = gpu_run(lib, d["q"], d["k"], d["w"], d["pos"], H=wl.H, D=wl.D, dtype=wl.dtype,
                      ratio=wl.ratio, topk=wl.topk, scores=True)
    say(f"full-size prefill64k: oracle on all {wl.T} tokens")
    want, osc = orc.score_topk(d["q"], d["k"], d["w"], d["pos"], H=wl.H, D=wl.D, dtype=wl.dtype,
                               ratio=wl.ratio, topk=wl.topk, want_scores=True, threads=16)
    ns = visible(d["pos"], wl.ratio, wl.N)
    same = 0
    for t in range(wl.T):
        check_tolerant(out[t], sc[t], osc[t], int(ns[t]), wl.topk, f"64k token {t}")
        same += int(np.array_equal(out[t], want[t]))
    say(f"full-size prefill64k: {same} of {wl.T} tokens select exactly the oracle's rows")
    check_all_tokens(out, sc, d["pos"], wl.ratio, wl.N, wl.topk, "64k")


def test_decode1m_full_size(lib, orc):
    say("full-size decode1m (fp16 gaussian, 262144 rows)")
    d = synth.make("decode1m")
    wl = d["wl"]
    out, sc = gpu_run(lib, d["q"], d["k"], d["w"], d["pos"], H=wl.H, D=wl.D, dtype=wl.dtype,
                      ratio=wl.ratio, topk=wl.topk, scores=True)
    want, osc = orc.score_topk(d["q"], d["k"], d["w"], d["pos"], H=wl.H, D=wl.D, dtype=wl.dtype,
                               ratio=wl.ratio, topk=wl.topk, want_scores=True, threads=1)
    n = int(visible(d["pos"], wl.ratio, wl.N)[0])
    assert n == 262144
    check_tolerant(out[0], sc[0], osc[0], n, wl.topk, "decode1m")
    check_all_tokens(out, sc, d["pos"], wl.ratio, wl.N, wl.topk, "decode1m")


def test_timing_markers_do_not_change_results(lib):
    """Per-kernel HIP events (ds_indexer_timing): every launch class is counted once per
    call, durations are positive, and the outputs are the same with markers on or off."""
    say("timing markers: prefill and decode calls")
    rng = np.random.default_rng(77)
    H, D, topk = 8, 64, 32
    for T, N, p0 in ((40, 600, 2000), (1, 5000, 4 * 5000 - 1)):
        q, k, w, _ = rand_int_case(rng, T, N, H, D, -4, 4, 4, 1, "f16")
        pos = np.arange(p0, p0 + T, dtype=np.int32)
        ix = lib.Indexer(H, D, "f16", topk, T, N, device=0)
        try:
            plain = gpu_run(lib, q, k, w, pos, H=H, D=D, dtype="f16", ratio=4, topk=topk, ix=ix)
            ix.timing(True)
            ix.timing_read()
            marked = gpu_run(lib, q, k, w, pos, H=H, D=D, dtype="f16", ratio=4, topk=topk, ix=ix)
            per = ix.timing_read()
            ix.timing(False)
            after = gpu_run(lib, q, k, w, pos, H=H, D=D, dtype="f16", ratio=4, topk=topk, ix=ix)
            silent = ix.timing_read()
        finally:
            ix.close()
        assert np.array_equal(plain, marked) and np.array_equal(plain, after)
        classes = ("decode_score", "decode_select") if T == 1 else ("score", "select")
        for c, (ms, n) in per.items():
            if c in classes:
                assert n == 1 and ms > 0.0, (c, ms, n)
            else:
                assert n == 0, (c, n)
        assert all(n == 0 for _, n in silent.values())


def test_sampled_threshold_restart(lib, orc):
    """Rows long enough for the sampled starting threshold, built so that the sample
    overestimates it: every sampled row (a multiple of the sampling step) has the top
    score, so fewer than k rows of the whole row reach the estimate and the row must
    be streamed again from threshold 0.  Bit-exact against the oracle either way."""
    say("sampled threshold restart: n = 4096..8192, sampled rows carry the top score")
    H, D, topk, ratio = 4, 32, 512, 1
    for N in (4096, 6000, 8192):
        step = N // 1024
        k = np.zeros((N, D), dtype=np.float64)
        j = np.arange(N)
        k[:, 0] = np.where(j % step == 0, 4, j % 3)
        q = np.zeros((3, H, D), dtype=np.float64)
        q[:, :, 0] = 1
        w = np.ones((3, H), dtype=np.float32)
        pos = np.array([N - 1, N - 2, N + 5], dtype=np.int32)
        exact_case(lib, orc, synth.to_bits(q, "f16"), synth.to_bits(k, "f16"), w, pos, H=H, D=D,
                   dtype="f16", ratio=ratio, topk=topk, where=f"restart N={N}")


def test_sampled_threshold_restart_short_rows(lib, orc):
    """Rows of 1024..4095, sampled with 4 runs of 64 rows: the sampled runs (at
    s (n - 64) / 3, s = 0..3) carry the top score and every other row a lower
    one, so the estimate is the top score, which only 256 < k rows reach: the
    row must be streamed again from threshold 0.  Bit-exact against the
    oracle either way."""
    H, D, topk, ratio = 4, 32, 512, 1
    for N in (1024, 2048, 3000, 4095):
        say(f"sampled threshold restart, short rows: n = {N}")
        j = np.arange(N)
        top = np.zeros(N, dtype=bool)
        for r in range(4):
            a = r * (N - 64) // 3
            top[a:a + 64] = True
        k = np.zeros((N, D), dtype=np.float64)
        k[:, 0] = np.where(top, 8, j % 5)
        q = np.zeros((3, H, D), dtype=np.float64)
        q[:, :, 0] = 1
        w = np.ones((3, H), dtype=np.float32)
        pos = np.array([N - 1, N - 1, N + 2], dtype=np.int32)
        exact_case(lib, orc, synth.to_bits(q, "f16"), synth.to_bits(k, "f16"), w, pos, H=H, D=D,
                   dtype="f16", ratio=ratio, topk=topk, where=f"short-row restart N={N}")


def test_long_rows_with_a_top_run_bit_exact(lib, orc):
    """Long rows (7168..16384) whose first 64 rows -- the first run of the
    starting-threshold sample, one row per lane -- carry the top score and the
    rest three lower levels: the sample overweights the top, and the row has
    thousands of equal scores at each lower level, so the selection is a pure
    tie-break by row below the top 64.  Bit-exact against the oracle."""
    H, D, topk, ratio = 4, 32, 512, 1
    for N in (7168, 8192, 16384):
        say(f"long rows with a top run N={N}")
        k = np.zeros((N, D), dtype=np.float64)
        j = np.arange(N)
        k[:, 0] = np.where(j < 64, 4, j % 3)
        q = np.zeros((3, H, D), dtype=np.float64)
        q[:, :, 0] = 1
        w = np.ones((3, H), dtype=np.float32)
        pos = np.array([N - 1, N - 7, N + 5], dtype=np.int32)
        exact_case(lib, orc, synth.to_bits(q, "f16"), synth.to_bits(k, "f16"), w, pos, H=H, D=D,
                   dtype="f16", ratio=ratio, topk=topk, where=f"top run N={N}")


@pytest.mark.parametrize("sure,bucket,topk", [(500, 30, 512), (400, 300, 512), (100, 1500, 512),
                                               (0, 2000, 512), (980, 50, 1000),
                                               (700, 600, 1000), (200, 3000, 1000)])
def test_split_score_boundary_buckets_exact(lib, orc, sure, bucket, topk):
    """The selection streams the high 16 bits of each ordered score and
    completes only the boundary's high half with the low 16 bits.  Rows of
    8192: `sure` rows score above every other, `bucket` rows score distinct
    values in [1024, 1032) (one high half, different low halves, in an order
    unrelated to the row), the rest score below.  k falls inside the
    bucket, so the answer depends on the low halves: 30 or 50 rows are ranked
    one per lane, 300 or 600 go through the exact search, and 1500 to 3000
    are more than a streaming shrink can keep as a whole high half, so the
    row is streamed again with exact scores (k = 1000 uses the larger buffer
    that reads its low words from LDS).  Bit-exact against the oracle."""
    H, D, ratio, N = 4, 32, 1, 8192
    rng = np.random.default_rng(sure * 7 + bucket + topk)
    rows = rng.permutation(N)
    k = np.zeros((N, D), dtype=np.float64)
    hi_rows, b_rows, lo_rows = rows[:sure], rows[sure:sure + bucket], rows[sure + bucket:]
    k[hi_rows, 0] = 300.0
    k[hi_rows, 1] = rng.integers(0, 64, size=sure) / 64.0
    k[b_rows, 0] = 256.0
    # every fp16 value in [1/32, 2) is a multiple of 2^-15, so 256 + k1 and
    # s = 4 (256 + k1) in [1024, 1032) are exact in fp32: one high half, 6144
    # distinct scores to draw from
    frac = np.arange(0x2800, 0x4000, dtype=np.uint16).view(np.float16).astype(np.float64)
    k[b_rows, 1] = rng.permutation(frac)[:bucket]
    k[lo_rows, 0] = rng.integers(0, 200, size=len(lo_rows))
    q = np.zeros((3, H, D), dtype=np.float64)
    q[:, :, 0] = 1
    q[:, :, 1] = 1
    w = np.ones((3, H), dtype=np.float32)
    pos = np.array([N - 1, N + 4, N - 1], dtype=np.int32)
    say(f"split-score boundary bucket: {sure} above, {bucket} in the boundary's high half, k={topk}")
    exact_case(lib, orc, synth.to_bits(q, "f16"), synth.to_bits(k, "f16"), w, pos, H=H, D=D,
               dtype="f16", ratio=ratio, topk=topk, where=f"bucket {sure}/{bucket} k={topk}")


@pytest.mark.parametrize("N,topk", [(8192, 512), (16384, 512), (5000, 100), (2048, 512)])
def test_concentrated_and_tied_rows_exact(lib, orc, N, topk):
    """64 index heads, rows of 2048..16384: scores rising with the row (every
    top row at the end of the row, against the sampled starting threshold),
    all-equal scores (a pure tie-break by row: the top rows all at the start),
    a ReLU that cuts every score to 0, and one token of ordinary integer data.
    Bit-exact against the oracle."""
    H, D, ratio = 64, 128, 1
    rng = np.random.default_rng(N + topk)
    kf = np.zeros((N, D))
    kf[:, 0] = np.floor(np.arange(N) / 8)                 # rising, exact in fp16 up to 2048
    kf[:, 1:] = rng.integers(-1, 2, size=(N, D - 1))
    qf = np.zeros((4, H, D))
    qf[0, :, 0] = 1                                       # rising scores
    qf[2, :, :] = rng.integers(-4, 5, size=(H, D))         # ordinary integer data
    qf[3, :, 0] = -1                                      # ReLU cuts everything: all scores 0
    w = np.ones((4, H), np.float32)
    w[2] = np.ldexp(1.0, -rng.integers(0, 4, size=H)).astype(np.float32)
    pos = np.array([N - 1, N - 1, N + 3, N - 1], np.int32)  # token 1: q = 0, all scores 0
    say(f"rising / ties / integer / relu-cut rows, N={N} k={topk}")
    exact_case(lib, orc, synth.to_bits(qf, "f16"), synth.to_bits(kf, "f16"), w, pos, H=H, D=D,
               dtype="f16", ratio=ratio, topk=topk, where=f"concentrated rows N={N} k={topk}")


def test_decode_at_the_row_limit(lib, orc):
    """Single-token decode at the most rows the decode path takes (2048 partitions
    of 512 rows = 1048576 rows, 256 MiB of K): the merge holds the 16384-key union
    of 8-key lists in its widest form.  Integer-valued inputs (many equal scores:
    the merge's histogram bin is crowded and the bisection decides) bit-exact, and
    Gaussian inputs (the histogram decides) within the tolerance."""
    N, H, D, topk = 1 << 20, 64, 128, 512
    rng = np.random.default_rng(20)
    say(f"decode at the row limit, integers, N={N}")
    q, k, w, _ = rand_int_case(rng, 1, N, H, D, -4, 4, 4, 1, "f16")
    for p in (4 * N - 1, 4 * (N // 2) + 1):
        out = gpu_run(lib, q, k, w, np.array([p], np.int32), H=H, D=D, dtype="f16", ratio=4,
                      topk=topk)
        want = orc.score_topk(q, k, w, np.array([p], np.int32), H=H, D=D, dtype="f16", ratio=4,
                              topk=topk, threads=16)
        assert np.array_equal(out, want), f"row limit, integers, pos {p}"
    say(f"decode at the row limit, gaussian, N={N}")
    q = synth.to_bits(rng.standard_normal((1, H, D)) / np.sqrt(128.0), "f16")
    k = synth.to_bits(rng.standard_normal((N, D)) / np.sqrt(128.0), "f16")
    w = rng.random((1, H), dtype=np.float32)
    pos = np.array([4 * N - 1], np.int32)
    out, sc = gpu_run(lib, q, k, w, pos, H=H, D=D, dtype="f16", ratio=4, topk=topk, scores=True)
    want, osc = orc.score_topk(q, k, w, pos, H=H, D=D, dtype="f16", ratio=4, topk=topk,
                               want_scores=True, threads=16)
    check_tolerant(out[0], sc[0], osc[0], N, topk, "row limit, gaussian")
