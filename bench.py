#!/usr/bin/env python3
"""Benchmark of the lightning indexer (score + top-k) on one MI355X.

One step = one ds_indexer_score_topk call over one 2048-token prefill chunk at
32k context (positions 30720..32767, ratio 4 -> 8192 compressed rows, 64 index
heads x 128, top-512, fp16 integer-valued synthetic inputs): the scorer
kernel, the skip path and the streaming top-k.  Inputs are resident in HBM
before the timed region.  The headline value is scored pairs per second
(sum over tokens of visible rows / step time); query tokens per second is
reported beside it.

The same run also times the 64k chunk (bf16 Gaussian, 16384 rows), the
single-token decode at the 1M window (262144 rows, 64 MiB of K streamed per
call, 8 distinct K buffers rotated so every call reads HBM rather than the
256 MB last-level cache) and the sparse attention that consumes the 32k
chunk's indices (2048 tokens x 64 heads over a 128-row local window plus 512
listed pooled rows each), and times the CPU oracle on a bounded token sample of
the headline workload.

Every workload is warmed up for at least --warmup calls AND at least
--warmup-ms milliseconds of back-to-back calls (the GPU needs some tens of
milliseconds of work to reach its steady clock, whatever the call count), and
the warm-up actually done is reported.  The step time is then taken over
exactly K calls between two device synchronisations, with nothing else on the
stream; a second pass of K calls with an event between consecutive calls gives
the median and minimum single-call time.  The per-kernel durations come from a
third pass of K calls in which the library has each of its kernels record HIP
events from its own dispatch (ds_indexer_timing: start of the first kernel of a
step, end of the last, on the call's stream); launches that carry events are
dispatched more slowly, so that pass's step time is reported apart.  The
headline workload is timed again at the end of the run as a bracketing control
(machine-speed drift between the first and the last measurement).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--warmup-ms M]
                       (defaults K = 50, W = 200, M = 300)
       python bench.py --only prefill32k|prefill64k|decode1m|prefill2k|decode1m_b8|qproj32k|attn32k|attn32k_r128
                                                                 (one workload, for profilers)
       python bench.py --phases WORKLOAD                        (per-phase durations from the
                       timestamped build, libds_indexer_stamps.so)
       python bench.py --copy-calibration                       (plain copy kernel, for counters)
       python bench.py --ceilings                               (vendor GEMM and plain-copy
                       rates with the workloads' value distributions)
       python bench.py --summarize-pmc DIR                      (fold rocprofv3 counter CSVs)
       python bench.py --summarize-trace DIR                    (kernel table of a rocprofv3 trace)
       python bench.py --summarize-mfma DIR                     (clock and MFMA use per kernel
                       from a rocprofv3 counter run)
       python bench.py --record-traffic WL FETCH WRITE CFETCH CWRITE
                       (HBM bytes per launch of WL's dominant kernel from counter runs)
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "indexer scored pairs/sec + query tokens/sec at 32k/64k context; decode HBM GB/s"
PEAK_MFMA_TFLOPS = {"f16": 2500.0, "bf16": 2500.0}  # MI355X dense fp16/bf16 MFMA
PEAK_HBM_GBS = 8000.0                               # MI355X HBM3E
HEADLINE = "prefill32k"
SECONDARY = ("prefill8k", "prefill64k", "decode1m", "prefill2k")
DECODE_K_BUFFERS = 8
KERNEL_SOURCES = {  # kernel class -> sources whose change invalidates stored counters
    "score": ["sparse_attention_kv_ds_amd/csrc/scorer.hip", "sparse_attention_kv_ds_amd/csrc/common.hpp"],
    "decode_score": ["sparse_attention_kv_ds_amd/csrc/scorer.hip", "sparse_attention_kv_ds_amd/csrc/common.hpp",
                     "sparse_attention_kv_ds_amd/csrc/select.hpp"],
    "attention": ["sparse_attention_kv_ds_amd/csrc/attention.hip", "sparse_attention_kv_ds_amd/csrc/common.hpp"],
    "project": ["sparse_attention_kv_ds_amd/csrc/qproj.hip", "sparse_attention_kv_ds_amd/csrc/common.hpp"],
    "select": ["sparse_attention_kv_ds_amd/csrc/topk.hip", "sparse_attention_kv_ds_amd/csrc/select.hpp",
               "sparse_attention_kv_ds_amd/csrc/common.hpp"],
}
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_counters.json")


def log(msg: str) -> None:
    print(msg, file=sys.stderr, flush=True)


def source_hash(cls: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[cls]:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def visible_pairs(wl) -> int:
    import numpy as np
    p = wl.positions.astype(np.int64)
    n = np.clip(np.where(p < 0, 0, (p + 1) // wl.ratio), 0, wl.N)
    return int(n.sum())


def upload(d, dev):
    import numpy as np
    import torch
    return (torch.from_numpy(d["q"].view(np.int16)).to(dev),
            torch.from_numpy(d["k"].view(np.int16)).to(dev),
            torch.from_numpy(d["w"]).to(dev),
            torch.from_numpy(d["pos"]).to(dev))


WARMUP_MS = 300.0  # default least warm-up time per workload


def warm_up(call, warmup: int, warmup_ms: float, dev):
    """At least `warmup` calls and at least `warmup_ms` of back-to-back calls
    (issued in chunks of about 10 ms between synchronisations); returns
    (calls, milliseconds) actually spent."""
    import torch
    torch.cuda.synchronize(dev)
    t0 = time.perf_counter()
    n, chunk = 0, 2
    while True:
        for _ in range(chunk):
            call(n)
            n += 1
        torch.cuda.synchronize(dev)
        el = (time.perf_counter() - t0) * 1e3
        if n >= warmup and el >= warmup_ms:
            return n, el
        chunk = max(1, min(2000, int(10.0 / max(el / n, 1e-3))))


def timed_calls(call, steps: int, dev, first: int = 0):
    """Exactly `steps` calls between two device synchronisations; the average
    milliseconds per call from events around them."""
    import torch
    a = torch.cuda.Event(enable_timing=True)
    b = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize(dev)
    a.record()
    for i in range(steps):
        call(first + i)
    b.record()
    torch.cuda.synchronize(dev)
    return a.elapsed_time(b) / steps


def per_call_stats(call, steps: int, dev):
    """`steps` calls with an event between consecutive calls: the median and the
    minimum of the single-call durations (each includes one event record)."""
    import statistics

    import torch
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize(dev)
    ev[0].record()
    for i in range(steps):
        call(i)
        ev[i + 1].record()
    torch.cuda.synchronize(dev)
    d = [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]
    return {"median_ms": statistics.median(d), "min_ms": min(d), "max_ms": max(d)}


def time_workload(name: str, steps: int, warmup: int, warmup_ms: float = WARMUP_MS):
    """Time `steps` calls of one workload; returns a result dict."""
    import torch
    from sparse_attention_kv_ds_amd import synth
    from sparse_attention_kv_ds_amd.indexer import Indexer

    dev = torch.device("cuda", 0)
    d = synth.make(name)
    wl = d["wl"]
    q, k, w, pos = upload(d, dev)
    ks = [k]
    if wl.T == 1:  # decode: rotate distinct K buffers (> last-level cache) so reads hit HBM
        ks += [torch.roll(k, shifts=997 * (i + 1), dims=0).contiguous()
               for i in range(DECODE_K_BUFFERS - 1)]
    out = torch.empty((wl.T, wl.topk), dtype=torch.int32, device=dev)
    ix = Indexer(wl.H, wl.D, wl.dtype, wl.topk, wl.T, wl.N, device=0)

    def call(i):
        ix.score_topk(q, ks[i % len(ks)], w, pos, wl.ratio, wl.topk, out=out)

    try:
        nw, wms = warm_up(call, warmup, warmup_ms, dev)
        # the step time without per-kernel events (launches that record them are
        # dispatched more slowly) ...
        ms = timed_calls(call, steps, dev)
        stats = per_call_stats(call, steps, dev)
        # ... then the same steps again with the kernels recording HIP events from
        # their own dispatch, for the kernel durations
        ix.timing(True)
        ix.timing_read()
        ms_marked = timed_calls(call, steps, dev)
        per = ix.timing_read()
        stream_only = None
        if wl.T == 1:
            # the decode stream alone: the same scorer without its partition
            # lists, as ds_indexer_scores runs it (its kernel timed the same way)
            srow = torch.empty((1, wl.N), dtype=torch.float32, device=dev)
            timed_calls(lambda i: ix.scores(q, ks[i % len(ks)], w, pos, wl.ratio, out=srow),
                        steps, dev)
            st_per = ix.timing_read()
            stream_only = st_per["decode_score"][0] / max(st_per["decode_score"][1], 1)
        ix.timing(False)
    finally:
        ix.close()
    kernels = {c: {"avg_ms": v[0] / v[1], "launches": v[1]} for c, v in per.items() if v[1]}
    pairs = visible_pairs(wl)
    res = {"workload": name, "ms_per_step": ms, "ms_per_step_with_markers": ms_marked,
           "step_stats": stats, "warmup_calls": nw, "warmup_ms": wms,
           "pairs": pairs, "tokens": wl.T,
           "pairs_per_s": pairs / (ms * 1e-3), "query_tokens_per_s": wl.T / (ms * 1e-3),
           "kernels": kernels, "wl": wl, "stream_only_ms": stream_only}
    log(f"[bench] {name}: {ms * 1e3:.1f} us/step (median {stats['median_ms'] * 1e3:.1f}, "
        f"min {stats['min_ms'] * 1e3:.1f}; {ms_marked * 1e3:.1f} with kernel markers; "
        f"warm-up {nw} calls, {wms:.0f} ms), "
        + ", ".join(f"{c} {v['avg_ms'] * 1e3:.1f} us" for c, v in kernels.items()))
    return res


ATTN_WORKLOAD = "attn32k"
ATTN_SECONDARY = ("attn32k_r128",)


DECODE_BATCH = "decode1m_b8"
PROJECTION = "qproj32k"


def time_projection(name: str, steps: int, warmup: int, warmup_ms: float = WARMUP_MS):
    """Time `steps` calls of the query projection fused ahead of the indexer on
    the 32k chunk (projection, then score + top-k, in one call)."""
    import numpy as np
    import torch
    from sparse_attention_kv_ds_amd import synth
    from sparse_attention_kv_ds_amd.indexer import Indexer

    dev = torch.device("cuda", 0)
    d = synth.make_projection(name)
    wl = d["wl"]
    up = {kk: torch.from_numpy(np.ascontiguousarray(d[kk]).view(np.int16)).to(dev)
          for kk in ("x", "wq", "k")}
    w = torch.from_numpy(d["w"]).to(dev)
    pos = torch.from_numpy(d["pos"]).to(dev)
    out = torch.empty((wl.T, wl.topk), dtype=torch.int32, device=dev)
    ix = Indexer(wl.H, wl.D, d["dtype"], wl.topk, wl.T, wl.N, device=0)

    def call(i):
        ix.project_score_topk(up["x"], up["wq"], up["k"], w, pos, wl.ratio, wl.topk, out=out)

    try:
        nw, wms = warm_up(call, warmup, warmup_ms, dev)
        ms = timed_calls(call, steps, dev)
        stats = per_call_stats(call, steps, dev)
        ix.timing(True)
        ix.timing_read()
        ms_marked = timed_calls(call, steps, dev)
        per = ix.timing_read()
        ix.timing(False)
    finally:
        ix.close()
    kernels = {c: v[0] / v[1] for c, v in per.items() if v[1]}
    flops = 2.0 * wl.T * d["din"] * wl.H * wl.D
    ach = flops / (kernels["project"] * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[d["dtype"]]
    log(f"[bench] {name}: {ms * 1e3:.1f} us/call ({ms_marked * 1e3:.1f} with kernel markers), "
        + ", ".join(f"{c} {v * 1e3:.1f} us" for c, v in kernels.items())
        + f"; projection {ach:.0f} TFLOP/s ({ach / peak * 100:.1f} % of {d['dtype']} MFMA peak)")
    return {"workload": name, "dtype": d["dtype"], "ms_per_step": ms,
            "ms_per_step_with_markers": ms_marked, "step_stats": stats, "warmup_calls": nw,
            "warmup_ms": wms, "kernels_ms": kernels,
            "value": wl.T / (ms * 1e-3), "unit": "query tokens/s (projection + score + top-k)",
            "roofline": {"bound": "mfma", "kernel": "qproj", "achieved": ach, "peak": peak,
                         "unit": "TFLOP/s", "frac": ach / peak,
                         "traffic": stored_traffic("project", name),
                         "algorithmic_flops_per_launch": flops}}


def time_decode_batch(name: str, steps: int, warmup: int, warmup_ms: float = WARMUP_MS):
    """Time `steps` batched decode calls (B sequences of 262144 rows: 512 MiB of K,
    above the last-level cache, so every call streams K from HBM)."""
    import numpy as np
    import torch
    from sparse_attention_kv_ds_amd import synth
    from sparse_attention_kv_ds_amd.indexer import Indexer

    dev = torch.device("cuda", 0)
    d = synth.make_decode_batch(name)
    wl, B = d["wl"], d["B"]
    q = torch.from_numpy(np.ascontiguousarray(d["q"]).view(np.int16)).to(dev)
    k = torch.from_numpy(np.ascontiguousarray(d["k"]).view(np.int16)).to(dev)
    w = torch.from_numpy(d["w"]).to(dev)
    pos = torch.from_numpy(d["pos"]).to(dev)
    out = torch.empty((B, wl.topk), dtype=torch.int32, device=dev)
    ix = Indexer(wl.H, wl.D, wl.dtype, wl.topk, B, wl.N, device=0)

    def call(i):
        ix.score_topk_batch(q, k, w, pos, wl.ratio, wl.topk, out=out)

    try:
        nw, wms = warm_up(call, warmup, warmup_ms, dev)
        ms = timed_calls(call, steps, dev)
        stats = per_call_stats(call, steps, dev)
        ix.timing(True)
        ix.timing_read()
        ms_marked = timed_calls(call, steps, dev)
        per = ix.timing_read()
        ix.timing(False)
    finally:
        ix.close()
    kernels = {c: v[0] / v[1] for c, v in per.items() if v[1]}
    algo = B * (wl.N * wl.D * 2 + wl.H * wl.D * 2 + wl.H * 4 + wl.topk * 4)
    t = kernels["decode_score"] * 1e-3
    ach = algo / t / 1e9
    log(f"[bench] {name}: {ms * 1e3:.1f} us/call for {B} sequences ({ms_marked * 1e3:.1f} with "
        f"kernel markers), " + ", ".join(f"{c} {v * 1e3:.1f} us" for c, v in kernels.items())
        + f"; scorer {ach:.0f} GB/s ({ach / PEAK_HBM_GBS * 100:.1f} % of HBM)")
    return {"workload": name, "dtype": wl.dtype, "sequences": B, "ms_per_step": ms,
            "ms_per_step_with_markers": ms_marked, "step_stats": stats, "warmup_calls": nw,
            "warmup_ms": wms, "kernels_ms": kernels,
            "value": algo / (ms * 1e-3) / 1e9, "unit": "GB/s (whole batched decode call, K from HBM)",
            "sequences_per_s": B / (ms * 1e-3),
            "roofline": {"bound": "hbm", "kernel": "decode_scorer (batched)", "achieved": ach,
                         "peak": PEAK_HBM_GBS, "unit": "GB/s", "frac": ach / PEAK_HBM_GBS,
                         "traffic": stored_traffic("decode_score", name),
                         "algorithmic_bytes_per_launch": algo}}


def time_attention(name: str, steps: int, warmup: int, warmup_ms: float = WARMUP_MS):
    """Time `steps` calls of the sparse attention (one kernel per call) on one
    workload; the duration of a call is events around back-to-back calls on
    the stream the kernel runs on."""
    import numpy as np
    import torch
    from sparse_attention_kv_ds_amd import synth
    from sparse_attention_kv_ds_amd.indexer import sparse_attention, sparse_attention_all

    dev = torch.device("cuda", 0)
    d = synth.make_attention(name)
    wl = d["wl"]
    t = {k: torch.from_numpy(np.ascontiguousarray(d[k]).view(np.int16)).to(dev)
         for k in ("q", "kp", "vp", "kl", "vl")}
    idx = torch.from_numpy(d["idx"]).to(dev)
    pos = torch.from_numpy(d["pos"]).to(dev)
    out = torch.empty((wl.T, wl.HA, wl.DV), dtype=torch.float32, device=dev)

    def call(i):
        if wl.ratio > 0:  # every visible pooled row, no index list
            sparse_attention_all(t["q"], t["kp"], t["vp"], t["kl"], t["vl"], pos, ratio=wl.ratio,
                                 window=wl.window, scale=wl.scale, dtype=wl.dtype, out=out)
        else:
            sparse_attention(t["q"], t["kp"], t["vp"], t["kl"], t["vl"], idx, pos,
                             window=wl.window, scale=wl.scale, dtype=wl.dtype, out=out)

    nw, wms = warm_up(call, warmup, warmup_ms, dev)
    ms = timed_calls(call, steps, dev)
    stats = per_call_stats(call, steps, dev)
    # rows attended per token: the local window (clamped to positions 0..L-1)
    # plus the listed pooled rows
    p = wl.positions.astype(np.int64)
    lo = np.maximum(0, p - wl.window + 1)
    hi = np.minimum(p, wl.L - 1)
    n_loc = np.where((p >= 0) & (wl.window > 0), np.maximum(0, hi - lo + 1), 0)
    if wl.ratio > 0:
        n_pool = np.clip((p + 1) // wl.ratio, 0, wl.N)
    else:
        n_pool = ((d["idx"] >= 0) & (d["idx"] < wl.N)).sum(axis=1)
    rows = int((n_loc + n_pool).sum())
    flops = 2.0 * wl.HA * (wl.DK + wl.DV) * rows
    ach = flops / (ms * 1e-3) / 1e12
    peak = PEAK_MFMA_TFLOPS[wl.dtype]
    byt = (wl.T * wl.HA * wl.DK * 2 + wl.N * (wl.DK + wl.DV) * 2 + wl.L * (wl.DK + wl.DV) * 2
           + d["idx"].nbytes + wl.T * 4 + wl.T * wl.HA * wl.DV * 4)
    log(f"[bench] {name}: {ms * 1e3:.1f} us/call, {rows / wl.T:.0f} rows per token, "
        f"{ach:.0f} TFLOP/s ({ach / peak * 100:.1f} % of {wl.dtype} MFMA peak)")
    return {"workload": name, "dtype": wl.dtype, "ms_per_step": ms, "step_stats": stats,
            "warmup_calls": nw, "warmup_ms": wms,
            "value": wl.T / (ms * 1e-3), "unit": "query tokens/s",
            "rows_attended_per_token": rows / wl.T,
            "roofline": {"bound": "mfma", "kernel": "sparse_attention", "achieved": ach,
                         "peak": peak, "unit": "TFLOP/s", "frac": ach / peak,
                         "traffic": stored_traffic("attention", name) if name in DOMINANT else None,
                         "algorithmic_flops_per_launch": flops,
                         "input_output_bytes_per_launch": byt}}


def stored_traffic(cls: str, workload: str):
    """HBM bytes per launch from committed counter runs, if the kernel is unchanged."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    with open(TRAFFIC_FILE) as f:
        rec = json.load(f).get(f"{cls}:{workload}")
    if not rec or rec.get("source_hash") != source_hash(cls):
        return None
    return rec.get("hbm_bytes_per_launch")


def roofline(res):
    wl = res["wl"]
    if "score" not in res["kernels"] and "decode_score" not in res["kernels"]:
        # every row fits (N <= topk): only the sequential-rows kernel runs
        cls = "select" if wl.T > 1 else "decode_select"
        t = res["kernels"][cls]["avg_ms"] * 1e-3
        algo = wl.T * wl.topk * 4 + wl.T * 4  # out written, pos read
        ach = algo / t / 1e9
        return {"bound": "hbm", "kernel": "sequential_rows", "achieved": ach, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": ach / PEAK_HBM_GBS, "traffic": None,
                "algorithmic_bytes_per_launch": algo}
    if wl.T == 1:
        cls = "decode_score"
        t = res["kernels"][cls]["avg_ms"] * 1e-3
        # K streamed once + q + w + out (algorithmic bytes of one call)
        algo = wl.N * wl.D * 2 + wl.H * wl.D * 2 + wl.H * 4 + wl.topk * 4
        ach = algo / t / 1e9
        return {"bound": "hbm", "kernel": "decode_scorer", "achieved": ach, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": ach / PEAK_HBM_GBS, "traffic": stored_traffic(cls, res["workload"]),
                "algorithmic_bytes_per_launch": algo}
    cls = "score"
    t = res["kernels"][cls]["avg_ms"] * 1e-3
    flops = 2.0 * wl.H * wl.D * res["pairs"]
    ach = flops / t / 1e12
    peak = PEAK_MFMA_TFLOPS[wl.dtype]
    return {"bound": "mfma", "kernel": "prefill_scorer", "achieved": ach, "peak": peak,
            "unit": "TFLOP/s", "frac": ach / peak, "traffic": stored_traffic(cls, res["workload"]),
            "algorithmic_flops_per_launch": flops}


def cpu_threads():
    """(host cores this process may run on, threads the oracle uses): every core of
    the affinity mask, or the process's CPU share when OMP_NUM_THREADS sets a
    smaller one (a GPU machine hands each GPU's jobs a share of its cores)."""
    try:
        host = len(os.sched_getaffinity(0))
    except AttributeError:
        host = os.cpu_count() or 1
    share = os.environ.get("OMP_NUM_THREADS", "")
    threads = min(host, int(share)) if share.isdigit() and int(share) > 0 else host
    return host, max(1, threads)


def oracle_rate(name: str, threads: int, budget_s: float):
    """The oracle, as it stands, on `threads` threads over an evenly spaced token
    sample of one workload, repeated until about `budget_s` seconds have passed:
    (pairs/s, tokens in the sample, passes, pairs, seconds)."""
    import numpy as np
    from oracle import oracle
    from sparse_attention_kv_ds_amd import synth

    d = synth.make(name)
    wl = d["wl"]
    orc = oracle.load()
    p = wl.positions.astype(np.int64)
    n_t = np.clip((p + 1) // wl.ratio, 0, wl.N)

    def run(toks):
        t = time.perf_counter()
        orc.score_topk(d["q"], d["k"], d["w"], d["pos"], H=wl.H, D=wl.D, dtype=wl.dtype,
                       ratio=wl.ratio, topk=wl.topk, tokens=toks, threads=threads)
        return time.perf_counter() - t

    probe = np.linspace(0, wl.T - 1, min(wl.T, 2 * threads)).astype(np.int64)
    tp = run(probe)
    count = int(min(wl.T, max(len(probe), len(probe) * budget_s / max(tp, 1e-3))))
    toks = np.linspace(0, wl.T - 1, count).astype(np.int64)
    el, reps = 0.0, 0
    while reps == 0 or el < budget_s:
        el += run(toks)
        reps += 1
    pairs = int(n_t[toks].sum()) * reps
    return pairs / el, count, reps, pairs, el


def cpu_baseline(name: str, budget_s: float = 12.0):
    """The oracle on the host's CPU share over a bounded sample of the headline
    workload, plus 1-thread runs on the tiny, 8k and decode workloads."""
    host, threads = cpu_threads()
    from sparse_attention_kv_ds_amd import synth
    T = synth.WORKLOADS[name].T
    rate, count, reps, pairs, el = oracle_rate(name, threads, budget_s)
    log(f"[bench] cpu oracle: {count} tokens x {reps}, {pairs} pairs in {el:.2f} s on {threads} "
        f"threads ({host} host cores)")
    single = {}
    for wname, b in (("tiny", 1.0), ("prefill8k", 4.0), ("decode1m", 1.0)):
        r1, c1, n1, p1, e1 = oracle_rate(wname, 1, b)
        single[wname] = {"value": r1, "unit": "pairs/s", "sample_tokens": c1, "passes": n1,
                         "pairs": p1, "seconds": e1}
        log(f"[bench] cpu oracle, 1 thread: {wname} {r1:.3g} pairs/s ({c1} tokens x {n1})")
    return {"value": rate, "unit": "pairs/s", "cores": threads, "host_cores": host,
            "kind": "oracle",
            "sample": f"{count} of {T} query tokens of {name} (evenly spaced), {reps} pass(es), "
                      f"{pairs} scored pairs, fp64 scoring + full sort, {el:.1f} s wall on "
                      f"{threads} threads",
            "threads_rule": "every core of the affinity mask, or the CPU share OMP_NUM_THREADS "
                            "sets when smaller",
            "single_thread": single}


def copy_calibration(mib: int = 512, reps: int = 3):
    """A plain device copy of known size, for scaling memory counters."""
    import torch
    dev = torch.device("cuda", 0)
    a = torch.empty(mib * 2**20 // 4, dtype=torch.float32, device=dev).fill_(1.0)
    b = torch.empty_like(a)
    torch.cuda.synchronize(dev)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize(dev)
    print(json.dumps({"copy_bytes_read": a.numel() * 4, "copy_bytes_written": b.numel() * 4,
                      "reps": reps}))


def ceilings(reps: int = 20):
    """Reference rates on this GPU with the workloads' value distributions:
    a vendor (hipBLASLt, through torch.matmul) dense 8192^3 GEMM on
    integer-valued fp16 operands and on Gaussian fp16 / bf16 operands (the
    matrix cores draw more power on random mantissas and the clock drops),
    a plain device copy of 64 MiB (torch copy_ over 8 rotating buffer
    pairs, so that every pass reads and writes HBM), and plain reads of 64 MiB
    and 512 MiB (torch sum).  Times are events around back-to-back launches on
    one stream."""
    import torch
    dev = torch.device("cuda", 0)
    g = torch.Generator(device=dev).manual_seed(0)
    n = 8192
    out = {}

    def timed(fn, k):
        for _ in range(3):
            fn(0)
        torch.cuda.synchronize(dev)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for i in range(k):
            fn(i)
        b.record()
        torch.cuda.synchronize(dev)
        return a.elapsed_time(b) / k * 1e-3

    cases = {
        "gemm_f16_integers": lambda: torch.randint(-4, 5, (n, n), device=dev, generator=g).to(torch.float16),
        "gemm_f16_gaussian": lambda: (torch.randn(n, n, device=dev, generator=g) / 128 ** 0.5).to(torch.float16),
        "gemm_bf16_gaussian": lambda: (torch.randn(n, n, device=dev, generator=g) / 128 ** 0.5).to(torch.bfloat16),
    }
    for name, make in cases.items():
        x, y = make(), make()
        # warm the clock with some tens of ms of work, then time
        t = timed(lambda i: torch.matmul(x, y), reps)
        t = timed(lambda i: torch.matmul(x, y), reps)
        tf = 2.0 * n ** 3 / t / 1e12
        out[name] = {"tflops": tf, "frac_of_2500": tf / PEAK_MFMA_TFLOPS["f16"]}
        log(f"[ceilings] {name}: {tf:.0f} TFLOP/s ({tf / PEAK_MFMA_TFLOPS['f16'] * 100:.1f} % of 2.5 PFLOP/s)")
        del x, y
    src = [torch.randn(32 * 2 ** 20, device=dev, generator=g).to(torch.float16) for _ in range(8)]
    dst = [torch.empty_like(src[0]) for _ in range(8)]
    t = timed(lambda i: dst[i % 8].copy_(src[(i + 3) % 8]), 8 * reps)
    gbs = 2 * 64 * 2 ** 20 / t / 1e9
    out["copy_64MiB"] = {"GBps_read_plus_write": gbs, "frac_of_8000": gbs / PEAK_HBM_GBS, "us": t * 1e6}
    log(f"[ceilings] device copy of 64 MiB (torch copy_, 8 rotating buffer pairs): {t * 1e6:.1f} us, "
        f"{gbs:.0f} GB/s read + write ({gbs / PEAK_HBM_GBS * 100:.1f} % of 8 TB/s)")
    # read-only: a vendor reduction (torch sum into float32) over one 64 MiB
    # buffer per call (8 rotating buffers, the single-sequence decode's K), and
    # over 512 MiB in one call (the eight-sequence decode's K)
    acc = torch.empty((), dtype=torch.float32, device=dev)
    t = timed(lambda i: torch.sum(src[i % 8], dim=0, dtype=torch.float32, out=acc), 8 * reps)
    gbs = 64 * 2 ** 20 / t / 1e9
    out["read_64MiB"] = {"GBps": gbs, "frac_of_8000": gbs / PEAK_HBM_GBS, "us": t * 1e6}
    log(f"[ceilings] read of 64 MiB (torch sum, 8 rotating buffers): {t * 1e6:.1f} us, "
        f"{gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS * 100:.1f} % of 8 TB/s)")
    del dst
    big = torch.cat(src)
    del src
    t = timed(lambda i: torch.sum(big, dim=0, dtype=torch.float32, out=acc), reps)
    gbs = 512 * 2 ** 20 / t / 1e9
    out["read_512MiB"] = {"GBps": gbs, "frac_of_8000": gbs / PEAK_HBM_GBS, "us": t * 1e6}
    log(f"[ceilings] read of 512 MiB (torch sum, one buffer): {t * 1e6:.1f} us, "
        f"{gbs:.0f} GB/s ({gbs / PEAK_HBM_GBS * 100:.1f} % of 8 TB/s)")
    print(json.dumps(out))


def summarize_pmc(directory: str):
    """Average per-dispatch counter values per kernel from rocprofv3 counter CSVs."""
    rows = []
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            rows += list(csv.DictReader(f))
    acc = {}
    for r in rows:
        name = r.get("Kernel_Name", "?")
        key = (name, r.get("Counter_Name", "?"))
        acc.setdefault(key, {})
        acc[key].setdefault(r.get("Dispatch_Id", "0"), 0.0)
        acc[key][r.get("Dispatch_Id", "0")] += float(r.get("Counter_Value", 0.0))
    out = {}
    for (name, ctr), per in sorted(acc.items()):
        vals = list(per.values())
        out.setdefault(name, {})[ctr] = {"dispatches": len(vals), "avg": sum(vals) / len(vals)}
    print(json.dumps(out, indent=1))


def summarize_mfma(directory: str):
    """Clock and matrix-core use per dispatch of the scorer kernels from a
    rocprofv3 counter run with GRBM_GUI_ACTIVE (summed over the 8 XCDs),
    SQ_VALU_MFMA_BUSY_CYCLES (summed over the 1024 SIMDs) and the MFMA op
    counters (units of 512 flops): clock = GUI-active cycles per XCD / the
    dispatch's duration; busy = MFMA-busy cycles per SIMD / GUI-active cycles
    per XCD; flops from the op counters; rate = flops / duration."""
    import statistics
    per = {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                key = (r["Kernel_Name"], r["Dispatch_Id"])
                d = per.setdefault(key, {})
                d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
                d["dur_ns"] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    rows = {}
    for (name, _), d in per.items():
        if "GRBM_GUI_ACTIVE" not in d or "SQ_VALU_MFMA_BUSY_CYCLES" not in d or d["dur_ns"] <= 0:
            continue
        gui = d["GRBM_GUI_ACTIVE"] / 8.0
        mops = d.get("SQ_INSTS_VALU_MFMA_MOPS_F16", 0.0) + d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0)
        rows.setdefault(name, []).append({
            "dur_us": d["dur_ns"] / 1e3, "clock_ghz": gui / d["dur_ns"],
            "mfma_busy": d["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024.0 / gui if gui else 0.0,
            "tflops": mops * 512.0 / (d["dur_ns"] * 1e-9) / 1e12,
            "coexec": d.get("SQ_VALU_MFMA_COEXEC_CYCLES", 0.0) / max(d["SQ_VALU_MFMA_BUSY_CYCLES"], 1.0)})
    print("| kernel | dispatches | median duration us | clock GHz | MFMA busy | MFMA TFLOP/s (counted ops) | VALU co-issued with MFMA |")
    print("|---|---|---|---|---|---|---|")
    for name, v in sorted(rows.items()):
        if not any(x["mfma_busy"] > 0 for x in v):
            continue
        med = {k: statistics.median(x[k] for x in v) for k in v[0]}
        print(f"| `{name[:90]}` | {len(v)} | {med['dur_us']:.1f} | {med['clock_ghz']:.2f} | "
              f"{med['mfma_busy'] * 100:.1f} % | {med['tflops']:.0f} | {med['coexec'] * 100:.0f} % of busy cycles |")


def _pmc_table(directory: str):
    """{kernel name: {counter: average per dispatch}} from rocprofv3 counter CSVs."""
    acc = {}
    for path in glob.glob(os.path.join(directory, "**", "*counter_collection.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                key = (r.get("Kernel_Name", "?"), r.get("Counter_Name", "?"))
                per = acc.setdefault(key, {})
                did = r.get("Dispatch_Id", "0")
                per[did] = per.get(did, 0.0) + float(r.get("Counter_Value", 0.0))
    out = {}
    for (name, ctr), per in acc.items():
        out.setdefault(name, {})[ctr] = sum(per.values()) / len(per)
    return out


DOMINANT = {"decode1m": ("decode_score", "decode_scorer_kernel"),
            "prefill8k": ("score", "prefill_scorer_kernel"),
            "prefill32k": ("score", "prefill_scorer_kernel"),
            "prefill64k": ("score", "prefill_scorer_kernel"),
            "attn32k": ("attention", "sparse_attention_kernel"),
            "attn32k_r128": ("attention", "sparse_attention_kernel"),
            "decode1m_b8": ("decode_score", "decode_scorer_kernel"),
            "qproj32k": ("project", "qproj_kernel"),
            # the prefill top-k of the same runs (for the record, not a bench roofline)
            "prefill8k_select": ("select", "topk_stream_kernel"),
            "prefill32k_select": ("select", "topk_stream_kernel"),
            "prefill64k_select": ("select", "topk_stream_kernel")}


def record_traffic(workload: str, fetch_dir: str, write_dir: str, copy_fetch: str, copy_write: str):
    """HBM bytes per launch of the workload's dominant kernel from FETCH_SIZE and
    WRITE_SIZE runs (KiB per dispatch), each scaled by what the same counter
    reads for the plain 512 MiB copy of --copy-calibration; stored in
    profiles/traffic_counters.json with the hash of the kernel's sources."""
    cls, needle = DOMINANT[workload]
    expect_kib = 512 * 1024.0

    def pick(directory, counter, match):
        tab = _pmc_table(directory)
        cands = [(n, v[counter]) for n, v in tab.items() if counter in v and match(n)]
        if not cands:
            raise SystemExit(f"no {counter} for the kernel in {directory}")
        return max(cands, key=lambda x: x[1])

    _, cf = pick(copy_fetch, "FETCH_SIZE", lambda n: True)
    _, cw = pick(copy_write, "WRITE_SIZE", lambda n: True)
    kname, f = pick(fetch_dir, "FETCH_SIZE", lambda n: needle in n)
    _, wr = pick(write_dir, "WRITE_SIZE", lambda n: needle in n)
    ff, wf = expect_kib / cf, expect_kib / cw
    rec = {"kernel": kname, "source_hash": source_hash(cls),
           "fetch_kib_per_dispatch": f, "write_kib_per_dispatch": wr,
           "copy_fetch_kib": cf, "copy_write_kib": cw, "fetch_scale": ff, "write_scale": wf,
           "hbm_bytes_per_launch": (f * ff + wr * wf) * 1024.0}
    data = {}
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            data = json.load(fh)
    data[f"{cls}:{workload}"] = rec
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(data, fh, indent=1, sort_keys=True)
        fh.write("\n")
    print(json.dumps(rec, indent=1))


def summarize_trace(directory: str):
    """Per-kernel calls and durations (us) from a rocprofv3 --kernel-trace run
    (its SQLite database, or its *kernel_stats.csv)."""
    import sqlite3
    rows = []
    for db in glob.glob(os.path.join(directory, "**", "*.db"), recursive=True):
        con = sqlite3.connect(db)
        q = ("select name, count(*), sum(duration), avg(duration), min(duration), max(duration), "
             "max(grid_x), max(grid_y), max(workgroup_x), max(vgpr_count), max(accum_vgpr_count), "
             "max(lds_size) from kernels group by name")
        for r in con.execute(q):
            rows.append((r[0], int(r[1]), r[2] / 1e3, r[3] / 1e3, r[4] / 1e3, r[5] / 1e3,
                         f"{r[6]}x{r[7]}", r[8], r[9], r[10], r[11]))
    for path in glob.glob(os.path.join(directory, "**", "*kernel_stats.csv"), recursive=True):
        with open(path) as f:
            for r in csv.DictReader(f):
                rows.append((r["Name"], int(r["Calls"]), float(r["TotalDurationNs"]) / 1e3,
                             float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                             float(r["MaxNs"]) / 1e3, "", "", "", "", ""))
    print("| kernel | calls | total us | avg us | min us | max us | grid (threads) | wg | vgpr | agpr | lds B |")
    print("|---|---|---|---|---|---|---|---|---|---|---|")
    for r in sorted(rows, key=lambda r: -r[2]):
        print(f"| `{r[0][:100]}` | {r[1]} | {r[2]:.1f} | {r[3]:.2f} | {r[4]:.2f} | {r[5]:.2f} | "
              f"{r[6]} | {r[7]} | {r[8]} | {r[9]} | {r[10]} |")


def phases(name: str, warmup_ms: float = WARMUP_MS):
    """Per-phase durations of one workload's kernels, from the timestamped build
    of the library (libds_indexer_stamps.so, selected through DS_INDEXER_LIB
    before the binding loads; its kernels record the GPU's 100 MHz real-time
    counter at the phase boundaries listed in ds_indexer.h).  After the warm-up,
    three calls are taken one at a time and their records read back; each line
    gives a phase's 10th percentile / median / 90th percentile / maximum over
    the work-groups or tokens, in microseconds."""
    import ctypes
    import numpy as np
    import torch
    from sparse_attention_kv_ds_amd import indexer, synth

    if os.path.basename(indexer.LIB_PATH) != "libds_indexer_stamps.so":
        raise SystemExit("--phases needs the stamps build (DS_INDEXER_LIB)")
    dev = torch.device("cuda", 0)
    rec = np.zeros(4096 * 8, dtype=np.uint64)

    def read(unit):
        st = indexer.ds_indexer_stamps_read(unit, rec.ctypes.data, rec.nbytes)
        assert st == indexer.DS_OK, st
        return rec.reshape(4096, 8).astype(np.int64)

    def pct(x):
        x = np.asarray(x, dtype=np.float64) / 100.0  # 100 MHz ticks -> us
        return [round(float(v), 2) for v in (np.percentile(x, 10), np.median(x),
                                              np.percentile(x, 90), x.max())]

    out = {"workload": name, "unit": "us (p10, median, p90, max)", "calls": []}
    if name in (ATTN_WORKLOAD, *ATTN_SECONDARY):
        from sparse_attention_kv_ds_amd.indexer import sparse_attention, sparse_attention_all
        d = synth.make_attention(name)
        wl = d["wl"]
        t = {k: torch.from_numpy(np.ascontiguousarray(d[k]).view(np.int16)).to(dev)
             for k in ("q", "kp", "vp", "kl", "vl")}
        idx = torch.from_numpy(d["idx"]).to(dev)
        pos = torch.from_numpy(d["pos"]).to(dev)
        o = torch.empty((wl.T, wl.HA, wl.DV), dtype=torch.float32, device=dev)

        def call(i):
            if wl.ratio > 0:
                sparse_attention_all(t["q"], t["kp"], t["vp"], t["kl"], t["vl"], pos,
                                     ratio=wl.ratio, window=wl.window, scale=wl.scale,
                                     dtype=wl.dtype, out=o)
            else:
                sparse_attention(t["q"], t["kp"], t["vp"], t["kl"], t["vl"], idx, pos,
                                 window=wl.window, scale=wl.scale, dtype=wl.dtype, out=o)
        warm_up(call, 20, warmup_ms, dev)
        for c in range(3):
            call(0)
            r = read(indexer.DS_STAMPS_ATTENTION)[:wl.T]
            t0 = r[:, 0].min()
            nb = np.ceil(np.minimum(wl.window, wl.positions + 1) / 32) + np.ceil(
                (wl.topk if wl.ratio == 0 else np.minimum(np.maximum((wl.positions + 1) // max(wl.ratio, 1), 0), wl.N)) / 32)
            mid = np.linspace(0, (r[:, 3] - t0).max(), 64)
            inflight = [int(((r[:, 0] - t0 <= x) & (r[:, 3] - t0 > x)).sum()) for x in mid[8:56]]
            out["calls"].append({
                "start": pct(r[:, 0] - t0), "first_block": pct(r[:, 1] - r[:, 0]),
                "blocks": pct(r[:, 2] - r[:, 1]), "per_block": pct((r[:, 2] - r[:, 1]) / nb),
                "output": pct(r[:, 3] - r[:, 2]), "token": pct(r[:, 3] - r[:, 0]),
                "end": pct(r[:, 3] - t0), "tokens_in_flight_median": int(np.median(inflight))})
    else:
        from sparse_attention_kv_ds_amd.indexer import Indexer
        d = synth.make(name)
        wl = d["wl"]
        q, k, w, pos = upload(d, dev)
        ks = [k]
        if wl.T == 1:
            ks += [torch.roll(k, shifts=997 * (i + 1), dims=0).contiguous()
                   for i in range(DECODE_K_BUFFERS - 1)]
        o = torch.empty((wl.T, wl.topk), dtype=torch.int32, device=dev)
        ix = Indexer(wl.H, wl.D, wl.dtype, wl.topk, wl.T, wl.N, device=0)

        def call(i):
            ix.score_topk(q, ks[i % len(ks)], w, pos, wl.ratio, wl.topk, out=o)
        try:
            warm_up(call, 20, warmup_ms, dev)
            for c in range(3):
                call(c)
                if wl.T == 1:
                    n = min(max((int(wl.positions[0]) + 1) // wl.ratio, 0), wl.N)
                    P = (n + 511) // 512
                    r = read(indexer.DS_STAMPS_DECODE_SCORE)[:P]
                    m = read(indexer.DS_STAMPS_MERGE)[0]
                    t0 = r[:, 0].min()
                    se = r[:, 2:6].max(axis=1)
                    out["calls"].append({
                        "scorer_start": pct(r[:, 0] - t0), "first_blocks": pct(r[:, 1] - r[:, 0]),
                        "stream": pct(se - r[:, 1]), "partition_list": pct(r[:, 6] - se),
                        "scorer_end": pct(r[:, 6] - t0),
                        "merge": {"start_after_scorer_end": round((m[0] - r[:, 6].max()) / 100, 2),
                                  "load_lists": round((m[1] - m[0]) / 100, 2),
                                  "kth_key": round((m[2] - m[1]) / 100, 2),
                                  "check": round((m[3] - m[2]) / 100, 2),
                                  "output": round((m[4] - m[3]) / 100, 2)}})
                else:
                    n = np.clip((wl.positions.astype(np.int64) + 1) // wl.ratio, 0, wl.N)
                    sel = n > wl.topk
                    r = read(indexer.DS_STAMPS_TOPK)[:wl.T][sel]
                    t0 = r[:, 0].min()
                    out["calls"].append({
                        "tokens": int(sel.sum()), "start": pct(r[:, 0] - t0),
                        "starting_threshold": pct(r[:, 1] - r[:, 0]), "stream": pct(r[:, 2] - r[:, 1]),
                        "final_selection": pct(r[:, 3] - r[:, 2]), "write": pct(r[:, 4] - r[:, 3]),
                        "token": pct(r[:, 4] - r[:, 0]), "end": pct(r[:, 4] - t0)})
        finally:
            ix.close()
    for i, c in enumerate(out["calls"]):
        log(f"[phases] {name} call {i}: " + "; ".join(f"{k} {v}" for k, v in c.items()))
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--warmup-ms", type=float, default=WARMUP_MS,
                    help="least warm-up time per workload, whatever --warmup says")
    ap.add_argument("--only", choices=[HEADLINE, *SECONDARY, ATTN_WORKLOAD, *ATTN_SECONDARY,
                                       DECODE_BATCH, PROJECTION])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--ceilings", action="store_true")
    ap.add_argument("--phases", choices=["prefill8k", HEADLINE, "prefill64k", "decode1m",
                                         ATTN_WORKLOAD, *ATTN_SECONDARY],
                    help="per-phase durations from the timestamped build")
    ap.add_argument("--summarize-pmc")
    ap.add_argument("--summarize-trace")
    ap.add_argument("--summarize-mfma")
    ap.add_argument("--record-traffic", nargs=5,
                    metavar=("WORKLOAD", "FETCH_DIR", "WRITE_DIR", "COPY_FETCH_DIR", "COPY_WRITE_DIR"))
    args = ap.parse_args()

    if args.phases:
        # the timestamped build, selected before anything loads the binding
        os.environ.setdefault("DS_INDEXER_LIB", os.path.join(
            ROOT, "sparse_attention_kv_ds_amd", "libds_indexer_stamps.so"))
        print(json.dumps(phases(args.phases, args.warmup_ms)))
        return
    if args.summarize_pmc:
        summarize_pmc(args.summarize_pmc)
        return 0
    if args.summarize_trace:
        summarize_trace(args.summarize_trace)
        return 0
    if args.summarize_mfma:
        summarize_mfma(args.summarize_mfma)
        return 0
    if args.record_traffic:
        record_traffic(*args.record_traffic)
        return 0
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the library runs on exactly one GPU (the indexer kernels shard over "
              "query tokens or rows without any collective; only the 1-GPU path is built); "
              "use --gpus 1", file=sys.stderr)
        return 2
    if args.copy_calibration:
        copy_calibration()
        return 0
    if args.ceilings:
        ceilings()
        return 0

    import torch
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1

    wms = args.warmup_ms
    if args.only == PROJECTION:
        print(json.dumps(time_projection(args.only, args.steps, args.warmup, wms)))
        return 0
    if args.only == DECODE_BATCH:
        res = time_decode_batch(args.only, args.steps, args.warmup, wms)
        print(json.dumps(res))
        return 0
    if args.only in (ATTN_WORKLOAD, *ATTN_SECONDARY):
        res = time_attention(args.only, args.steps, args.warmup, wms)
        print(json.dumps({k: v for k, v in res.items()}))
        return 0
    if args.only:
        res = time_workload(args.only, args.steps, args.warmup, wms)
        print(json.dumps({"workload": args.only, "ms_per_step": res["ms_per_step"],
                          "step_stats": res["step_stats"], "kernels": res["kernels"]}))
        return 0

    head = time_workload(HEADLINE, args.steps, args.warmup, wms)
    sec = [time_workload(n, args.steps, args.warmup, wms) for n in SECONDARY]
    line = {
        "metric": METRIC,
        "value": head["pairs_per_s"],
        "unit": "pairs/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "ms_per_step_with_markers": head["ms_per_step_with_markers"],
        "step_stats": head["step_stats"],
        "warmup_calls": head["warmup_calls"],
        "warmup_ms": head["warmup_ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["wl"].dtype,
        "data": "synthetic (seeded; integer-valued fp16 q,k, power-of-two w)",
        "config": {"workload": HEADLINE, "query_tokens": head["wl"].T,
                   "positions": f"{head['wl'].p0}..{head['wl'].p0 + head['wl'].T - 1}",
                   "compressed_rows": head["wl"].N, "ratio": head["wl"].ratio,
                   "index_heads": head["wl"].H, "head_dim": head["wl"].D, "topk": head["wl"].topk,
                   "scored_pairs_per_step": head["pairs"],
                   "query_tokens_per_s": head["query_tokens_per_s"], "parallelism": "1 GPU"},
        "roofline": roofline(head),
        "kernels_ms": {c: v["avg_ms"] for c, v in head["kernels"].items()},
        "secondary": [],
    }
    for r in sec:
        wl = r["wl"]
        entry = {"workload": r["workload"], "dtype": wl.dtype, "ms_per_step": r["ms_per_step"],
                 "ms_per_step_with_markers": r["ms_per_step_with_markers"],
                 "step_stats": r["step_stats"], "warmup_calls": r["warmup_calls"],
                 "warmup_ms": r["warmup_ms"],
                 "kernels_ms": {c: v["avg_ms"] for c, v in r["kernels"].items()},
                 "roofline": roofline(r)}
        if wl.T == 1:
            rf = entry["roofline"]
            entry.update({"value": rf["achieved"], "unit": "GB/s (decode scorer, K from HBM)",
                          "end_to_end_GBps": rf["algorithmic_bytes_per_launch"] / (r["ms_per_step"] * 1e-3) / 1e9})
            if r.get("stream_only_ms"):
                so = r["stream_only_ms"]
                entry["stream_only"] = {
                    "what": "the same scorer without its partition lists (ds_indexer_scores)",
                    "ms": so, "GBps": rf["algorithmic_bytes_per_launch"] / (so * 1e-3) / 1e9,
                    "frac": rf["algorithmic_bytes_per_launch"] / (so * 1e-3) / 1e9 / PEAK_HBM_GBS}
        elif "score" not in r["kernels"]:  # whole-call skip: nothing is scored
            entry.update({"value": r["query_tokens_per_s"],
                          "unit": "query tokens/s (every row fits: sequential rows, no scoring)"})
        else:
            entry.update({"value": r["pairs_per_s"], "unit": "pairs/s",
                          "query_tokens_per_s": r["query_tokens_per_s"]})
        line["secondary"].append(entry)
    # the consumer of the indices (sparse attention over the selected rows)
    # several sequences of one query token each in one call (batched decode)
    line["secondary"].append(time_decode_batch(DECODE_BATCH, args.steps, min(args.warmup, 50), wms))
    # the query projection fused ahead of the indexer
    line["secondary"].append(time_projection(PROJECTION, args.steps, min(args.warmup, 50), wms))
    for name in (ATTN_WORKLOAD, *ATTN_SECONDARY):
        line["secondary"].append(time_attention(name, args.steps, min(args.warmup, 50), wms))
    # bracketing control: the headline again, after everything else
    ctl = time_workload(HEADLINE, args.steps, args.warmup, wms)
    line["control_rerun"] = {"workload": HEADLINE, "ms_per_step": ctl["ms_per_step"],
                             "value": ctl["pairs_per_s"], "step_stats": ctl["step_stats"],
                             "drift_vs_first": ctl["ms_per_step"] / head["ms_per_step"] - 1.0}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(HEADLINE)
    print(json.dumps(line))
    return 0


if __name__ == "__main__":
    sys.exit(main())
