"""Host logic of bench.py (no GPU): the one-GPU guard, the HBM-traffic
calibration arithmetic from counter CSVs, and the stale-counter rule."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def _counters(directory, rows):
    """A rocprofv3-style counter_collection.csv with (dispatch, kernel, counter, value) rows."""
    os.makedirs(directory, exist_ok=True)
    with open(os.path.join(directory, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for d, k, c, v in rows:
            w.writerow({"Dispatch_Id": d, "Kernel_Name": k, "Counter_Name": c, "Counter_Value": v})


def test_record_traffic_scales_by_the_copy(tmp_path, monkeypatch):
    """The counters are per-XCD partial sums per dispatch: the table sums them
    per dispatch and averages over dispatches; FETCH_SIZE and WRITE_SIZE are
    scaled by what the 512 MiB copy reads for each."""
    kib = 512 * 1024.0
    # the copy: FETCH_SIZE reads half the bytes (two XCD halves per dispatch), WRITE_SIZE all
    _counters(tmp_path / "cf", [(1, "copy", "FETCH_SIZE", kib / 4), (1, "copy", "FETCH_SIZE", kib / 4)])
    _counters(tmp_path / "cw", [(1, "copy", "WRITE_SIZE", kib)])
    k = "void dsi::prefill_scorer_kernel<64>(...)"
    # two dispatches of the kernel: 100 and 140 KiB fetched, 10 and 30 written
    _counters(tmp_path / "kf", [(7, k, "FETCH_SIZE", 60.0), (7, k, "FETCH_SIZE", 40.0),
                                (9, k, "FETCH_SIZE", 140.0), (8, "other", "FETCH_SIZE", 1e6)])
    _counters(tmp_path / "kw", [(7, k, "WRITE_SIZE", 10.0), (9, k, "WRITE_SIZE", 30.0)])
    store = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(store))
    bench.record_traffic("prefill32k", str(tmp_path / "kf"), str(tmp_path / "kw"),
                         str(tmp_path / "cf"), str(tmp_path / "cw"))
    rec = json.loads(store.read_text())["score:prefill32k"]
    assert rec["kernel"] == k
    assert rec["fetch_kib_per_dispatch"] == pytest.approx(120.0)
    assert rec["write_kib_per_dispatch"] == pytest.approx(20.0)
    assert rec["fetch_scale"] == pytest.approx(2.0)
    assert rec["write_scale"] == pytest.approx(1.0)
    assert rec["hbm_bytes_per_launch"] == pytest.approx((120.0 * 2.0 + 20.0) * 1024.0)
    assert rec["source_hash"] == bench.source_hash("score")


def test_stored_traffic_is_dropped_when_the_kernel_changed(tmp_path, monkeypatch):
    store = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(store))
    assert bench.stored_traffic("score", "prefill32k") is None  # no file
    store.write_text(json.dumps({"score:prefill32k": {"source_hash": bench.source_hash("score"),
                                                      "hbm_bytes_per_launch": 123.0}}))
    assert bench.stored_traffic("score", "prefill32k") == 123.0
    assert bench.stored_traffic("score", "prefill64k") is None  # no record
    store.write_text(json.dumps({"score:prefill32k": {"source_hash": "0" * 16,
                                                      "hbm_bytes_per_launch": 123.0}}))
    assert bench.stored_traffic("score", "prefill32k") is None  # sources changed since
