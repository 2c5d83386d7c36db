"""Host-side logic of bench.py (no GPU): the one-GPU guard, the stored
counter figures and the CPU baseline's arithmetic."""

from __future__ import annotations

import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout.strip() == ""  # no JSON line for a run that did not happen


def test_stored_traffic_is_consistent_or_absent():
    t = bench.measured_traffic()
    with open(bench.TRAFFIC_FILE) as f:
        stored = json.load(f)
    if stored["decode_src_sha256_16"] != bench.decode_src_hash():
        assert t is None  # figures of another kernel are never reported
        return
    assert t == stored
    assert t["bytes_per_launch"] == t["fetch_bytes_per_launch"] + t["write_bytes_per_launch"]
    # each counter is scaled by what it read for a copy of known size
    assert t["fetch_scale"] == pytest.approx(t["copy_bytes_each_way"] / 1024 /
                                             t["copy_fetch_kib_raw"], rel=1e-4)
    assert t["write_scale"] == pytest.approx(t["copy_bytes_each_way"] / 1024 /
                                             t["copy_write_kib_raw"], rel=1e-4)
    assert t["traffic_over_algorithmic"] == pytest.approx(
        t["bytes_per_launch"] / t["algorithmic_bytes_per_launch"], abs=1e-4)


def test_decode_src_hash_tracks_the_kernel_sources(tmp_path, monkeypatch):
    h0 = bench.decode_src_hash()
    copies = []
    for i, path in enumerate(bench.DECODE_SRCS):
        c = tmp_path / f"src{i}"
        c.write_bytes(open(path, "rb").read())
        copies.append(str(c))
    monkeypatch.setattr(bench, "DECODE_SRCS", copies)
    assert bench.decode_src_hash() == h0
    with open(copies[0], "ab") as f:
        f.write(b"\n")
    assert bench.decode_src_hash() != h0


def test_cpu_baseline_scales_the_median_pair_time(monkeypatch):
    """value = median oracle time of one (b, h) pair x the number of pairs;
    the oracle call is replaced by a fixed 2 ms sleep to check the scaling."""
    import time

    import oracle

    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS["tiny"].replace(batch=3)
    inp = make_inputs(w, device="cpu")
    calls = []

    def fixed(*a, **k):
        calls.append(k.get("mode"))
        time.sleep(0.002)

    monkeypatch.setattr(oracle, "decode_pair", fixed)
    res = bench.cpu_baseline(inp, w, 0.1)
    pairs = w.batch * w.num_kv_heads
    assert res["kind"] == "oracle" and res["unit"] == "us/step" and res["cores"] >= 1
    assert 2000 * pairs <= res["value"] <= 3000 * pairs
    assert calls and all(m == w.mode for m in calls)
    assert f"of {pairs};" in res["sample"]
