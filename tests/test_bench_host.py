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


def _fixed_oracle(monkeypatch, seconds):
    import time

    import oracle
    calls = []

    def fixed(*a, **k):
        calls.append(k.get("mode"))
        time.sleep(seconds)

    monkeypatch.setattr(oracle, "decode_pair", fixed)
    return calls


def test_cpu_baseline_sums_every_pair(monkeypatch):
    """Within the budget the value is the whole step: every (b, h) pair timed
    three times, the medians summed.  The oracle call is replaced by a fixed
    2 ms sleep to check the arithmetic."""
    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS["tiny"].replace(batch=3)
    inp = make_inputs(w, device="cpu")
    calls = _fixed_oracle(monkeypatch, 0.002)
    res = bench.cpu_baseline(inp, w, 60.0)
    pairs = w.batch * w.num_kv_heads
    assert res["kind"] == "oracle" and res["unit"] == "us/step" and res["cores"] >= 1
    assert res["pairs_timed"] == res["pairs"] == pairs
    assert len(calls) == 3 * pairs and all(m == w.mode for m in calls)
    assert 2000 * pairs <= res["value"] <= 3000 * pairs
    assert res["os_cpu_count"] == os.cpu_count() and res["affinity_cpus"] >= 1
    assert "the whole step" in res["sample"]


def test_cpu_baseline_scales_a_cut_sample(monkeypatch):
    """A budget too small for every pair: the mean of the timed pairs times
    the number of pairs, and the line names how many were timed."""
    from workloads import WORKLOADS, make_inputs
    w = WORKLOADS["tiny"].replace(batch=5)
    inp = make_inputs(w, device="cpu")
    _fixed_oracle(monkeypatch, 0.002)
    res = bench.cpu_baseline(inp, w, 0.0)  # stops after the first pair
    pairs = w.batch * w.num_kv_heads
    assert res["pairs_timed"] == 1 < pairs
    assert 2000 * pairs <= res["value"] <= 3000 * pairs
    assert f"1 of {pairs}" in res["sample"]


def test_counter_summary_scales_each_group(tmp_path, monkeypatch):
    """--counter-summary on synthetic counter CSVs: each group's counters are
    averaged over its last launches, scaled by the copy's, and the decode's
    figures land in the traffic file with the pass's source hash."""
    cols = ("Dispatch_Id,Grid_Size,Workgroup_Size,Kernel_Name,Counter_Name,Counter_Value")
    kern = [("void seer::(anonymous namespace)::decode_kernel<128, 64, false, 8, false, false>"
             "(seer::(anonymous namespace)::DecodeParams)", 256, 512),
            ("void seer::(anonymous namespace)::gate_kernel<128, 128>(seer::GateParams)", 128, 512),
            ("void at::native::neg_kernel(...)", 65536, 256)]

    def csv_file(name, counter, values):
        lines = [cols]
        for i, (k, v) in enumerate(values):
            kname, wgs, wgsz = kern[k]
            lines.append(f'{i},{wgs * wgsz},{wgsz},"{kname}",{counter},{v}')
        path = tmp_path / name
        path.write_text("\n".join(lines) + "\n")
        return str(path)

    # decode: a cold first launch, then two at 100 KiB fetched / 2 written;
    # gate: 10 / 1; the copy: 131072 KiB fetched (scale 2), 262144 written
    fetch = csv_file("f.csv", "FETCH_SIZE", [(0, 999.0), (0, 100.0), (0, 100.0), (1, 10.0),
                                             (2, 131072.0), (2, 131072.0), (2, 131072.0)])
    write = csv_file("w.csv", "WRITE_SIZE", [(0, 2.0), (0, 2.0), (0, 2.0), (1, 1.0),
                                             (2, 262144.0), (2, 262144.0), (2, 262144.0)])
    info = {"counter_pass": True, "copy_kernel": "neg_kernel", "copy_bytes_each_way": 256 << 20,
            "copies": 3, "decode_src_sha256_16": "abc",
            "groups": [{"label": "sparse decode, top-k 52, fixed splits",
                        "kernel": "decode_kernel<128, 64, false, 8, false, false>",
                        "workgroups": 256, "algorithmic_bytes_per_launch": 200 * 1024,
                        "launches": 2},
                       {"label": "gate", "kernel": "gate_kernel<128, 128>", "workgroups": 128,
                        "algorithmic_bytes_per_launch": 20 * 1024, "launches": 1}]}
    pj = tmp_path / "pass.json"
    pj.write_text("[bench] log line\n" + json.dumps(info) + "\n")
    out = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(out))
    assert bench.counter_summary(str(pj), fetch, write) == 0
    t = json.loads(out.read_text())
    assert t["decode_src_sha256_16"] == "abc"
    assert t["fetch_scale"] == pytest.approx(2.0) and t["write_scale"] == pytest.approx(1.0)
    assert t["fetch_bytes_per_launch"] == 200 * 1024  # the cold launch is not averaged in
    assert t["write_bytes_per_launch"] == 2 * 1024
    assert t["traffic_over_algorithmic"] == pytest.approx(202 / 200, abs=1e-4)
