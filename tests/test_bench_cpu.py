"""bench.py's host-side contract (no GPU needed)."""

import json
import os
import subprocess
import sys

import bench


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(bench.ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_is_keyed_to_the_sources(monkeypatch):
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert {"verify", "prompt", "reduce"} <= set(t["kernels"])
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: t["source_hash"])
    v = bench.load_traffic("verify")
    assert v["read_bytes"] > 0 and v["write_bytes"] > 0
    assert v["total_bytes"] == v["read_bytes"] + v["write_bytes"]
    assert bench.load_traffic("no such kernel") is None
    # counters taken on other sources are not reported
    monkeypatch.setattr(bench, "kernel_source_hash", lambda: "0" * 16)
    assert bench.load_traffic("verify") is None


def test_source_hash_is_stable_and_short():
    h = bench.kernel_source_hash()
    assert h == bench.kernel_source_hash() and len(h) == 16
