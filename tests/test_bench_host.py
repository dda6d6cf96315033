"""Host-only checks of bench.py: the one-GPU refusal and the rule that ties the reported HBM traffic to the
kernel source the counters were taken on (a changed kernel reports no traffic rather than a stale figure)."""

import hashlib
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=600)
    assert r.returncode == 2
    assert "one MI355X" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_traffic_reported_only_for_the_source_it_was_measured_on(tmp_path, monkeypatch):
    src = tmp_path / "gemm.hip"
    src.write_bytes(b"// kernel source\n")
    rec = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "GEMM_SOURCE", str(src))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(rec))
    assert bench.gemm_traffic() is None  # no record
    rec.write_text(json.dumps({"bytes_per_launch": 1234.5,
                               "gemm_source_sha256": hashlib.sha256(src.read_bytes()).hexdigest()}))
    assert bench.gemm_traffic() == 1234.5
    src.write_bytes(b"// kernel source, edited\n")
    assert bench.gemm_traffic() is None  # the kernel changed since the counters were taken


def test_committed_traffic_record_is_well_formed():
    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    # FETCH_SIZE and WRITE_SIZE scaled by the plain-copy calibration: at least the algorithmic 496 MiB
    assert rec["bytes_per_launch"] >= 496 * 2**20
    assert abs(rec["write_scale"] - 1.0) < 0.01 and abs(rec["fetch_scale"] - 2.0) < 0.01
    assert len(rec["gemm_source_sha256"]) == 64
