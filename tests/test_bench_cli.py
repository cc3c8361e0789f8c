"""bench.py's command line and its traffic record, on the CPU (nothing here
touches a GPU)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_every_path_is_accepted(monkeypatch):
    for path in ("decode", "encode", "overlap", "fused", "lmhead", "adaptive", "workloads"):
        monkeypatch.setattr(sys, "argv", ["bench.py", "--path", path, "--steps", "3"])
        a = bench.parse()
        assert a.path == path and a.steps == 3 and a.gpus == 1


def test_traffic_is_reported_only_for_the_sources_it_was_taken_with(tmp_path, monkeypatch):
    rec = {"kernel_sources_sha256": bench.kernel_sources_sha256(),
           "fetch_bytes_per_launch": 3.0e8, "write_bytes_per_launch": 1.7e9}
    f = tmp_path / "traffic.json"
    f.write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic() == 2.0e9
    rec["kernel_sources_sha256"] = "0" * 64
    f.write_text(json.dumps(rec))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic() is None
