"""Host-side logic of bench.py that needs no GPU: the traffic figure is read
from the committed counter summary only while the GEMM source matches the hash
recorded with it, and a multi-GPU request is refused with a message."""
import hashlib
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_matches_committed_summary():
    with open(bench.GEMM_SOURCE, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    fields = {}
    with open(bench.TRAFFIC_FILE) as f:
        for line in f:
            key, sep, val = line.strip().partition(": ")
            if sep:
                fields[key] = val.strip()
    got = bench.measured_traffic("gemm_pair_kernel<true>")
    if fields.get("source_sha256") == sha:
        # bytes per pair launch of the gate/up linear: above its 0.777 GB of algorithmic traffic
        assert got is not None and 0.777e9 < got < 1e11
    else:
        assert got is None


def test_traffic_is_null_for_another_source(tmp_path, monkeypatch):
    other = tmp_path / "gemm.hip"
    other.write_text("// a different source\n")
    monkeypatch.setattr(bench, "GEMM_SOURCE", str(other))
    assert bench.measured_traffic("gemm_pair_kernel<true>") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.md"))
    assert bench.measured_traffic("gemm_pair_kernel<true>") is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in r.stderr
