"""Host-side checks of bench.py's contract (no GPU): the multi-GPU refusal and
the measured-traffic lookup, which must stop reporting once the kernel
sources differ from the ones the counters were taken on."""

import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120)
    assert res.returncode == 2
    line = json.loads(res.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"] and line["n_gpus"] == 2


def test_traffic_lookup_follows_the_kernel_sources(tmp_path, monkeypatch):
    sha = bench._kernel_sources_sha256()
    f = tmp_path / "traffic.txt"
    f.write_text(f"kernel_sources_sha256 {sha}\n"
                 "traffic decode15 splits=8 read_bytes=100 write_bytes=20\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench._traffic("decode15", 8) == {"read": 100, "write": 20, "total": 120}
    assert bench._traffic("decode15", 4) is None          # other split count
    assert bench._traffic("batch128", 8) is None          # other workload
    f.write_text("kernel_sources_sha256 " + "0" * 64 + "\n"
                 "traffic decode15 splits=8 read_bytes=100 write_bytes=20\n")
    assert bench._traffic("decode15", 8) is None          # taken on other kernel sources

