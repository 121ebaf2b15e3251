"""Host-side checks of bench.py's contract (no GPU): the committed HBM
traffic summary still describes the indexer sources as they are (else the
bench reports its traffic as null), and runs on more than one GPU are
refused with a message."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _summary_fields():
    t = {}
    with open(bench.TRAFFIC_FILE) as f:
        for line in f:
            if line.startswith("- ") and ": " in line:
                key, val = line[2:].strip().split(": ", 1)
                t[key] = val
    return t


def test_traffic_summary_matches_indexer_sources():
    t = _summary_fields()
    assert t["workload"] == "csa_decode_128k_bf16"
    assert t["source_sha256"] == bench.source_digest(bench.INDEXER_SOURCES), (
        "the indexer sources changed since the FETCH_SIZE / WRITE_SIZE counters were taken")
    assert float(t["traffic_bytes_per_launch"]) > 0


def test_multi_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
