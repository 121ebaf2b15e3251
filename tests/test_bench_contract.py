"""Host-side checks of bench.py's contract (no GPU): the committed HBM
counter summaries are well formed and the bench reports their traffic only
while the kernel's sources are the ones they were taken from; the step's
algorithmic bytes follow the per-query accounting of the workloads; runs on
more than one GPU are refused with a message; a stale library is detected."""

import os
import subprocess
import sys

import pytest

import bench
import workloads as WL

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_summaries_well_formed():
    sums = bench.traffic_summaries()
    assert sums, "no counter summary under profiles/"
    for t in sums:
        for key in ("workload", "kernel", "source_sha256", "traffic_bytes_per_launch"):
            assert key in t, (t["file"], key)
        assert t["workload"] in WL.BY_NAME, t["file"]
        assert float(t["traffic_bytes_per_launch"]) > 0
        got = bench.measured_traffic(t["workload"], t["kernel"])
        current = t["source_sha256"] == bench.source_digest(bench.kernel_sources(t["kernel"]))
        # reported while current, null once the kernel's sources changed
        assert (got is not None) == current, t["file"]


def test_step_bytes_per_query():
    # 128K decode, bf16: 32768 keys x 256 B scanned, 1024 + 128 K/V rows x
    # 2 x 256 B gathered, q (16 KiB) + indexer q (16 KiB) + head weights
    # (256 B) read, 64 x 128 fp32 outputs (32 KiB) written
    c2 = WL.BY_NAME["csa_decode_128k_bf16"]
    per_q = 32768 * 256 + 1152 * 512 + 16384 + 16384 + 256 + 32768
    assert bench.step_bytes(c2) == 32 * per_q
    # 1M decode, fp8 indexer: 262144 x (128 code bytes + 4 scale bytes)
    c5 = WL.BY_NAME["csa_decode_1m_fp8"]
    per_q = 262144 * 132 + 1152 * 512 + 64 * 132 + 256 + 16384 + 32768
    assert bench.step_bytes(c5) == 4 * per_q
    # HCA 1M: every one of the 8192 entries plus the window, no indexer
    c4 = WL.BY_NAME["hca_decode_1m_bf16"]
    assert bench.step_bytes(c4) == 16 * ((8192 + 128) * 512 + 16384 + 32768)


def test_multi_gpu_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)


def test_library_digest_matches_sources():
    import __graft_entry__
    b = __graft_entry__._build_module()
    b.ensure_current(verbose=False)
    assert b.library_digest() == b.source_digest()


def test_stale_library_detected(tmp_path):
    import __graft_entry__
    b = __graft_entry__._build_module()
    b.ensure_current(verbose=False)
    with open(b.LIB, "rb") as f:
        data = f.read()
    i = data.find(b.DIGEST_TAG) + len(b.DIGEST_TAG)
    stale = tmp_path / "libcsa.so"
    stale.write_bytes(data[:i] + b"0" * 64 + data[i + 64:])
    assert b.library_digest(str(stale)) == "0" * 64
    assert b.library_digest(str(stale)) != b.source_digest()
    assert b.library_digest(str(tmp_path / "missing.so")) is None


@pytest.mark.parametrize("name", bench.EXTRA_WORKLOADS)
def test_extra_workloads_exist(name):
    assert name in WL.BY_NAME
