"""Host-side checks of bench.py (no GPU): the one-GPU rule and the rule that
a profile's HBM traffic is reported only for the kernel source it was taken
on."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_recorded_traffic_needs_the_current_source(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    path = tmp_path / "fwd_1x2x4_pmc.txt"
    assert bench.recorded_traffic("fwd", "1x2x4") is None            # no summary
    path.write_text("# header: ignored\nkernel_source_sha256: 0123\nhbm_bytes_per_launch: 5000\n")
    assert bench.recorded_traffic("fwd", "1x2x4") is None            # another source
    path.write_text(f"kernel_source_sha256: {bench.source_digest('fwd')}\nhbm_bytes_per_launch: 5000.7\n")
    assert bench.recorded_traffic("fwd", "1x2x4") == 5000
    # the packer's and quantizers' summaries are checked against their own file
    ppath = tmp_path / "pack_1x4_pmc.txt"
    ppath.write_text(f"kernel_source_sha256: {bench.source_digest('fwd')}\nhbm_bytes_per_launch: 7\n")
    assert bench.source_digest("pack") != bench.source_digest("fwd")
    assert bench.recorded_traffic("pack", "1x4") is None
    ppath.write_text(f"kernel_source_sha256: {bench.source_digest('pack')}\nhbm_bytes_per_launch: 7\n")
    assert bench.recorded_traffic("pack", "1x4") == 7


def test_kernel_work_bytes():
    M, N, K = 16384, 3456, 1280
    assert bench.kernel_work("fwd", M, N, K) == (2 * M * N * K, M * K + N * K // 4 + 4 * M * N)
    assert bench.kernel_work("dx", M, N, K)[1] == M * N + N * K // 4 + 4 * M * K
    assert bench.kernel_work("dw", M, N, K)[1] == M * K + M * N + 4 * K * N
