"""Host-side logic of bench.py (no GPU): the one-GPU guard, the kernel-source
hash that ties a committed counter summary to the code it measured, and the
traffic figure's fallback to null when they no longer match."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_hash_ignores_comments_and_blank_lines(tmp_path, monkeypatch):
    src = open(bench.KERNEL_SRC, encoding="utf-8").read()
    a = tmp_path / "a.hip"
    b = tmp_path / "b.hip"
    c = tmp_path / "c.hip"
    a.write_text(src)
    b.write_text("// a new leading comment\n\n" + src.replace("\n", "   // trailing note\n", 3) + "\n\n")
    c.write_text(src.replace("constexpr int TILE = 64;", "constexpr int TILE = 32;"))
    hashes = {}
    for p in (a, b, c):
        monkeypatch.setattr(bench, "KERNEL_SRC", str(p))
        hashes[p.name] = bench.kernel_source_hash()
    assert hashes["a.hip"] == hashes["b.hip"]
    assert hashes["a.hip"] != hashes["c.hip"]


def test_traffic_is_used_only_for_the_measured_source(tmp_path, monkeypatch):
    summary = tmp_path / "traffic.txt"
    good = bench.kernel_source_hash()
    summary.write_text(f"kernel_source_sha256: {good}\ntraffic_bytes_per_launch: 12345\n")
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(summary))
    assert bench.traffic_from_profile() == 12345.0
    summary.write_text(f"kernel_source_sha256: {'0' * 64}\ntraffic_bytes_per_launch: 12345\n")
    assert bench.traffic_from_profile() is None
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "missing.txt"))
    assert bench.traffic_from_profile() is None
