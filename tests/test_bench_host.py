"""Host-side contract of bench.py, checked without a GPU: one GPU only, and
HBM byte counters reported only for the GEMM source they were taken on."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_kernel_hash_ignores_comments_and_layout(tmp_path, monkeypatch):
    src = open(bench.GEMM_SRC).read()
    h0 = bench.kernel_hash()
    p = tmp_path / "experts.hip"
    p.write_text("// a comment\n/* another\n one */\n" + src.replace("\n", "\n\n"))
    monkeypatch.setattr(bench, "GEMM_SRC", str(p))
    assert bench.kernel_hash() == h0
    p.write_text(src + "\nint changed_code;\n")
    assert bench.kernel_hash() != h0


def test_traffic_only_for_the_counted_source(tmp_path, monkeypatch):
    got = bench.traffic_for("prefill_bf16")
    assert got is None or (isinstance(got, int) and got > 0)
    p = tmp_path / "experts.hip"
    p.write_text(open(bench.GEMM_SRC).read() + "\nint changed_code;\n")
    monkeypatch.setattr(bench, "GEMM_SRC", str(p))
    assert bench.traffic_for("prefill_bf16") is None
    assert bench.traffic_for("no_such_workload") is None
