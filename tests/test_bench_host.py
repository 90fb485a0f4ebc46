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


def _copies(tmp_path, edit_index=None, edit=lambda s: s):
    """Copies of the GEMM sources, the one at edit_index passed through edit."""
    paths = []
    for i, src in enumerate(bench.GEMM_SRCS):
        p = tmp_path / os.path.basename(src)
        text = open(src).read()
        p.write_text(edit(text) if i == edit_index else text)
        paths.append(str(p))
    return paths


def test_kernel_hash_ignores_comments_and_layout(tmp_path, monkeypatch):
    h0 = bench.kernel_hash()
    for i in range(len(bench.GEMM_SRCS)):
        monkeypatch.setattr(bench, "GEMM_SRCS",
                            _copies(tmp_path, i, lambda s: "// a comment\n/* another\n one */\n" + s.replace("\n", "\n\n")))
        assert bench.kernel_hash() == h0


def test_kernel_hash_covers_every_gemm_source(tmp_path, monkeypatch):
    """The kernel file and each header compiled into the GEMM kernels: a code
    edit in any of them changes the hash."""
    names = [os.path.basename(p) for p in bench.GEMM_SRCS]
    assert {"experts.hip", "mfma.h", "tiles.h", "moe_internal.h"} <= set(names)
    h0 = bench.kernel_hash()
    for i in range(len(bench.GEMM_SRCS)):
        monkeypatch.setattr(bench, "GEMM_SRCS", _copies(tmp_path, i, lambda s: s + "\nint changed_code;\n"))
        assert bench.kernel_hash() != h0


def test_traffic_only_for_the_counted_source(tmp_path, monkeypatch):
    got = bench.traffic_for("prefill_bf16")
    assert got is None or (isinstance(got, int) and got > 0)
    for i in range(len(bench.GEMM_SRCS)):
        monkeypatch.setattr(bench, "GEMM_SRCS", _copies(tmp_path, i, lambda s: s + "\nint changed_code;\n"))
        assert bench.traffic_for("prefill_bf16") is None
    assert bench.traffic_for("no_such_workload") is None
