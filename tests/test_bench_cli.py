"""bench.py's host logic (CPU): the one-GPU guard and the source-keyed traffic lookup."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""          # no JSON line


def test_traffic_is_read_for_the_current_kernel_source():
    t = bench.committed_traffic("mha_causal_bf16_b2_h32_s4096_d128")
    # the committed summary holds HBM bytes per launch of the current forward kernel
    assert t is not None and 2.0e8 < t < 1.0e9


def test_traffic_is_null_for_another_kernel_source(tmp_path):
    src = tmp_path / "changed.hip"
    with open(bench.KERNEL_SRC, "rb") as f:
        src.write_bytes(f.read() + b"\n// changed\n")
    assert bench.committed_traffic("mha_causal_bf16_b2_h32_s4096_d128", src=str(src)) is None


def test_traffic_is_null_without_a_summary():
    assert bench.committed_traffic("no_such_workload") is None
