"""bench.py's host logic (CPU): the one-GPU guard, the source-keyed traffic lookup, the
clock summary over the timed interval and the window split of the timed steps."""
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
    with open(bench.KERNEL_SRC[0], "rb") as f:
        src.write_bytes(f.read() + b"\n// changed\n")
    assert bench.committed_traffic("mha_causal_bf16_b2_h32_s4096_d128",
                                   src=(str(src), bench.KERNEL_SRC[1])) is None
    # a change to the tile map header alone is a different kernel too
    hdr = tmp_path / "changed.h"
    with open(bench.KERNEL_SRC[1], "rb") as f:
        hdr.write_bytes(f.read() + b"\n// changed\n")
    assert bench.committed_traffic("mha_causal_bf16_b2_h32_s4096_d128",
                                   src=(bench.KERNEL_SRC[0], str(hdr))) is None


def test_traffic_is_null_without_a_summary():
    assert bench.committed_traffic("no_such_workload") is None


def test_clock_summary_keeps_the_timed_interval():
    s = bench.SclkSampler()
    # samples before, inside and after a timed interval [10, 20] (perf_counter seconds)
    s.values = [(5.0, 2400.0), (11.0, 1900.0), (15.0, 1880.0), (19.0, 1920.0), (25.0, 2400.0)]
    got = s.summary(10.0, 20.0)
    assert got["samples"] == 3
    assert got["median_mhz"] == 1900.0 and got["min_mhz"] == 1880.0 and got["max_mhz"] == 1920.0
    # no sample inside a short interval: every sample is reported instead of none
    assert s.summary(12.0, 13.0)["samples"] == 5


def test_timed_windows_cover_exactly_the_requested_steps():
    class Ev:
        t = 0.0

        def __init__(self, enable_timing=True):
            self.at = None

        def record(self, stream):
            self.at = Ev.t

        def elapsed_time(self, other):
            return other.at - self.at

    class Cuda:
        Event = Ev

        @staticmethod
        def synchronize():
            pass

    class Torch:
        cuda = Cuda

    calls = []

    def step():
        calls.append(1)
        Ev.t += 2.0                      # every step takes 2 ms of "device time"

    for steps in (1, 3, 5, 7, 20):
        calls.clear()
        wall, per_launch, wins, (t0, t1) = bench.timed_run(step, steps, None, Torch)
        assert len(calls) == steps
        assert len(wins) == min(5, steps)
        assert abs(per_launch - 2.0) < 1e-9 and all(abs(w - 2.0) < 1e-9 for w in wins)
        assert t1 >= t0
