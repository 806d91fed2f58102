"""Host test of the prefill kernels' workgroup -> tile mapping (CPU).

Builds tests/tile_map_check.cpp, which runs the mapping's own inline functions from
attn_fwd_tile_map.h on the host (the fast division, the bundle plan, the per-workgroup
decode), and checks it on the workloads' launch shapes and on odd ones: every
(batch, query head, query tile) is produced by exactly one workgroup, query tiles
come heaviest first inside a bundle, and with the XCD remap every workgroup of a
key/value-head group sits on one XCD.  The fast division is checked against `/` for
every divisor up to 4096 and a set of larger ones."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"

# (B, Hq, Hkv, query tiles): the named workloads with 256-query tiles (and the fp32
# workload with 32-query tiles), MQA and GQA-8, then shapes whose group counts do and
# do not split over the 8 XCDs, odd head ratios and single tiles
SHAPES = [
    (2, 32, 32, 16), (4, 16, 16, 4), (1, 32, 8, 32), (1, 16, 16, 64), (1, 2, 2, 4),
    (2, 32, 1, 16), (2, 32, 4, 16),
    (1, 1, 1, 1), (3, 12, 4, 3), (5, 6, 3, 7), (2, 9, 3, 5), (8, 8, 8, 1), (16, 32, 8, 2),
    (1, 64, 64, 1), (7, 14, 7, 11), (64, 32, 4, 1), (1, 40, 8, 33), (6, 24, 24, 9),
    (1, 5, 1, 300), (128, 1, 1, 1),
]


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_tile_map_is_a_bijection_with_heavy_tiles_first(tmp_path):
    exe = str(tmp_path / "tile_map_check")
    cmd = [HIPCC, "-O1", "-std=c++17", "-I", os.path.join(ROOT, "include"),
           "-I", os.path.join(ROOT, "attention_attn_fwd_02_amd", "csrc"),
           os.path.join(ROOT, "tests", "tile_map_check.cpp"), "-o", exe]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert b.returncode == 0, b.stderr[-3000:]
    args = [str(x) for s in SHAPES for x in s]
    r = subprocess.run([exe] + args, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr
