"""The binding loads the library against torch's HIP runtime (CPU test).

torch bundles its own copy of the HIP runtime under a different file name.  If the
library were loaded before torch, the process would hold two runtimes and the
library's kernels could not run on torch's streams and memory; `load_library`
therefore imports torch first.  Checked in a fresh process that calls
`load_library` before anything else imports torch."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "attention_attn_fwd_02_amd", "libattn_fwd.so")

PROG = r"""
import sys
sys.path.insert(0, %r)
from attention_attn_fwd_02_amd import attn
assert "torch" not in sys.modules
attn.load_library()
import torch
maps = open("/proc/self/maps").read().split("\n")
paths = sorted({l.split()[-1] for l in maps if "libamdhip64" in l and "/" in l})
print("\n".join(paths))
"""


@pytest.mark.skipif(not os.path.exists(LIB), reason="library not built")
def test_one_hip_runtime_when_the_library_is_loaded_first():
    r = subprocess.run([sys.executable, "-c", PROG % ROOT], capture_output=True, text=True,
                       timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    paths = [p for p in r.stdout.split("\n") if p.strip()]
    assert len(paths) == 1, "HIP runtimes mapped: %s" % paths
