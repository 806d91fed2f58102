"""Build the fp64 CPU oracle (test infrastructure only) with gcc.

The oracle is the reference the HIP attention path is tested against; building it is part of
the project's build step, but only the tests, the smoke check and the
benchmark's CPU-baseline leg ever load it.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "attn_oracle.c")
LIB = os.path.join(HERE, "liboracle.so")


def build(src: str = SRC, out: str = LIB, extra_flags=()) -> str:
    """Compile `src` into the shared library `out`; returns its path.

    -O2 without -ffast-math: the oracle keeps IEEE fp64 semantics and the
    summation order written in the source.
    """
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-std=c11", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
           "-fPIC", "-shared", *extra_flags, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(*sys.argv[1:2]))
