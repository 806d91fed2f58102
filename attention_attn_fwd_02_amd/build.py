"""Build the HIP library `libattn_fwd.so` (gfx950) in-tree with hipcc.

    python -m attention_attn_fwd_02_amd.build          # build the library
    python -m attention_attn_fwd_02_amd.build --asm D  # also write the device assembly to D/
"""
import argparse
import os
import subprocess

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(PKG, "libattn_fwd.so")
SOURCES = [os.path.join(CSRC, "attn_fwd_kernels.hip"), os.path.join(CSRC, "attn_fwd32_kernels.hip"),
           os.path.join(CSRC, "attn_decode_kernels.hip"),
           os.path.join(CSRC, "attn_bwd_kernels.hip"), os.path.join(CSRC, "attn_rope_kernels.hip"),
           os.path.join(CSRC, "attn_fwd_api.cpp")]
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the generated code (feature switched off).
COMMON = ["-O3", "-std=c++17", "--offload-arch=" + ARCH,
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-I" + INCLUDE, "-I" + CSRC, "-Wno-unused-command-line-argument"]


def build(out: str = LIB, verbose: bool = False) -> str:
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["hipcc", *COMMON, "-fPIC", "-shared", *SOURCES, "-o", tmp]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    _check_resolved(tmp)
    os.replace(tmp, out)
    return out


def _check_resolved(lib: str) -> None:
    """Every kernel launch stub must be defined in the library itself (a kernel
    the host pass failed to emit shows up as an undefined attn_impl symbol)."""
    res = subprocess.run(["nm", "-D", "--undefined-only", lib], check=True,
                         capture_output=True, text=True)
    missing = [ln.split()[-1] for ln in res.stdout.splitlines() if "attn_impl" in ln]
    if missing:
        os.remove(lib)
        raise RuntimeError("kernel stubs missing from %s: %s" % (lib, ", ".join(missing)))


def dump_asm(outdir: str) -> str:
    """Device assembly of the kernels (for register / LDS / instruction-mix review)."""
    os.makedirs(outdir, exist_ok=True)
    out = os.path.join(outdir, "attn_fwd_kernels-%s.s" % ARCH)
    cmd = ["hipcc", *COMMON, "-S", "--cuda-device-only", SOURCES[0], "-o", out]
    subprocess.run(cmd, check=True)
    return out


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="also write device assembly into this folder")
    ap.add_argument("-v", "--verbose", action="store_true")
    a = ap.parse_args()
    print(build(verbose=a.verbose))
    if a.asm:
        print(dump_asm(a.asm))
