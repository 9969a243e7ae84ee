"""Build the HIP library (libpa.so) for gfx950 with hipcc, in-tree.

    python -m adamw_step_amd.build          # or: python adamw_step_amd/build.py

Flags: contraction into FMA off (the update is a fixed sequence of binary32
operations), packed-FP32 instructions off, correctly rounded FP32 division
and square root (the HIP default, stated explicitly), no fast math.
"""
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libpa.so")
PROBE_LIB = os.path.join(HERE, "libpa_probe.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = [
    "-O3", "-std=c++17", "-fPIC", "-shared", f"--offload-arch={ARCH}",
    "-ffp-contract=off", "-fno-fast-math", "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-gpu-flush-denormals-to-zero",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-command-line-argument",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(src, out, extra=(), verbose=False):
    tmp = out + ".tmp%d" % os.getpid()
    cmd = [HIPCC, *COMMON, *extra, src, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(verbose: bool = False):
    """Compile every HIP library of the package; returns their paths."""
    libs = [_compile(os.path.join(CSRC, "pa_api.hip"), LIB, verbose=verbose)]
    probe_src = os.path.join(CSRC, "probe_copy.hip")
    if os.path.exists(probe_src):
        libs.append(_compile(probe_src, PROBE_LIB, verbose=verbose))
    return libs


if __name__ == "__main__":
    for p in build(verbose="-v" in sys.argv):
        print(p)
