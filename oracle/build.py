"""Compile the CPU oracle (plain C, gcc) into oracle/libpa_oracle.so.

Test infrastructure: the library this builds is loaded only by the tests,
the smoke check and the benchmark's cpu_baseline leg.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "pa_oracle.c")
OUT = os.path.join(HERE, "libpa_oracle.so")

# SSE arithmetic, no contraction into FMA, no fast math: every float
# operation in the oracle is one correctly rounded binary32 operation.
CFLAGS = [
    "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
    "-ffp-contract=off", "-fno-fast-math", "-msse2", "-mfpmath=sse",
    "-fexcess-precision=standard", "-fno-finite-math-only",
    "-Wall", "-Wextra",
]


def build(verbose: bool = False) -> str:
    tmp = OUT + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lquadmath", "-lm"]
    if verbose:
        print(" ".join(cmd))
    subprocess.run(cmd, check=True)
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
