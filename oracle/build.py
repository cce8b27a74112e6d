"""Build the FP64 CPU oracle library (test infrastructure only).

Compiles oracle_f64.c with gcc into liboracle_f64.so next to this file.
No fast-math and no FP contraction, so the double-precision arithmetic is
exactly what the C source states.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "oracle_f64.c")
LIB = os.path.join(HERE, "liboracle_f64.so")

CFLAGS = ["-O2", "-std=c11", "-ffp-contract=off", "-fno-fast-math",
          "-fPIC", "-shared", "-pthread", "-Wall", "-Wextra"]


def build(verbose: bool = False) -> str:
    """Compile the oracle library; returns its path."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", *CFLAGS, SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
    sys.exit(0)
