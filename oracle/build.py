"""Build the C oracle (test infrastructure only) with gcc.

The oracle library is compiled from ``gemm_f64.c`` with plain ``gcc``: no HIP
headers, no code from the GPU library.  ``-ffp-contract=off`` keeps every
multiply and add a separately rounded binary64 operation.
"""
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "gemm_f64.c")
LIB = os.path.join(HERE, "_build", "liboracle_gemm.so")


def build(verbose: bool = False) -> str:
    os.makedirs(os.path.dirname(LIB), exist_ok=True)
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-shared", "-fPIC", "-std=c11", "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
