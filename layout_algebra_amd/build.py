"""Compile the HIP library (liblagemm.so) for gfx950 with hipcc.

Every source is compiled with ``--offload-arch=gfx950`` only, and with the
packed-FP32 instructions switched off (``-target-feature -packed-fp32-ops``).
Objects are built in parallel under ``_build/`` and linked into
``layout_algebra_amd/liblagemm.so``.
"""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "liblagemm.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SOURCES = ["layout.cpp", "planner.cpp", "capi.cpp", "kernels.cpp", "gemm_tiled_64.hip", "gemm_tiled_128.hip", "gemm_tiled_p3.hip", "gemm_f32.hip", "gemm_fast.hip", "gemm_fast_gu.hip", "gemm_fast_128.hip", "gemm_fast_f8.hip", "gemm_skinny.hip", "rms_norm.hip", "row_reduce.hip", "split_sum.hip", "attention.hip", "probe.hip"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "--offload-arch=gfx950",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-command-line-argument"]


def _compile(src: str, verbose: bool) -> str:
    obj = os.path.join(BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + COMMON + ["-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("hipcc failed on %s:\n%s" % (src, r.stderr))
    noise = "packed-fp32-ops"
    for line in r.stderr.splitlines():
        if line.strip() and noise not in line and verbose:
            print(line)
    return obj


def build(verbose: bool = False, jobs: int = 8) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=jobs) as ex:
        objs = list(ex.map(lambda s: _compile(s, verbose), SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=gfx950", "-o", tmp] + objs
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
