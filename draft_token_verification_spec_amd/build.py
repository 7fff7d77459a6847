"""Build the HIP libraries (gfx950) in-tree.

    python -m draft_token_verification_spec_amd.build

compiles every ``csrc/*.hip`` and ``csrc/api.cpp`` with hipcc into
``draft_token_verification_spec_amd/libspecverify.so`` (the verification
library behind ``include/specverify.h``), and ``csrc/bench/*.hip`` into
``libsvbench.so`` (measurement aids for ``bench.py``: a read-bandwidth probe).
Sources are compiled in parallel.
"""
from __future__ import annotations

import glob
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libspecverify.so")
BENCH_LIB = os.path.join(PKG, "libsvbench.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# Packed fp32 VALU forms are disabled for every device compile.
DEVICE_FLAGS = ["--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function"]


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip"))) + [os.path.join(CSRC, "api.cpp")]


def bench_sources():
    return sorted(glob.glob(os.path.join(CSRC, "bench", "*.hip")))


def _jobs() -> int:
    for var in ("MAX_JOBS", "OMP_NUM_THREADS"):
        v = os.environ.get(var)
        if v and v.isdigit() and int(v) > 0:
            return min(int(v), 16)
    return max(1, min(8, len(os.sched_getaffinity(0))))


def _compile(src, obj, extra, verbose):
    lang = ["-x", "hip"] if src.endswith(".hip") else []
    cmd = [HIPCC, *COMMON, *DEVICE_FLAGS, *extra, *lang, "-c", src, "-o", obj]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return obj


def _link(objs, out, verbose):
    tmp = out + ".tmp"
    cmd = [HIPCC, "-shared", "-fPIC", *DEVICE_FLAGS, *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)


def build(verbose: bool = False, extra=()) -> str:
    """Compile both libraries; returns the verification library's path.
    Always recompiles."""
    objdir = os.path.join(PKG, "_build")
    os.makedirs(objdir, exist_ok=True)
    groups = {LIB: sources(), BENCH_LIB: bench_sources()}
    work = [(out, src, os.path.join(objdir, os.path.basename(src) + ".o")) for out, srcs in groups.items()
            for src in srcs]
    with ThreadPoolExecutor(max_workers=_jobs()) as pool:
        futures = [pool.submit(_compile, src, obj, extra, verbose) for _, src, obj in work]
        for f in futures:
            f.result()
    for out in groups:
        _link([obj for o, _, obj in work if o == out], out, verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
