"""Build libmhc.so (gfx950) in-tree with hipcc.

    python -m manifold_constrained_hyper_mhc_amd.build

Every HIP translation unit is compiled with packed fp32 instructions
disabled; the shared library lands next to this file.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libmhc.so")
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["mhc_kernels.hip", "mhc_api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def common_flags():
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", os.path.join(ROOT, "include"),
    ]


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{err}")
    if err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        cmd = [cc, *common_flags(), "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print("[build]", " ".join(cmd), flush=True)
        _run(cmd)
        objs.append(obj)
    tmp = LIB + ".tmp"
    cmd = [cc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    _run(cmd)
    os.replace(tmp, LIB)
    build_bench_helper(cc, verbose)
    build_test_helpers(cc, verbose)
    return LIB


# The measurement aid of bench.py (plain copies for the bandwidth ceilings),
# a library of its own next to libmhc.so.
BENCH_LIB = os.path.join(HERE, "libmhc_bench.so")


def build_bench_helper(cc: str, verbose: bool = True) -> None:
    tmp = BENCH_LIB + ".tmp"
    cmd = [cc, *common_flags(), "-shared", "-x", "hip", os.path.join(CSRC, "bench_copy.hip"), "-o", tmp]
    if verbose:
        print("[build]", " ".join(cmd), flush=True)
    _run(cmd)
    os.replace(tmp, BENCH_LIB)


# Test-only HIP helpers (not part of libmhc): built next to their source in
# tests/, loaded only by the GPU tests.
TEST_HELPERS = [("mx_consumer.hip", "libmx_consumer.so")]


def build_test_helpers(cc: str, verbose: bool = True) -> None:
    tests = os.path.join(ROOT, "tests")
    for src, lib in TEST_HELPERS:
        out = os.path.join(tests, lib)
        tmp = out + ".tmp"
        cmd = [cc, *common_flags(), "-shared", "-x", "hip", os.path.join(tests, src), "-o", tmp]
        if verbose:
            print("[build]", " ".join(cmd), flush=True)
        _run(cmd)
        os.replace(tmp, out)


if __name__ == "__main__":
    print(build())
