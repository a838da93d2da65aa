"""Build libpagedkv.so in-tree: HIP kernels for gfx950 plus the host C++ parts.

    python -m paged_kv_cache_411_amd.build

HIP sources are compiled with hipcc for gfx950 only; the host-only sources
(allocator, error state) with g++ so they stay free of HIP. Objects go to
``_build/`` next to this file, the shared library to
``paged_kv_cache_411_amd/libpagedkv.so``; the benchmark's gather probe (for
counter calibration, not part of the decode path) goes to its own
``libpagedkv_probe.so``. Every call rebuilds everything.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OUT_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")
ARCH = "gfx950"

HIP_SOURCES = ["pa_decode.hip", "kv_ops.hip"]
HOST_SOURCES = ["block_allocator.cpp", "decode_step.cpp", "schedule.cpp", "status.cpp"]
# measurement only (the benchmark's counter calibration): its own library
PROBE_SOURCES = ["probe_gather.hip"]
PROBE_LIB = os.path.join(PKG, "libpagedkv_probe.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HIP_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall",
    # keep hipcc from forming packed fp32 instructions on its own
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]
HOST_FLAGS = ["-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra", "-I", INCLUDE, "-I", CSRC]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    # hipcc's host pass warns that it does not know the gfx feature: harmless
    err = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"build failed: {' '.join(cmd)}\n{err}")
    if verbose and err.strip():
        print(err, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source and link libpagedkv.so; returns its path."""
    os.makedirs(OUT_DIR, exist_ok=True)
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        jobs.append(([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    for src in HOST_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        jobs.append((["g++", *HOST_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    probe_jobs = []
    for src in PROBE_SOURCES:
        obj = os.path.join(OUT_DIR, src + ".o")
        probe_jobs.append(([HIPCC, *HIP_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj], obj))
    with ThreadPoolExecutor(max_workers=min(8, len(jobs) + len(probe_jobs))) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs + probe_jobs))
    for out, objs in ((LIB, jobs), (PROBE_LIB, probe_jobs)):
        tmp = out + ".tmp"
        _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *[o for _, o in objs]], verbose)
        os.replace(tmp, out)
    return LIB


def clean() -> None:
    shutil.rmtree(OUT_DIR, ignore_errors=True)
    for f in (LIB, PROBE_LIB):
        if os.path.exists(f):
            os.remove(f)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
