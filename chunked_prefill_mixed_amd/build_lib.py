"""Compile libcpa.so for gfx950 in-tree.

HIP sources are compiled with hipcc (one process per file, in parallel); the
host-only work planner is compiled with g++ so it provably needs no HIP
runtime; everything is linked into ``chunked_prefill_mixed_amd/libcpa.so``.
The bench's measured-ceiling kernels go into ``libcpa_peaks.so``.
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
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libcpa.so")
PEAKS_LIB = os.path.join(PKG, "libcpa_peaks.so")

HIP_SOURCES = ["append.hip", "decode.hip", "chunk.hip", "mixed.hip", "merge.hip", "abi.hip"]
HOST_SOURCES = ["builder.cpp"]
ARCH = os.environ.get("CPA_OFFLOAD_ARCH", "gfx950")

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-fPIC", "-std=c++17", "-Wall", "-Wno-unused-result",
    # code object v5 loads in both the ROCm 7.2 runtime and the one bundled with torch
    "-mcode-object-version=5",
    # packed fp32 VALU forms stay off: the compiler may not emit v_pk_{add,mul,fma}_f32
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"),
]
# per-source additions: the decode kernel's small 16x16 MFMA accumulators are
# kept in ordinary VGPRs (no accumulator-register copies around every MFMA)
FILE_FLAGS = {"decode.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form=1"]}
GXX_FLAGS = ["-O2", "-fPIC", "-std=c++17", "-Wall", "-I", os.path.join(ROOT, "include")]


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libcpa.so)")


def _run(cmd: list[str]) -> None:
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in r.stdout.splitlines()
                    if "packed-fp32-ops" not in line)  # host-pass notice about the feature flag
    if r.returncode != 0:
        raise RuntimeError(f"command failed ({r.returncode}): {' '.join(cmd)}\n{out}")
    if out.strip():
        print(out, file=sys.stderr)


def build(verbose: bool = False) -> str:
    """Compile every source and link libcpa.so; returns its path.

    CPA_HIPCC_EXTRA (environment) adds hipcc flags, e.g. -D overrides of the
    kernels' compile-time tuning macros."""
    os.makedirs(BUILD, exist_ok=True)
    hipcc = _hipcc()
    extra = os.environ.get("CPA_HIPCC_EXTRA", "").split()
    jobs = []
    for src in HIP_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        jobs.append([hipcc, *HIPCC_FLAGS, *FILE_FLAGS.get(src, []), *extra, "-c",
                     os.path.join(CSRC, src), "-o", obj])
    for src in HOST_SOURCES:
        obj = os.path.join(BUILD, src.replace(".cpp", ".host.o"))
        jobs.append(["g++", *GXX_FLAGS, "-c", os.path.join(CSRC, src), "-o", obj])
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    with ThreadPoolExecutor(workers) as ex:
        for cmd in jobs:
            if verbose:
                print(" ".join(cmd))
        list(ex.map(_run, jobs))
    objs = [j[-1] for j in jobs]
    tmp = LIB + ".tmp"
    _run([hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    # the bench's measured ceilings (streaming copy, MFMA-only loop): a separate
    # library, not part of the attention path
    tmp = PEAKS_LIB + ".tmp"
    _run([hipcc, *HIPCC_FLAGS, *extra, "-shared", os.path.join(CSRC, "peaks.hip"), "-o", tmp])
    os.replace(tmp, PEAKS_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
