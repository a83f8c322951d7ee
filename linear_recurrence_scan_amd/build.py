"""Builds librlscan.so in-tree with hipcc for gfx950.

Usage: ``python -m linear_recurrence_scan_amd.build`` (or ``build()`` from
Python).  The shared object lands next to this file, where the ctypes binding
looks for it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librlscan.so")
SOURCES = ["rlscan_kernels.hip", "rlscan_api.cpp"]
ARCH = os.environ.get("RLSCAN_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def command(out: str, defines=()) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
        "-Wall", "-Wno-unused-parameter",
        # packed fp32 VALU forms stay disabled in every HIP translation unit
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        *[f"-D{d}" for d in defines],
        "-x", "hip", *[os.path.join(CSRC, s) for s in SOURCES],
        "-o", out,
    ]


def build(verbose: bool = False, out: str = LIB, defines=()) -> str:
    tmp = out + f".tmp{os.getpid()}"
    cmd = command(tmp, defines)
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}):\n{proc.stderr[-6000:]}")
    if verbose and proc.stderr.strip():
        print(proc.stderr[-3000:], file=sys.stderr)
    os.replace(tmp, out)
    return out


if __name__ == "__main__":
    print(build(verbose=True))
