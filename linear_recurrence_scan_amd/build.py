"""Builds librlscan.so in-tree with hipcc for gfx950.

Usage: ``python -m linear_recurrence_scan_amd.build`` (or ``build()`` from
Python).  Each HIP source compiles to its own object, in parallel; the host
API is compiled and everything linked into one shared object next to this
file, where the ctypes binding looks for it.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "librlscan.so")
# The same library with per-tile phase stamps compiled in (profiling only).
STAMPS_LIB = os.path.join(HERE, "librlscan_stamps.so")
HIP_SOURCES = ["op_gae.hip", "op_gae_skip.hip", "op_gae_compact.hip", "op_gae_norm.hip", "op_gae_norm_one.hip", "op_vtrace.hip", "op_vtrace_clip.hip", "op_returns.hip",
               "op_prefix.hip", "op_retrace.hip", "op_traces_vec.hip", "aux_kernels.hip",
               "noalloc.hip"]
HOST_SOURCES = ["rlscan_api.cpp"]
ARCH = os.environ.get("RLSCAN_OFFLOAD_ARCH", "gfx950")


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found: install ROCm or set HIPCC")


def _common(defines) -> list[str]:
    return [
        hipcc(), f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        "-Wall", "-Wno-unused-parameter",
        # packed fp32 VALU forms stay disabled in every HIP translation unit
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        # the look-back atomics are issued by one lane; the compiler's
        # wave-level aggregation of atomics made the ticket's add wait for its
        # return at tile start, ahead of the tile's data loads
        "-mllvm", "-amdgpu-atomic-optimizer-strategy=None",
        *[f"-D{d}" for d in defines],
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    proc = subprocess.run(cmd, capture_output=True, text=True)
    if proc.returncode != 0:
        raise RuntimeError(f"hipcc failed ({proc.returncode}): {' '.join(cmd[-3:])}\n"
                           f"{proc.stderr[-6000:]}")
    return proc


def build(verbose: bool = False, out: str = LIB, defines=(), csrc: str = CSRC) -> str:
    """Compiles every source under `csrc` and links `out`.  Returns `out`."""
    with tempfile.TemporaryDirectory(prefix="rlscan_build_") as tmp:
        jobs = []
        for src in HIP_SOURCES + HOST_SOURCES:
            obj = os.path.join(tmp, os.path.splitext(src)[0] + ".o")
            jobs.append((_common(defines) + ["-c", "-x", "hip", os.path.join(csrc, src), "-o", obj],
                         obj))
        workers = min(len(jobs), max(1, min(os.cpu_count() or 1, 8)))
        with ThreadPoolExecutor(max_workers=workers) as pool:
            list(pool.map(lambda j: _run(j[0], verbose), jobs))
        tmp_out = out + f".tmp{os.getpid()}"
        _run(_common(defines) + ["-shared", *[o for _, o in jobs], "-o", tmp_out], verbose)
        os.replace(tmp_out, out)
    return out


def build_stamps(verbose: bool = False) -> str:
    """Builds librlscan_stamps.so: the library with RLSCAN_PHASE_STAMPS."""
    return build(verbose=verbose, out=STAMPS_LIB, defines=("RLSCAN_PHASE_STAMPS",))


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
    if "--stamps" in sys.argv:
        print(build_stamps(verbose="-v" in sys.argv))
