"""Build libswz.so in-tree with hipcc for gfx950.

Usage: python tiled_movement_amd/build.py [--verbose]

Run by path (not with -m): importing the package loads the library, which
may not exist yet.
"""

from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB = os.path.join(HERE, "libswz.so")

SOURCES = [
    "capi.cpp",
    "chooser.cpp",
    "bank_model.cpp",
    "kernels_tile.hip",
    "kernels_gemm.hip",
    "kernels_gemm_tiles.hip",
    "kernels_map.hip",
    "kernels_rows.hip",
    "kernels_copy.hip",
    "lds_probe.hip",
]

ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), shutil.which("hipcc"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found")


def flags():
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-fvisibility=hidden",
        "-Wall",
        "-Wno-unused-function",
        # Packed fp32 VALU ops stay off: the path has no float arithmetic,
        # and the compiler must not introduce them.
        "-Xclang",
        "-target-feature",
        "-Xclang",
        "-packed-fp32-ops",
        # Kernel arguments arrive in SGPRs (gfx950 kernarg preload; the code
        # object keeps an entry that loads them itself where the firmware
        # does not): a tile kernel's wave then needs no scalar memory round
        # trip before its first global load.
        "-mllvm",
        "-amdgpu-kernarg-preload-count=16",
        f"-I{INCLUDE}",
        f"-I{CSRC}",
    ]


def build_test_helper(verbose: bool = False) -> str:
    """The tests' hardware probes (tests/hw_probe.hip -> tests/libhw_probe.so)."""
    src = os.path.join(ROOT, "tests", "hw_probe.hip")
    out = os.path.join(ROOT, "tests", "libhw_probe.so")
    cmd = [hipcc()] + flags() + ["-shared", "-o", out + ".tmp", "-x", "hip", src]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


def build(verbose: bool = False, out: str = LIB, extra=()) -> str:
    """Compile every source to an object (in parallel: each is its own
    translation unit, kernels launched from the file that defines them),
    then link one shared library; returns its path."""
    objdir = os.path.join(HERE, "_build", os.path.basename(out) + ".objs")
    os.makedirs(objdir, exist_ok=True)
    jobs = []
    for s in SOURCES:
        obj = os.path.join(objdir, s + ".o")
        # hipcc compiles .cpp as HIP too; the host files include hip_runtime.h.
        jobs.append((obj, [hipcc()] + flags() + list(extra) + ["-c", "-o", obj, "-x", "hip", os.path.join(CSRC, s)]))
    workers = max(1, min(len(jobs), os.cpu_count() or 1, 16))
    with concurrent.futures.ThreadPoolExecutor(workers) as pool:
        for obj, cmd in jobs:
            if verbose:
                print(" ".join(cmd), flush=True)
        for r in pool.map(lambda c: subprocess.run(c, capture_output=True, text=True), [c for _, c in jobs]):
            if r.stderr:
                sys.stderr.write(r.stderr)
            r.check_returncode()
    link = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-o", out + ".tmp"] + [o for o, _ in jobs]
    if verbose:
        print(" ".join(link), flush=True)
    subprocess.run(link, check=True)
    os.replace(out + ".tmp", out)
    return out


if __name__ == "__main__":
    print(build(verbose="--verbose" in sys.argv))
    print(build_test_helper(verbose="--verbose" in sys.argv))
