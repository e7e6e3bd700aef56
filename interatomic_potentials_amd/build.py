"""Build libe2f.so (HIP kernels for gfx950 + the C-ABI host code) in place.

Usage:  python interatomic_potentials_amd/build.py [--verbose]

(Run it as a file: importing the package itself needs the built library.)

The library lands next to this file, so it travels with the source tree.
Every HIP translation unit is compiled with packed-FP32 instructions turned
off (``-Xclang -target-feature -Xclang -packed-fp32-ops``).
"""

from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libe2f.so")
ARCH = os.environ.get("E2F_OFFLOAD_ARCH", "gfx950")

ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
HIPCC = shutil.which("hipcc") or f"{ROCM}/bin/hipcc"
COMMON = ["-O3", "-std=c++17", "-fPIC", f"-I{INCLUDE}", f"-I{CSRC}"]
DEVICE = ["-x", "hip", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-munsafe-fp-atomics"]

SOURCES = [
    ("e2f_kernels.hip", True),
    ("e2f_aggregate_generic.hip", True),
    ("e2f_aggregate_tile.hip", True),
    ("e2f_backward.hip", True),
    ("e2f_project.hip", True),
    ("e2f_project_bwd.hip", True),
    ("e2f_neighbours.hip", True),
    ("e2f_dense.hip", True),
    ("e2f_noalloc.hip", True),
    ("e2f_host.cpp", False),
]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        raise RuntimeError(f"command failed ({res.returncode}): {' '.join(cmd)}\n"
                           f"{res.stdout}\n{res.stderr}")
    return res


def build(verbose: bool = False) -> str:
    """Compile every source and link libe2f.so; returns the library path."""
    os.makedirs(BUILD, exist_ok=True)
    jobs = []
    for name, is_hip in SOURCES:
        src = os.path.join(CSRC, name)
        obj = os.path.join(BUILD, name + ".o")
        host = ["-x", "c++", "-D__HIP_PLATFORM_AMD__",  # plain C++ against the HIP runtime API
                f"-I{ROCM}/include"]
        cmd = [HIPCC] + COMMON + (DEVICE if is_hip else host) + ["-c", src, "-o", obj]
        jobs.append((cmd, obj))
    with cf.ThreadPoolExecutor(max_workers=min(len(jobs), 8)) as ex:
        list(ex.map(lambda j: _run(j[0], verbose), jobs))
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + [o for _, o in jobs],
         verbose)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    path = build(verbose="--verbose" in sys.argv)
    print(path)
