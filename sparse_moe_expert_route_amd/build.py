"""Build libmoe_mi355x.so for gfx950 with hipcc, in-tree.

    python -m sparse_moe_expert_route_amd.build

The library lands in sparse_moe_expert_route_amd/lib/.  Cross-compiles
without a GPU.
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_DIR = os.path.join(PKG, "lib")
LIB_NAME = "libmoe_mi355x.so"
LIB_PATH = os.path.join(LIB_DIR, LIB_NAME)

SOURCES = ["ffn.hip", "route.hip", "dense.hip", "pack.hip", "calib.hip", "residual.hip",
           "noalloc.hip", "api.cpp"]
ARCH = "gfx950"


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build the HIP library)")


def flags() -> list:
    return [
        f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
        # packed fp32 VALU ops are kept out of every kernel
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-Wall", "-Wextra", "-Wno-unused-function",
        "-I", INCLUDE, "-I", CSRC,
    ]


def _run(cmd, verbose):
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError(f"hipcc failed with exit code {res.returncode}: {' '.join(cmd)}")


def build(verbose: bool = False) -> str:
    """Compile every source to an object under lib/obj (in parallel), link
    the shared library."""
    from concurrent.futures import ThreadPoolExecutor
    obj_dir = os.path.join(LIB_DIR, "obj")
    os.makedirs(obj_dir, exist_ok=True)
    objs = [os.path.join(obj_dir, s + ".o") for s in SOURCES]
    jobs = max(1, min(len(SOURCES), len(os.sched_getaffinity(0)), 8))
    with ThreadPoolExecutor(jobs) as ex:
        list(ex.map(lambda so: _run([hipcc()] + flags() + ["-c", os.path.join(CSRC, so[0]), "-o",
                                                           so[1]], verbose),
                    zip(SOURCES, objs)))
    tmp = LIB_PATH + ".tmp"
    _run([hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC"] + objs + ["-o", tmp], verbose)
    os.replace(tmp, LIB_PATH)
    return LIB_PATH


if __name__ == "__main__":
    print(build(verbose=True))
