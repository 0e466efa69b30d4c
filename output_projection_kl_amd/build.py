"""Build libfkl.so in-tree with hipcc for gfx950.

Usage: python -m output_projection_kl_amd.build [-v] [--debug]

--debug builds libfkl_debug.so instead: the same sources with FKL_DEBUG
defined, whose kernels check their global accesses against the extents the
host planned and whose entry points report any that fall outside
(csrc/fkl_debug.h).
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIB_PATH = os.path.join(PKG_DIR, "libfkl.so")
DEBUG_BUILD_DIR = os.path.join(ROOT, "_build_debug")
DEBUG_LIB_PATH = os.path.join(PKG_DIR, "libfkl_debug.so")

SOURCES = ["fkl_kernels.hip", "fkl_topk.hip", "fkl_api.cpp", "fkl_trace.cpp"]
ARCH = "gfx950"


def _hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    raise RuntimeError("hipcc not found (ROCm is required to build libfkl)")


def _common_flags() -> list[str]:
    return [
        f"--offload-arch={ARCH}",
        "-O3",
        "-std=c++17",
        "-fPIC",
        "-Wall",
        "-Wno-unused-function",
        # keep the compiler from emitting packed fp32 ALU ops
        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
        "-I", INCLUDE,
        "-I", CSRC,
    ]


def build(verbose: bool = False, debug: bool = False) -> str:
    """Compile every source and link libfkl.so (libfkl_debug.so with debug)
    next to this file. Returns its path."""
    hipcc = _hipcc()
    build_dir = DEBUG_BUILD_DIR if debug else BUILD_DIR
    lib_path = DEBUG_LIB_PATH if debug else LIB_PATH
    os.makedirs(build_dir, exist_ok=True)
    flags = _common_flags() + (["-DFKL_DEBUG"] if debug else [])

    def compile_one(src: str) -> str:
        obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
        cmd = [hipcc, *flags, "-c", os.path.join(CSRC, src), "-o", obj]
        if src.endswith(".hip"):
            cmd[1:1] = ["-x", "hip"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, capture_output=True, text=True)
        if r.returncode != 0:
            raise RuntimeError(f"hipcc failed on {src}:\n{r.stdout}\n{r.stderr}")
        if verbose and r.stderr.strip():
            print(r.stderr, file=sys.stderr)
        return obj

    with ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(compile_one, SOURCES))
    tmp = lib_path + ".tmp"
    cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib_path)
    return lib_path


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv, debug="--debug" in sys.argv))
