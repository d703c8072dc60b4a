"""Builds the MBOK HIP library in-tree: boolean_weight_amd/libmbok.so for gfx950.

Run as `python -m boolean_weight_amd.build` or through __graft_entry__.build().
Every call recompiles (the objects go to _build/ at the repository root).
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
BUILD_DIR = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libmbok.so")
# measurement only: the part's own ceilings (read stream, matrix cores, launch)
CEILINGS_LIB = os.path.join(PKG, "libmbok_ceilings.so")
CEILINGS_SOURCES = ["ceilings.hip"]

SOURCES = ["mbok_api.cpp", "allocate.cpp", "quantize.hip", "refit.hip", "svid.hip", "pack.hip", "gemv.hip", "gemv_f4.hip", "gemvt.hip", "gemm.hip", "skinny.hip"]
ARCH = "gfx950"

COMMON = [
    "-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
    "-Wall", "-Wno-unused-function",
    # no packed fp32 instructions anywhere in the device code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # the first kernel arguments arrive preloaded in SGPRs at wave launch,
    # so the address arithmetic does not wait for a kernarg load (about
    # 0.45 us of a 4096 x 4096 decode call); code objects keep the loading
    # prologue for firmware without preload
    "-mllvm", "-amdgpu-kernarg-preload-count=16",
]


def hipcc() -> str:
    path = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(path):
        raise RuntimeError("hipcc not found: the MBOK library needs ROCm's hipcc")
    return path


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(lib: str, objs: list[str]) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"linking failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source, link libmbok.so and the ceilings library;
    returns the MBOK library path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    # a failed build must not leave an older library behind to be loaded
    for lib in (LIB, CEILINGS_LIB):
        if os.path.exists(lib):
            os.remove(lib)
    extra = list(extra or [])
    every = SOURCES + CEILINGS_SOURCES
    with ThreadPoolExecutor(max_workers=min(8, len(every))) as ex:
        objs = dict(zip(every, ex.map(lambda s: _compile(s, extra), every)))
    _link(LIB, [objs[s] for s in SOURCES])
    _link(CEILINGS_LIB, [objs[s] for s in CEILINGS_SOURCES])
    if verbose:
        print(f"built {LIB} and {CEILINGS_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
