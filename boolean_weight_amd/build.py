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


def _compile(src: str, extra: list[str], out_dir: str = BUILD_DIR) -> str:
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    cmd = [hipcc(), *COMMON, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(lib: str, objs: list[str], extra: list[str] | None = None) -> None:
    tmp = lib + ".tmp"
    cmd = [hipcc(), "-shared", f"--offload-arch={ARCH}", *(extra or []), "-o", tmp, *objs]
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


# Host-side sanitizers only: each -fsanitize= applies to the host pass of
# hipcc (the device code is built as usual).  The library then expects the
# clang AddressSanitizer runtime in the process (LD_PRELOAD of
# sanitizer_runtime()).
SANITIZE_HOST = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                 "-Xarch_host", "-fno-sanitize-recover=undefined",
                 "-Xarch_host", "-fno-omit-frame-pointer", "-g"]
SANITIZED_DIR = os.path.join(BUILD_DIR, "sanitized")


def sanitizer_runtime() -> str | None:
    """The clang AddressSanitizer runtime of ROCm's LLVM, or None."""
    base = "/opt/rocm/llvm/lib/clang"
    if not os.path.isdir(base):
        return None
    for ver in sorted(os.listdir(base), reverse=True):
        path = os.path.join(base, ver, "lib", "linux", "libclang_rt.asan-x86_64.so")
        if os.path.exists(path):
            return path
    return None


def build_sanitized(verbose: bool = False) -> str:
    """libmbok.so with AddressSanitizer and UndefinedBehaviorSanitizer on the
    host code (argument checks, descriptor and size arithmetic, the kernel
    allocator, the launchers), under _build/sanitized/; returns its path.
    Load it with MBOK_LIBRARY=<path> and the runtime preloaded."""
    os.makedirs(SANITIZED_DIR, exist_ok=True)
    lib = os.path.join(SANITIZED_DIR, "libmbok.so")
    if os.path.exists(lib):
        os.remove(lib)
    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda s: _compile(s, SANITIZE_HOST, SANITIZED_DIR), SOURCES))
    _link(lib, objs, ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
                      "-shared-libsan"])
    if verbose:
        print(f"built {lib}")
    return lib


if __name__ == "__main__":
    if sys.argv[1:2] == ["sanitized"]:
        build_sanitized(verbose=True)
    else:
        build(verbose=True, extra=sys.argv[1:])
