"""The C ABI's host code under AddressSanitizer and UndefinedBehaviorSanitizer.

libmbok.so is rebuilt with both sanitizers on its host code (argument checks,
descriptor and size arithmetic, the kernel-count allocator, the launchers;
device code is built as usual) and the CPU tests of the ABI run against it in
a child process: any out-of-bounds access, use after free, signed overflow or
other undefined behaviour on those paths ends the child with a report.  No GPU
is needed: with none present every compute call stops at its host checks.
"""
import glob
import os
import subprocess
import sys

import pytest

from boolean_weight_amd import build as B

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


def _sanitized_library() -> str:
    lib = os.path.join(B.SANITIZED_DIR, "libmbok.so")
    sources = [os.path.join(B.CSRC, s) for s in B.SOURCES]
    sources += glob.glob(os.path.join(B.CSRC, "*.h")) + glob.glob(os.path.join(ROOT, "include", "*.h"))
    sources.append(B.__file__)
    if not os.path.exists(lib) or os.path.getmtime(lib) < max(map(os.path.getmtime, sources)):
        lib = B.build_sanitized()
    return lib


def _env(lib: str, runtime: str) -> dict:
    env = dict(os.environ)
    env.update(MBOK_LIBRARY=lib, LD_PRELOAD=runtime,
               ASAN_OPTIONS="detect_leaks=0:halt_on_error=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1",
               HIP_VISIBLE_DEVICES="")
    return env


@pytest.fixture(scope="module")
def sanitized():
    runtime = B.sanitizer_runtime()
    if runtime is None:
        pytest.skip("ROCm's clang AddressSanitizer runtime is not installed")
    try:
        B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not found")
    return _sanitized_library(), runtime


def test_sanitized_library_is_the_one_loaded(sanitized):
    lib, runtime = sanitized
    probe = ("import boolean_weight_amd as bw; bw.load_library(); "
             "maps = open('/proc/self/maps').read(); "
             f"assert {lib!r} in maps, 'sanitized library not mapped'; "
             "assert 'libclang_rt.asan' in maps, 'sanitizer runtime not mapped'; "
             "print(bw.mbok_version())")
    r = subprocess.run([sys.executable, "-c", probe], cwd=ROOT, env=_env(lib, runtime),
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stdout[-3000:] + r.stderr[-3000:]


def test_abi_cpu_tests_pass_under_sanitizers(sanitized):
    lib, runtime = sanitized
    cmd = [sys.executable, "-m", "pytest", os.path.join(HERE, "test_abi_cpu.py"), "-x", "-q",
           "-p", "no:cacheprovider", "-m", "not gpu"]
    r = subprocess.run(cmd, cwd=ROOT, env=_env(lib, runtime), capture_output=True, text=True,
                       timeout=900)
    out = r.stdout[-4000:] + r.stderr[-4000:]
    assert r.returncode == 0, out
    assert "ERROR: AddressSanitizer" not in out and "runtime error:" not in out, out
