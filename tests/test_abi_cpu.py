"""The C ABI on the CPU: the library loads, exports every symbol that
include/mbok.h declares, and rejects bad arguments on the host before any
launch.  No call here reaches a kernel."""
import ctypes
import os
import re
import subprocess

import pytest

import boolean_weight_amd as bw
import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mbok.h")


def header_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mbok_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return bw.load_library()


def test_header_declares_the_boundary():
    fns = header_functions()
    for name in ("mbok_residual_binarize", "mbok_refit", "mbok_pack", "mbok_gemv", "mbok_gemm"):
        assert name in fns


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", bw.library_path()],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mbok_[a-z0-9_]+)\b", out))
    for name in header_functions():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_header_compiles_as_c(tmp_path):
    src = tmp_path / "t.c"
    src.write_text('#include "mbok.h"\nint main(void){mbok_desc d; return mbok_desc_init(&d,1,128,1,MBOK_F16);}\n')
    r = subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER),
                        "-c", str(src), "-o", str(tmp_path / "t.o")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


def test_version_and_status_strings(lib):
    assert "mbok" in bw.mbok_version()
    for code in (0, -1, -2, -3, -4, -5, -6):
        s = bw.mbok_status_str(code)
        assert s.startswith("MBOK_"), s
    assert bw.mbok_status_str(-99) == "unknown status"


@pytest.mark.parametrize("m,n,K,dt,err", [
    (0, 128, 1, bw.MBOK_F16, -2), (5, 100, 1, bw.MBOK_F16, -2), (5, 0, 1, bw.MBOK_F16, -2),
    (5, 128 * 3 + 1, 1, bw.MBOK_F16, -2), (5, 128, 0, bw.MBOK_F16, -6),
    (5, 128, 5, bw.MBOK_F16, -6), (5, 128, 2, bw.MBOK_BF16, -3), (5, 128, 2, 7, -3),
    ((1 << 24) + 1, 128, 1, bw.MBOK_F32, -2),
])
def test_desc_init_rejects(m, n, K, dt, err):
    with pytest.raises(bw.MbokError) as e:
        bw.mbok_desc_init(m, n, K, dt)
    assert e.value.status == err


def test_desc_init_null(lib):
    assert lib.mbok_desc_init(None, 4, 128, 1, bw.MBOK_F16) == -1


@pytest.mark.parametrize("m,n,K,dt", [(1, 128, 1, "f32"), (65, 256, 2, "f16"), (4096, 4096, 2, "f16"),
                                      (11008, 4096, 3, "f16"), (5120, 13824, 3, "f16"),
                                      (256, 512, 4, "f32")])
def test_sizes_match_layout_spec(m, n, K, dt):
    d = bw.mbok_desc_init(m, n, K, bw.MBOK_F16 if dt == "f16" else bw.MBOK_F32)
    assert bw.mbok_packed_bytes(d) == oracle.packed_nbytes(m, n, K, dt)
    assert bw.mbok_alpha_bytes(d) == K * m * (n // 128) * (2 if dt == "f16" else 4)


def test_sizes_of_invalid_desc_are_zero(lib):
    d = bw.mbok_desc(m=4, n=100, K=1, group=128, alpha_dtype=1, layout=1)
    assert lib.mbok_packed_bytes(ctypes.byref(d)) == 0
    assert lib.mbok_alpha_bytes(ctypes.byref(d)) == 0
    assert lib.mbok_packed_bytes(None) == 0


def _desc(**kw):
    d = bw.mbok_desc_init(64, 256, 2, bw.MBOK_F16)
    for k, v in kw.items():
        setattr(d, k, v)
    return d


# Fake device addresses: validation must reject the call before anything is
# launched, so these are never dereferenced.
A16 = 0x7f0000000000
MIS = A16 + 2


def test_compute_calls_validate_before_launch(lib):
    d = _desc()
    R = ctypes.byref
    # NULL pointers
    assert lib.mbok_gemv(R(d), None, A16, bw.MBOK_BF16, A16, None, None) == -1
    assert lib.mbok_gemv(R(d), A16, None, bw.MBOK_BF16, A16, None, None) == -1
    assert lib.mbok_gemv(R(d), A16, A16, bw.MBOK_BF16, None, None, None) == -1
    assert lib.mbok_gemm(R(d), None, A16, bw.MBOK_BF16, 4, 256, A16, 64, None) == -1
    assert lib.mbok_pack(R(d), None, A16, A16, None) == -1
    assert lib.mbok_residual_binarize(R(d), None, 256, A16, A16, None, None) == -1
    # bad dtype
    assert lib.mbok_gemv(R(d), A16, A16, bw.MBOK_F16, A16, None, None) == -3
    assert lib.mbok_gemm(R(d), A16, A16, bw.MBOK_F32, 4, 256, A16, 64, None) == -3
    # misalignment
    assert lib.mbok_gemv(R(d), MIS, A16, bw.MBOK_BF16, A16, None, None) == -4
    assert lib.mbok_gemv(R(d), A16, MIS, bw.MBOK_BF16, A16, None, None) == -4
    assert lib.mbok_gemv(R(d), A16, A16, bw.MBOK_BF16, A16 + 1, None, None) == -4
    assert lib.mbok_gemv(R(d), A16, A16, bw.MBOK_BF16, A16, A16 + 16, None) == -4
    assert lib.mbok_gemm(R(d), A16, A16, bw.MBOK_BF16, 4, 260, A16, 64, None) == -4
    assert lib.mbok_pack(R(d), MIS, A16, A16, None) == -4
    assert lib.mbok_residual_binarize(R(d), A16, 258, A16, A16, None, None) == -4
    assert lib.mbok_residual_binarize(R(d), A16, 256, A16, A16, A16 + 2, None) == -4
    # shapes and leading dimensions
    assert lib.mbok_gemm(R(d), A16, A16, bw.MBOK_BF16, 0, 256, A16, 64, None) == -2
    assert lib.mbok_gemm(R(d), A16, A16, bw.MBOK_BF16, 65537, 256, A16, 64, None) == -2
    assert lib.mbok_gemm(R(d), A16, A16, bw.MBOK_BF16, 4, 128, A16, 64, None) == -1
    assert lib.mbok_gemm(R(d), A16, A16, bw.MBOK_BF16, 4, 256, A16, 63, None) == -1
    assert lib.mbok_residual_binarize(R(d), A16, 128, A16, A16, None, None) == -1
    # the refit: NULLs, leading dimension, rounds, alignment
    assert lib.mbok_refit(R(d), None, 256, A16, A16, 2, None) == -1
    assert lib.mbok_refit(R(d), A16, 256, None, A16, 2, None) == -1
    assert lib.mbok_refit(R(d), A16, 256, A16, None, 2, None) == -1
    assert lib.mbok_refit(R(d), A16, 128, A16, A16, 2, None) == -1
    assert lib.mbok_refit(R(d), A16, 256, A16, A16, -1, None) == -1
    assert lib.mbok_refit(R(d), A16, 256, A16, A16, bw.MBOK_MAX_REFIT_ROUNDS + 1, None) == -1
    assert lib.mbok_refit(R(d), A16, 258, A16, A16, 2, None) == -4
    assert lib.mbok_refit(R(d), A16, 256, MIS, A16, 2, None) == -4
    assert lib.mbok_refit(R(d), A16, 256, A16, MIS, 2, None) == -4
    assert lib.mbok_refit(R(_desc(K=5)), A16, 256, A16, A16, 2, None) == -6
    # descriptors edited by hand
    assert lib.mbok_gemv(R(_desc(group=64)), A16, A16, bw.MBOK_BF16, A16, None, None) == -6
    assert lib.mbok_gemv(R(_desc(layout=2)), A16, A16, bw.MBOK_BF16, A16, None, None) == -6
    assert lib.mbok_gemv(R(_desc(K=9)), A16, A16, bw.MBOK_BF16, A16, None, None) == -6
    assert lib.mbok_gemv(R(_desc(n=200)), A16, A16, bw.MBOK_BF16, A16, None, None) == -2
    assert lib.mbok_gemv(R(_desc(alpha_dtype=2)), A16, A16, bw.MBOK_BF16, A16, None, None) == -3
    assert lib.mbok_gemv(None, A16, A16, bw.MBOK_BF16, A16, None, None) == -1


def test_binding_refuses_host_tensors():
    import torch
    d = bw.mbok_desc_init(64, 256, 2, bw.MBOK_F16)
    with pytest.raises(ValueError):
        bw.mbok_gemv(d, torch.zeros(10, dtype=torch.uint8), torch.zeros(256),
                     torch.zeros(64))
