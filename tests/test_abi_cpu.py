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
    for code in (0, -1, -2, -3, -4, -5, -6, -7, -8):
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
    # the two-term prefill product takes the same checks
    for args, code in [((None, A16, bw.MBOK_BF16, 4, 256, A16, 64), -1),
                       ((A16, A16, bw.MBOK_F32, 4, 256, A16, 64), -3),
                       ((A16, A16, bw.MBOK_BF16, 4, 260, A16, 64), -4),
                       ((A16, MIS, bw.MBOK_BF16, 4, 256, A16, 64), -4),
                       ((A16, A16, bw.MBOK_BF16, 0, 256, A16, 64), -2),
                       ((A16, A16, bw.MBOK_BF16, 65537, 256, A16, 64), -2),
                       ((A16, A16, bw.MBOK_BF16, 4, 128, A16, 64), -1),
                       ((A16, A16, bw.MBOK_BF16, 4, 256, A16, 63), -1)]:
        assert lib.mbok_gemm_precise(R(d), *args, None) == code, args
    assert lib.mbok_residual_binarize(R(d), A16, 128, A16, A16, None, None) == -1
    # SVID
    assert lib.mbok_svid_decompose(R(d), None, 256, A16, A16, A16, 8, A16, None) == -1
    assert lib.mbok_svid_decompose(R(d), A16, 256, A16, A16, A16, 8, None, None) == -1
    assert lib.mbok_svid_decompose(R(d), A16, 128, A16, A16, A16, 8, A16, None) == -1
    assert lib.mbok_svid_decompose(R(d), A16, 256, A16, A16, A16, 0, A16, None) == -1
    assert lib.mbok_svid_decompose(R(d), A16, 256, A16, A16, A16, 1001, A16, None) == -1
    assert lib.mbok_svid_decompose(R(d), A16, 256, A16, A16, A16, 8, A16 + 16, None) == -4
    assert lib.mbok_svid_decompose(R(d), A16, 256, MIS, A16, A16, 8, A16, None) == -4
    assert lib.mbok_svid_pack(R(d), None, A16, A16, None) == -1
    assert lib.mbok_svid_pack(R(d), A16, A16 + 2, A16, None) == -4
    assert lib.mbok_svid_gemv(R(d), A16, None, A16, bw.MBOK_BF16, A16, None, None) == -1
    assert lib.mbok_svid_gemv(R(d), A16, A16, A16, bw.MBOK_F16, A16, None, None) == -3
    assert lib.mbok_svid_gemv(R(d), A16, A16, A16, bw.MBOK_BF16, A16, A16 + 64, None) == -4
    assert lib.mbok_svid_gemv(R(d), A16, A16 + 8, A16, bw.MBOK_BF16, A16, None, None) == -4
    assert lib.mbok_svid_gemv(R(d), A16, A16, A16 + 8, bw.MBOK_BF16, A16, None, None) == -4
    assert lib.mbok_svid_gemv_workspace_bytes(R(d)) == 0
    assert lib.mbok_svid_workspace_bytes(R(d)) > 0 and lib.mbok_svid_workspace_bytes(None) == 0
    # transposed product
    assert lib.mbok_gemvt(R(d), None, A16, bw.MBOK_BF16, A16, None, None) == -1
    assert lib.mbok_gemvt(R(d), A16, None, bw.MBOK_BF16, A16, None, None) == -1
    assert lib.mbok_gemvt(R(d), A16, A16, bw.MBOK_BF16, None, None, None) == -1
    assert lib.mbok_gemvt(R(d), A16, A16, bw.MBOK_F16, A16, None, None) == -3
    assert lib.mbok_gemvt(R(d), MIS, A16, bw.MBOK_BF16, A16, None, None) == -4
    assert lib.mbok_gemvt(R(d), A16, A16 + 1, bw.MBOK_BF16, A16, None, None) == -4
    assert lib.mbok_gemvt(R(d), A16, A16 + 2, bw.MBOK_F32, A16, None, None) == -4
    assert lib.mbok_gemvt(R(d), A16, A16, bw.MBOK_F32, A16 + 2, None, None) == -4
    assert lib.mbok_gemvt(R(d), A16, A16, bw.MBOK_F32, A16, A16 + 16, None) == -4
    assert lib.mbok_gemvt(R(_desc(K=9)), A16, A16, bw.MBOK_F32, A16, None, None) == -6
    assert lib.mbok_gemvt_workspace_bytes(None) == 0
    # residual energies: NULLs, leading dimension, alignment
    assert lib.mbok_residual_energy(R(d), None, 256, A16, A16, None) == -1
    assert lib.mbok_residual_energy(R(d), A16, 256, None, A16, None) == -1
    assert lib.mbok_residual_energy(R(d), A16, 256, A16, None, None) == -1
    assert lib.mbok_residual_energy(R(d), A16, 128, A16, A16, None) == -1
    assert lib.mbok_residual_energy(R(d), MIS, 256, A16, A16, None) == -4
    assert lib.mbok_residual_energy(R(d), A16, 258, A16, A16, None) == -4
    assert lib.mbok_residual_energy(R(d), A16, 256, A16 + 4, A16, None) == -4
    assert lib.mbok_residual_energy(R(_desc(K=5)), A16, 256, A16, A16, None) == -6
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


def test_missing_library_fails_loudly(tmp_path):
    """Without the built HIP library the binding raises; there is no CPU path."""
    import sys
    code = ("import boolean_weight_amd as bw\n"
            "try:\n"
            "    bw.load_library()\n"
            "except RuntimeError as e:\n"
            "    print('RAISED', e)\n"
            "else:\n"
            "    print('LOADED')\n")
    env = dict(os.environ, MBOK_LIBRARY=str(tmp_path / "absent" / "libmbok.so"))
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "RAISED" in r.stdout and "not built" in r.stdout, r.stdout


def test_binding_refuses_host_tensors():
    import torch
    d = bw.mbok_desc_init(64, 256, 2, bw.MBOK_F16)
    with pytest.raises(ValueError):
        bw.mbok_gemv(d, torch.zeros(10, dtype=torch.uint8), torch.zeros(256),
                     torch.zeros(64))


# ------------------------------------------------ kernel allocation (host)

def _alloc(sizes, errors, budget):
    return bw.mbok_allocate_kernels(sizes, errors, budget)


def test_allocation_matches_oracle_hand_worked():
    import oracle_pins as P
    for name, sizes, kmax, errors, budget, want in P._read_allocations():
        if want is None:
            with pytest.raises(bw.MbokError) as e:
                _alloc(sizes, errors, budget)
            assert e.value.status == -7
        else:
            assert tuple(_alloc(sizes, errors, budget)) == want, (name, budget)


def test_allocation_matches_oracle_random():
    """The library's dynamic program against the oracle's search over every
    K vector, on oracle-side random instances with many exact ties."""
    import numpy as np
    rng = np.random.default_rng(51)
    for trial in range(150):
        L = int(rng.integers(1, 6))
        kmax = int(rng.integers(1, 5))
        sizes = [int(v) for v in rng.integers(1, 6, size=L)]
        # small dyadic values: many equal totals, so the tie rules matter
        errors = [sorted((rng.integers(0, 6, size=kmax) / 4.0).tolist(), reverse=True)
                  for _ in range(L)]
        budget = int(rng.integers(sum(sizes), kmax * sum(sizes) + 2))
        want = oracle.allocate_kernels(errors, sizes, budget, kmax)
        assert tuple(_alloc(sizes, errors, budget)) == want, (trial, sizes, errors, budget)


def test_allocation_exact_sums_beat_float_rounding():
    """Errors whose float64 sums would tie are still ordered by their exact
    sums: 1 + 2^-60 beats 1 in total once 2^-60 is added elsewhere."""
    sizes = [1, 1]
    errors = [[1.0, 2.0 ** -60], [2.0 ** -60, 0.0]]
    # budget 3: (1,2): 1 + 0 = 1; (2,1): 2^-60 + 2^-60 = 2^-59 <- smaller
    assert _alloc(sizes, errors, 3) == [2, 1]
    assert oracle.allocate_kernels(errors, sizes, 3, 2) == (2, 1)


def test_allocation_rejects_bad_arguments(lib):
    import numpy as np
    sz = np.array([4, 4], dtype=np.int64)
    er = np.array([[1.0, 0.5], [1.0, 0.5]])
    out = np.zeros(2, dtype=np.int32)
    A = lambda L, s, e, k, b, o: lib.mbok_allocate_kernels(L, s, e, k, b, o)
    assert A(2, sz.ctypes.data, er.ctypes.data, 2, 16, out.ctypes.data) == 0
    assert list(out) == [2, 2]
    assert A(0, sz.ctypes.data, er.ctypes.data, 2, 16, out.ctypes.data) == -1
    assert A(2, None, er.ctypes.data, 2, 16, out.ctypes.data) == -1
    assert A(2, sz.ctypes.data, er.ctypes.data, 5, 16, out.ctypes.data) == -1
    assert A(2, sz.ctypes.data, er.ctypes.data, 2, -1, out.ctypes.data) == -1
    assert A(2, sz.ctypes.data, er.ctypes.data, 2, 7, out.ctypes.data) == -7
    bad = er.copy()
    bad[1, 1] = np.nan
    assert A(2, sz.ctypes.data, bad.ctypes.data, 2, 16, out.ctypes.data) == -1
    bad[1, 1] = -1.0
    assert A(2, sz.ctypes.data, bad.ctypes.data, 2, 16, out.ctypes.data) == -1
    zs = sz.copy()
    zs[0] = 0
    assert A(2, zs.ctypes.data, er.ctypes.data, 2, 16, out.ctypes.data) == -1


def test_allocation_many_weights_is_fast():
    """A whole 32-layer model of seven linears each (224 weights, config-4
    sizes in units of 5120 x 512 entries) allocates in well under a second."""
    import time
    import numpy as np
    rng = np.random.default_rng(52)
    sizes = [10, 10, 10, 10, 27, 27, 27] * 32
    errors = []
    for sz in sizes:
        e0 = sz * (1.0 + 0.2 * rng.random())
        errors.append([e0 * 0.36, e0 * 0.13, e0 * 0.057, e0 * 0.024])
    budget = int(2.5 * sum(sizes))
    t0 = time.perf_counter()
    K = _alloc(sizes, errors, budget)
    assert time.perf_counter() - t0 < 5.0
    assert sum(k * s for k, s in zip(K, sizes)) <= budget
    assert min(K) >= 1 and max(K) <= 4


def test_gemvt_noalloc_validates_before_launch(lib):
    """The no-allocation transposed product checks its arguments on the host
    (before looking up the device scratch) exactly as mbok_gemvt does."""
    d = _desc()
    R = ctypes.byref
    assert lib.mbok_gemvt_noalloc(R(d), None, A16, bw.MBOK_BF16, A16, None) == -1
    assert lib.mbok_gemvt_noalloc(R(d), A16, None, bw.MBOK_BF16, A16, None) == -1
    assert lib.mbok_gemvt_noalloc(R(d), A16, A16, bw.MBOK_BF16, None, None) == -1
    assert lib.mbok_gemvt_noalloc(R(d), A16, A16, bw.MBOK_F16, A16, None) == -3
    assert lib.mbok_gemvt_noalloc(R(d), MIS, A16, bw.MBOK_BF16, A16, None) == -4
    assert lib.mbok_gemvt_noalloc(R(d), A16, A16 + 1, bw.MBOK_BF16, A16, None) == -4
    assert lib.mbok_gemvt_noalloc(R(d), A16, A16, bw.MBOK_F32, A16 + 2, None) == -4
    assert lib.mbok_gemvt_noalloc(R(_desc(K=9)), A16, A16, bw.MBOK_BF16, A16, None) == -6
    assert lib.mbok_gemvt_noalloc(None, A16, A16, bw.MBOK_BF16, A16, None) == -1


def test_gemvt_static_scratch_covers_every_shape():
    """The static scratch (512 KiB) holds the workspace of every shape the
    descriptor accepts: n over all 8192 group counts, m from one row block to
    the maximum (the workspace depends on the row blocks only up to a point)."""
    cap = bw.mbok_gemvt_scratch_bytes()
    assert cap == 512 * 1024
    worst = 0
    for G in range(1, 8193):
        for m in (1, 64, 65, 200, 320, 1000, 4096, 65536, 1 << 24):
            need = bw.mbok_gemvt_workspace_bytes(bw.mbok_desc_init(m, 128 * G, 1, bw.MBOK_F16))
            worst = max(worst, need)
    assert 0 < worst <= cap, worst


def test_ceilings_library_exports_its_header():
    """The measurement library (libmbok_ceilings.so) loads and exports every
    function include/mbok_ceilings.h declares; its argument checks run on
    the host."""
    from boolean_weight_amd import ceilings
    hdr = os.path.join(ROOT, "include", "mbok_ceilings.h")
    text = re.sub(r"/\*.*?\*/", "", open(hdr).read(), flags=re.S)
    fns = sorted(set(re.findall(r"\b(mbok_[a-z0-9_]+)\s*\(", text)))
    assert fns == ["mbok_ceiling_empty", "mbok_ceiling_marker", "mbok_ceiling_mfma",
                   "mbok_ceiling_read", "mbok_ceiling_spin"]
    lib = ceilings.load()
    out = subprocess.run(["nm", "-D", "--defined-only", lib._name],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (mbok_[a-z0-9_]+)\b", out))
    assert set(fns) <= exported
    assert lib.mbok_ceiling_empty(0, 64, None) == -1      # grid out of range
    assert lib.mbok_ceiling_empty(1, 100, None) == -1     # block not a multiple of 64
    assert lib.mbok_ceiling_read(None, 16, A16, 1, 64, None) == -1
    assert lib.mbok_ceiling_read(A16, 15, A16, 1, 64, None) == -1
    assert lib.mbok_ceiling_mfma(9, A16, 1, 1, 64, None) == -1
    assert lib.mbok_ceiling_spin(0, A16, None) == -1
    assert lib.mbok_ceiling_spin(100001, A16, None) == -1
    assert lib.mbok_ceiling_spin(10, None, None) == -1
