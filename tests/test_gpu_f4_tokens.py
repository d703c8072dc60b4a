"""The fp4 x fp8 matrix-core product for 2..4 tokens (mbok_gemm, T = 2 by
default, T = 2..4 with MBOK_SKINNY_VARIANT=f4):
two tokens per matrix-core instruction in the operand rows the one-token
kernel leaves empty.

Bars: exact regime (integer X in [-8, 8], scales 2^-e) equal values for every
shape, kernel count, scale type and leading dimension; bf16 activations
spread over up to 6 binades inside each 32-column block with K = 1 also
exact, over 12 binades within 1e-4 of the bound; a layer of at most 32
groups gives, token by token, the one-token kernel's bits (the same
arithmetic in the same order); Gaussian workloads within
1e-3 * sum |W_hat| |x|; a non-finite activation makes its own token's row
NaN and leaves the other tokens exact.
"""
import os

import numpy as np
import pytest
import torch

import boolean_weight_amd as bw
import mbok_synth as syn
import oracle
from gpu_util import DEV, gemm, gemv, np_alpha, pack_on_gpu, say, to_dev, x_to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bw.load_library()
    keys = ("MBOK_SKINNY_VARIANT", "MBOK_GEMV_VARIANT")
    old = {k: os.environ.get(k) for k in keys}
    os.environ["MBOK_SKINNY_VARIANT"] = "f4"
    os.environ.pop("MBOK_GEMV_VARIANT", None)
    yield
    for k, v in old.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v
    torch.cuda.synchronize()


# (m, n): one row, ragged row blocks, 1..3 column slabs (at most 32 groups
# per slab for K >= 2, 48 for K = 1), and layers whose workgroups walk 3 and
# 5 tiles of 16 rows
SHAPES = [(1, 128), (65, 384), (300, 512), (130, 5120), (70, 11008), (9000, 256),
          (20000, 256)]


@pytest.mark.parametrize("m,n", SHAPES)
@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("T", [2, 3, 4])
def test_f4_tokens_exact(T, K, m, n):
    dt = "f16" if (m + n + K + T) % 2 else "f32"
    say(f"f4 tokens exact T={T} K={K} m={m} n={n} {dt}")
    S = syn.random_signs(K, m, n, seed=T * 13 + K + m)
    A = syn.exact_alpha(K, m, n // 128, seed=T + 7 * K).astype(np_alpha(dt))
    X = syn.exact_activations(T, n, seed=T * 3 + K + n)
    d, packed = pack_on_gpu(S, A, dt)
    Y = gemm(d, packed, X, ldx=n + 24, ldy=m + 7)
    assert np.array_equal(Y, oracle.product(S, A, X))


@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_f4_tokens_exact_4096(dt):
    K, m, n, T = 2, 4096, 4096, 4
    say(f"f4 tokens exact 4096x4096 {dt}")
    S = syn.random_signs(K, m, n, seed=90)
    A = syn.exact_alpha(K, m, n // 128, seed=91).astype(np_alpha(dt))
    X = syn.exact_activations(T, n, seed=92)
    d, packed = pack_on_gpu(S, A, dt)
    assert np.array_equal(gemm(d, packed, X), oracle.product(S, A, X))


def _spread_x(T, n, seed, binades):
    rng = np.random.default_rng(seed)
    mant = rng.integers(128, 256, size=(T, n))
    e = rng.integers(-binades, 1, size=(T, n))
    x = np.ldexp(mant.astype(np.float64) / 128.0, e) * rng.choice([-1.0, 1.0], size=(T, n))
    return x.astype(np.float32)


@pytest.mark.parametrize("binades", [0, 6, 12])
@pytest.mark.parametrize("T", [2, 4])
def test_f4_tokens_exact_split_of_bf16(T, binades):
    """As for one token: within 6 binades the fp8 parts hold every bf16 value
    and the sums are exact; over 12 binades the matrix cores drop bits far
    below a block's largest product."""
    K, m, n = 1, 300, 1024
    say(f"f4 tokens split T={T} binades={binades}")
    S = syn.random_signs(K, m, n, seed=100 + binades)
    A = syn.exact_alpha(K, m, n // 128, seed=101).astype(np.float16)
    X = _spread_x(T, n, 102 + binades, binades)
    d, packed = pack_on_gpu(S, A, "f16")
    Y = gemm(d, packed, X)
    want = oracle.product(S, A, X)
    if binades <= 6:
        assert np.array_equal(Y, want)
    else:
        ratio = oracle.max_error_ratio(Y, want, oracle.bound(S, A, X))
        say(f"  err/bound {ratio:.3e}")
        assert ratio <= 0.1 * TOL, ratio


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_f4_tokens_nonfinite_is_per_token(bad):
    K, m, n, T = 2, 200, 512, 3
    say(f"f4 tokens non-finite {bad}")
    S = syn.random_signs(K, m, n, seed=110)
    A = syn.exact_alpha(K, m, n // 128, seed=111).astype(np.float16)
    X = syn.exact_activations(T, n, seed=112)
    X[1, 300] = bad
    d, packed = pack_on_gpu(S, A, "f16")
    Y = gemm(d, packed, X)
    assert np.all(np.isnan(Y[1]))
    want = oracle.product(S, A, X[[0, 2]])
    assert np.array_equal(Y[[0, 2]], want)
    X[1, 300] = 1.0
    assert np.array_equal(gemm(d, packed, X), oracle.product(S, A, X))


@pytest.mark.parametrize("cfg,li", [(2, 0), (3, 0)])
def test_f4_tokens_equal_the_decode_per_token(cfg, li):
    """Layers of at most 32 groups run one column slab with the same
    wavefronts in both kernels, so each token's row is bit for bit the
    one-token kernel's y on that token (Gaussian data)."""
    w = syn.WORKLOADS[cfg]
    name, m, n = w["linears"][li]
    say(f"f4 tokens vs decode config {cfg} {name}")
    W = syn.weight(m, n, syn.weight_seed(cfg, li))
    X = syn.activations(4, n, syn.act_seed(cfg, li), "bf16")
    d, packed, signs, alpha = bw.quantize_and_pack(to_dev(W), w["K"], bw.MBOK_F16)
    del signs, alpha
    old = os.environ.get("MBOK_GEMV_VARIANT")
    os.environ["MBOK_GEMV_VARIANT"] = "f4"
    try:
        ys = [gemv(d, packed, X[t], "bf16") for t in range(4)]
    finally:
        if old is None:
            os.environ.pop("MBOK_GEMV_VARIANT", None)
        else:
            os.environ["MBOK_GEMV_VARIANT"] = old
    for T in (2, 3, 4):
        Y = gemm(d, packed, X[:T])
        for t in range(T):
            assert np.array_equal(Y[t], ys[t]), (T, t)


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_f4_tokens_workloads_tolerance(cfg):
    w = syn.WORKLOADS[cfg]
    for li, (name, m, n) in enumerate(w["linears"]):
        if cfg == 4 and name in ("k_proj", "v_proj", "up_proj"):
            continue  # same shapes as q_proj / gate_proj
        T = 4 if cfg != 2 else 3
        say(f"f4 tokens config {cfg} {name} {m}x{n} T={T}")
        W = syn.weight(m, n, syn.weight_seed(cfg, li))
        X = syn.activations(T, n, syn.act_seed(cfg, li), "bf16")
        d, packed, signs, alpha = bw.quantize_and_pack(to_dev(W), w["K"], bw.MBOK_F16)
        del signs, alpha
        Y = gemm(d, packed, X, ldy=m + 5)
        rng = np.random.default_rng(li + 10 * cfg)
        rows = np.unique(np.r_[rng.choice(m, 192, replace=False), np.arange(m - 48, m)])
        S, A, _ = oracle.residual_binarize(W[rows], w["K"], alpha_dtype="f16")
        ratio = oracle.max_error_ratio(Y[:, rows], oracle.product(S, A, X),
                                       oracle.bound(S, A, X))
        say(f"  err/bound {ratio:.3e}")
        assert ratio <= TOL, (name, ratio)
        assert np.array_equal(Y, gemm(d, packed, X, ldy=m + 5))  # deterministic
        del packed
        torch.cuda.empty_cache()


def test_f4_tokens_default_dispatch_and_precise_path():
    """Without MBOK_SKINNY_VARIANT, mbok_gemm takes the matrix-core kernel for
    2 tokens (same bits as with =f4); mbok_gemm_precise keeps the
    bf16 +-1 few-token kernel there (its exact fp32 scaling): for 512 rows
    that is the per-tile form, =blocks."""
    K, m, n, T = 3, 512, 2048, 2
    say("f4 tokens dispatch")
    W = syn.weight(m, n, 120)
    X = syn.activations(T, n, 121, "bf16")
    d, packed, signs, alpha = bw.quantize_and_pack(to_dev(W), K, bw.MBOK_F16)
    del signs, alpha
    Xd = x_to_dev(X, "bf16").view(T, n)

    def run(fn):
        Y = torch.empty((T, m), dtype=torch.float32, device=DEV)
        fn(d, packed, Xd, Y)
        return Y.cpu().numpy()

    f4 = run(bw.mbok_gemm)
    os.environ.pop("MBOK_SKINNY_VARIANT", None)
    try:
        default = run(bw.mbok_gemm)
        precise = run(bw.mbok_gemm_precise)
        os.environ["MBOK_SKINNY_VARIANT"] = "blocks"
        blocks = run(bw.mbok_gemm)
    finally:
        os.environ["MBOK_SKINNY_VARIANT"] = "f4"
    assert np.array_equal(default, f4)
    assert np.array_equal(precise, blocks)
    assert not np.array_equal(f4, blocks)  # two different kernels ran
