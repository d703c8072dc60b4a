"""The fp4 x fp8 matrix-core products for several tokens (mbok_gemm): two
tokens per instruction in the operand rows the one-token kernel leaves empty
(MBOK_SKINNY_VARIANT=f4, 2..4 tokens), and one product per group with 8
tokens in its rows (=f4g, 2..16 tokens).

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


# the two matrix-core few-token kernels: "f4" puts two tokens in the rows of
# the one-token products (2..4 tokens), "f4g" gives each product one group
# and 8 tokens (2..16 tokens)
VARIANTS = {"f4": [2, 3, 4], "f4g": [2, 3, 5, 8, 9, 16]}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bw.load_library()
    keys = ("MBOK_SKINNY_VARIANT", "MBOK_GEMV_VARIANT")
    old = {k: os.environ.get(k) for k in keys}
    os.environ.pop("MBOK_GEMV_VARIANT", None)
    yield
    for k, v in old.items():
        if v is None:
            os.environ.pop(k, None)
        else:
            os.environ[k] = v
    torch.cuda.synchronize()


def _set_variant(v):
    os.environ["MBOK_SKINNY_VARIANT"] = v


def _cases():
    return [(v, T) for v, ts in VARIANTS.items() for T in ts]


# (m, n): one row, ragged row blocks, 1..3 column slabs (at most 32 groups
# per slab for K >= 2, 48 for K = 1), and layers whose workgroups walk 3 and
# 5 tiles of 16 rows
SHAPES = [(1, 128), (65, 384), (300, 512), (130, 5120), (70, 11008), (9000, 256),
          (20000, 256)]


@pytest.mark.parametrize("m,n", SHAPES)
@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("variant,T", _cases())
def test_f4_tokens_exact(variant, T, K, m, n):
    _set_variant(variant)
    dt = "f16" if (m + n + K + T) % 2 else "f32"
    say(f"{variant} tokens exact T={T} K={K} m={m} n={n} {dt}")
    S = syn.random_signs(K, m, n, seed=T * 13 + K + m)
    A = syn.exact_alpha(K, m, n // 128, seed=T + 7 * K).astype(np_alpha(dt))
    X = syn.exact_activations(T, n, seed=T * 3 + K + n)
    d, packed = pack_on_gpu(S, A, dt)
    Y = gemm(d, packed, X, ldx=n + 24, ldy=m + 7)
    assert np.array_equal(Y, oracle.product(S, A, X))


@pytest.mark.parametrize("variant,T", [("f4", 4), ("f4g", 16)])
@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_f4_tokens_exact_4096(dt, variant, T):
    _set_variant(variant)
    K, m, n = 2, 4096, 4096
    say(f"{variant} tokens exact 4096x4096 T={T} {dt}")
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
@pytest.mark.parametrize("variant,T", [("f4", 2), ("f4", 4), ("f4g", 8), ("f4g", 16)])
def test_f4_tokens_exact_split_of_bf16(variant, T, binades):
    """As for one token: within 6 binades the fp8 parts hold every bf16 value
    and the sums are exact; over 12 binades the matrix cores drop bits far
    below a block's largest product."""
    _set_variant(variant)
    K, m, n = 1, 300, 1024
    say(f"{variant} tokens split T={T} binades={binades}")
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
@pytest.mark.parametrize("variant,T,tok", [("f4", 3, 1), ("f4g", 3, 1), ("f4g", 12, 10)])
def test_f4_tokens_nonfinite_is_per_token(bad, variant, T, tok):
    _set_variant(variant)
    K, m, n = 2, 200, 512
    say(f"{variant} tokens non-finite {bad} T={T}")
    S = syn.random_signs(K, m, n, seed=110)
    A = syn.exact_alpha(K, m, n // 128, seed=111).astype(np.float16)
    X = syn.exact_activations(T, n, seed=112)
    X[tok, 300] = bad
    d, packed = pack_on_gpu(S, A, "f16")
    Y = gemm(d, packed, X)
    assert np.all(np.isnan(Y[tok]))
    others = [t for t in range(T) if t != tok]
    assert np.array_equal(Y[others], oracle.product(S, A, X[others]))
    X[tok, 300] = 1.0
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
    _set_variant("f4")
    for T in (2, 3, 4):
        Y = gemm(d, packed, X[:T])
        for t in range(T):
            assert np.array_equal(Y[t], ys[t]), (T, t)


@pytest.mark.parametrize("cfg,li", [(2, 0), (3, 0)])
def test_f4g_tokens_do_not_depend_on_the_token_count(cfg, li):
    """Each token's row is computed from its own A rows only: for layers of
    at most 32 groups (one slab of 8 wavefronts with one or two octets) the
    first T rows of a 16-token call equal a T-token call bit for bit."""
    _set_variant("f4g")
    w = syn.WORKLOADS[cfg]
    name, m, n = w["linears"][li]
    say(f"f4g token count config {cfg} {name}")
    W = syn.weight(m, n, syn.weight_seed(cfg, li))
    X = syn.activations(16, n, syn.act_seed(cfg, li) + 1, "bf16")
    d, packed, signs, alpha = bw.quantize_and_pack(to_dev(W), w["K"], bw.MBOK_F16)
    del signs, alpha
    Y16 = gemm(d, packed, X)
    for T in (2, 5, 8, 9, 13):
        assert np.array_equal(gemm(d, packed, X[:T]), Y16[:T]), T


@pytest.mark.parametrize("variant", ["f4", "f4g"])
@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_f4_tokens_workloads_tolerance(cfg, variant):
    _set_variant(variant)
    w = syn.WORKLOADS[cfg]
    for li, (name, m, n) in enumerate(w["linears"]):
        if cfg == 4 and name in ("k_proj", "v_proj", "up_proj"):
            continue  # same shapes as q_proj / gate_proj
        T = (4 if cfg != 2 else 3) if variant == "f4" else (16 if cfg == 3 else 8)
        say(f"{variant} tokens config {cfg} {name} {m}x{n} T={T}")
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


@pytest.mark.parametrize("T,m,n,want", [(2, 512, 2048, "f4"), (4, 512, 2048, "blocks"),
                                         (4, 8192, 4096, "f4g"), (6, 8192, 4096, "f4g"),
                                         (7, 8192, 4096, "stream")])
def test_f4_tokens_default_dispatch_and_precise_path(T, m, n, want):
    """Without MBOK_SKINNY_VARIANT, mbok_gemm takes the two-token
    matrix-core kernel for 2 tokens, the one-product-per-group kernel for
    3..6 tokens on layers of at least 2^26 sign bits, and the bf16 +-1
    kernels otherwise (per-tile below 8192 rows, streaming from there);
    mbok_gemm_precise always keeps the bf16 +-1 kernels (their exact fp32
    scaling) for 2..16 tokens."""
    K = 2
    say(f"few-token dispatch T={T} m={m} n={n}")
    W = syn.weight(m, n, 120 + T)
    X = syn.activations(T, n, 121 + T, "bf16")
    d, packed, signs, alpha = bw.quantize_and_pack(to_dev(W), K, bw.MBOK_F16)
    del signs, alpha
    Xd = x_to_dev(X, "bf16").view(T, n)
    skinny = "stream" if (m >= 8192 and n // 128 <= 32) else "blocks"

    def run(fn, variant):
        if variant is None:
            os.environ.pop("MBOK_SKINNY_VARIANT", None)
        else:
            _set_variant(variant)
        Y = torch.empty((T, m), dtype=torch.float32, device=DEV)
        fn(d, packed, Xd, Y)
        return Y.cpu().numpy()

    default = run(bw.mbok_gemm, None)
    precise = run(bw.mbok_gemm_precise, None)
    forced = run(bw.mbok_gemm, want)
    assert np.array_equal(default, forced)
    assert np.array_equal(precise, run(bw.mbok_gemm, skinny))
    if want in ("f4", "f4g"):
        assert not np.array_equal(default, precise)  # two different kernels ran
