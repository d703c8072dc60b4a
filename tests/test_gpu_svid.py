"""GPU parity of the SVID scale variant: the successive decomposition
(mbok_svid_decompose), its packing (mbok_svid_pack) and product
(mbok_svid_gemv), through the C ABI, against the oracle.

Bars: signs identical and the rounded scale vectors bit-identical (the
device's float64 power iteration converges to the oracle's library SVD far
below the scale dtype's rounding); the product equal to the oracle's in the
exact regime (power-of-two scale vectors, integer activations) and within
|y - y_ref| <= 1e-3 * sum_j |W_hat[i, j]| |x_j| on Gaussian inputs, where the
product runs on the oracle's own decomposition.
"""
import numpy as np
import pytest
import torch

import boolean_weight_amd as bw
import mbok_synth as syn
import oracle
from gpu_util import DEV, alpha_enum, np_alpha, say, to_dev, x_to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-3
ITERS = 32


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bw.load_library()
    yield
    torch.cuda.synchronize()


def decompose_on_gpu(W: np.ndarray, K: int, dt: str, iters: int = ITERS):
    m, n = W.shape
    d = bw.mbok_desc_init(m, n, K, alpha_enum(dt))
    at = bw.alpha_torch_dtype(d.alpha_dtype)
    signs = torch.zeros((K, m, n), dtype=torch.int8, device=DEV)
    s_out = torch.zeros((K, m), dtype=at, device=DEV)
    s_in = torch.zeros((K, n), dtype=at, device=DEV)
    bw.mbok_svid_decompose(d, to_dev(W), signs, s_out, s_in, iters)
    return d, signs, s_out, s_in


def assert_bits_equal(a: np.ndarray, b: np.ndarray, what):
    view = np.uint16 if a.dtype == np.float16 else np.uint32
    bad = np.argwhere(a.view(view) != b.view(view))
    assert bad.size == 0, (what, bad[:5], a[tuple(bad[0])], b[tuple(bad[0])])


@pytest.mark.parametrize("K", [1, 2, 3])
@pytest.mark.parametrize("dt", ["f16", "f32"])
@pytest.mark.parametrize("m,n", [(64, 256), (130, 384), (512, 2048)])
def test_svid_decompose_matches_oracle(m, n, K, dt):
    say(f"svid decompose m={m} n={n} K={K} {dt}")
    W = syn.weight(m, n, seed=900 + m + K)
    W[3, :7] = 0.0
    W[4, 5:9] = -0.0
    d, signs, s_out, s_in = decompose_on_gpu(W, K, dt)
    S, SO, SI, _ = oracle.svid_decompose(W, K, alpha_dtype=dt)
    assert np.array_equal(signs.cpu().numpy(), S)
    assert_bits_equal(s_out.cpu().numpy(), SO, "s_out")
    assert_bits_equal(s_in.cpu().numpy(), SI, "s_in")


def test_svid_exact_rank1_recovered():
    """S (.) (a b^T) with equal-norm fp16 vectors (a zero row and column
    included) comes back exactly."""
    say("svid exact rank-1")
    rng = np.random.default_rng(971)
    n = 256
    a = (rng.integers(16, 64, size=n) / 256.0).astype(np.float16)
    a[5] = 0.0
    b = a[rng.permutation(n)]
    S = rng.choice(np.array([-1, 1], dtype=np.int8), size=(n, n))
    W = (S.astype(np.float64) * (a.astype(np.float64)[:, None] * b.astype(np.float64)[None, :]))
    W = W.astype(np.float32)
    d, signs, s_out, s_in = decompose_on_gpu(W, 1, "f16")
    Sr, SO, SI, R = oracle.svid_decompose(W, 1, alpha_dtype="f16")
    assert np.array_equal(s_out.cpu().numpy()[0], a) and np.array_equal(s_in.cpu().numpy()[0], b)
    assert np.array_equal(signs.cpu().numpy(), Sr)


@pytest.mark.parametrize("cfg,K", [(2, 2), (3, 3)])
def test_svid_decompose_workload(cfg, K):
    """The first linear of workloads 2 and 3 at full size."""
    name, m, n = syn.WORKLOADS[cfg]["linears"][0]
    say(f"svid decompose config {cfg} {name} {m}x{n} K={K}")
    W = syn.weight(m, n, syn.weight_seed(cfg, 0))
    d, signs, s_out, s_in = decompose_on_gpu(W, K, "f16")
    S, SO, SI, _ = oracle.svid_decompose(W, K, alpha_dtype="f16")
    assert np.array_equal(signs.cpu().numpy(), S)
    assert_bits_equal(s_out.cpu().numpy(), SO, "s_out")
    assert_bits_equal(s_in.cpu().numpy(), SI, "s_in")


def gemv_svid(d, packed, s_in_np: np.ndarray, x: np.ndarray, xdt: str, dt: str) -> np.ndarray:
    y = torch.full((d.m,), -1.0, dtype=torch.float32, device=DEV)
    bw.mbok_svid_gemv(d, packed, to_dev(s_in_np.astype(np_alpha(dt))), x_to_dev(x, xdt), y)
    return y.cpu().numpy().astype(np.float64)


def pack_svid(S, SO, dt):
    K, m, n = S.shape
    d = bw.mbok_desc_init(m, n, K, alpha_enum(dt))
    packed = torch.empty(bw.mbok_packed_bytes(d), dtype=torch.uint8, device=DEV)
    bw.mbok_svid_pack(d, to_dev(S), to_dev(SO.astype(np_alpha(dt))), packed)
    return d, packed


# the product on the fp4 x fp8 decode kernel (default) and in the bf16 +-1
# few-token kernel (MBOK_SVID_VARIANT=skinny)
SVID_VARIANTS = ["f4", "skinny"]


@pytest.fixture(params=SVID_VARIANTS)
def svid_variant(request, monkeypatch):
    if request.param == "skinny":
        monkeypatch.setenv("MBOK_SVID_VARIANT", "skinny")
    else:
        monkeypatch.delenv("MBOK_SVID_VARIANT", raising=False)
    return request.param


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("m,n", [(1, 128), (64, 128), (130, 640), (4096, 4096), (70, 13824),
                                 (20000, 256)])
def test_svid_gemv_exact_regime(m, n, K, svid_variant):
    for dt, xdt in (("f16", "bf16"), ("f32", "f32")):
        say(f"svid gemv exact m={m} n={n} K={K} {dt}/{xdt} {svid_variant}")
        rng = np.random.default_rng(m + n + K)
        S = syn.random_signs(K, m, n, seed=m * 3 + n + K)
        SO = np.ldexp(1.0, -rng.integers(2, 5, size=(K, m))).astype(np_alpha(dt))
        SI = np.ldexp(1.0, -rng.integers(2, 5, size=(K, n))).astype(np_alpha(dt))
        x = syn.exact_activations(1, n, seed=n + 5)[0]
        d, packed = pack_svid(S, SO, dt)
        y = gemv_svid(d, packed, SI, x, xdt, dt)
        want = oracle.svid_product(S, SO, SI, x)
        assert np.array_equal(y, want), np.max(np.abs(y - want))


def test_svid_pack_layout():
    """The packed buffer equals the oracle's packer with s_out in every group."""
    say("svid pack layout")
    K, m, n = 3, 70, 384
    S = syn.random_signs(K, m, n, seed=31)
    SO = np.random.default_rng(32).random((K, m)).astype(np.float16)
    d, packed = pack_svid(S, SO, "f16")
    A = np.repeat(SO[:, :, None], n // 128, axis=2)
    assert np.array_equal(packed.cpu().numpy(), oracle.pack(S, A, "f16"))


@pytest.mark.parametrize("cfg", [1, 2, 3])
def test_svid_gemv_workload_tolerance(cfg, svid_variant):
    """Gaussian weights decomposed by the oracle, packed and multiplied on the
    device, against the oracle's product (sampled rows)."""
    w = syn.WORKLOADS[cfg]
    name, m, n = w["linears"][0]
    dt, xdt, K = w["alpha_dtype"], w["x_dtype"], w["K"]
    say(f"svid gemv config {cfg} {name} {m}x{n} K={K} {svid_variant}")
    W = syn.weight(m, n, syn.weight_seed(cfg, 0))
    S, SO, SI, _ = oracle.svid_decompose(W, K, alpha_dtype=dt)
    x = syn.activations(1, n, syn.act_seed(cfg, 0), xdt)[0]
    d, packed = pack_svid(S, SO, dt)
    y = gemv_svid(d, packed, SI, x, xdt, dt)
    rows = np.array(sorted({0, m - 1, *np.random.default_rng(cfg).choice(m, 128).tolist()}))
    want = oracle.svid_product(S[:, rows], SO[:, rows], SI, x)
    E = oracle.svid_bound(S[:, rows], SO[:, rows], SI, x)
    ratio = oracle.max_error_ratio(y[rows], want, E)
    assert ratio <= TOL, ratio
    # close to float64 as well: both forms keep 16 significant bits of each
    # s_in^k x_j (bf16 hi/lo parts; four fp8 parts of one word scale)
    assert ratio <= 1e-2 * TOL, ratio
