"""The fp4 x fp8 matrix-core decode kernel (MBOK_GEMV_VARIANT=f4) beyond the
shared variant tests: activations split into exact high and low fp8 parts
per 32-column block, wide scale spreads, non-finite activations, and the
workload shapes in tolerance mode.

Bars: exact regime (integer x in [-8, 8], scales 2^-e) equal values; bf16
activations spread over up to 13 binades inside each 32-column block, with
power-of-two scales and K = 1, are also exact (the two fp8 parts hold every
such bf16 value and the products are small integers times powers of two);
Gaussian workloads within 1e-3 * sum |W_hat| |x|.
"""
import os

import numpy as np
import pytest
import torch

import boolean_weight_amd as bw
import mbok_synth as syn
import oracle
from gpu_util import DEV, gemv, pack_on_gpu, say, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bw.load_library()
    old = os.environ.get("MBOK_GEMV_VARIANT")
    os.environ["MBOK_GEMV_VARIANT"] = "f4"
    yield
    if old is None:
        os.environ.pop("MBOK_GEMV_VARIANT", None)
    else:
        os.environ["MBOK_GEMV_VARIANT"] = old
    torch.cuda.synchronize()


def _spread_x(n, seed, binades):
    """bf16 values +-m * 2^e with an 8-bit significand m and e spread over
    `binades` binades (so within any block all values lie within that many
    binades of each other)."""
    rng = np.random.default_rng(seed)
    mant = rng.integers(128, 256, size=n)           # 8 significant bits
    e = rng.integers(-binades, 1, size=n)
    x = np.ldexp(mant.astype(np.float64) / 128.0, e) * rng.choice([-1.0, 1.0], size=n)
    return x.astype(np.float32)                       # exact in bf16


@pytest.mark.parametrize("m,n", [(64, 128), (300, 512), (4096, 4096), (130, 5120)])
@pytest.mark.parametrize("binades", [0, 6, 12])
def test_f4_exact_split_of_bf16(m, n, binades):
    """K = 1, scales 2^-e: y is a sum of +-x_j * 2^-e.  Within 6 binades the
    two fp8 parts hold every x exactly, the matrix cores add the products
    exactly and every fp32 partial sum stays on a grid of 2^-(7 + 6 + 8)
    below 2^24 of it: equal values.  Over 12 binades the matrix cores drop
    bits far below a block's largest product (about 1e-5 of the bound here),
    so that case is held to the tolerance with a 10x margin."""
    say(f"f4 split m={m} n={n} binades={binades}")
    K = 1
    S = syn.random_signs(K, m, n, seed=m + n + binades)
    A = syn.exact_alpha(K, m, n // 128, seed=m + binades).astype(np.float16)
    x = _spread_x(n, 7 + binades, binades)
    d, packed = pack_on_gpu(S, A, "f16")
    y = gemv(d, packed, x, "bf16", guard=5)
    want = oracle.product(S, A, x)
    if binades <= 6:
        assert np.array_equal(y, want), np.max(np.abs(y - want))
    else:
        ratio = oracle.max_error_ratio(y, want, oracle.bound(S, A, x))
        say(f"  err/bound {ratio:.3e}")
        assert ratio <= 0.1 * TOL, ratio


@pytest.mark.parametrize("K", [2, 3, 4])
def test_f4_scales_spread_wide(K):
    """Power-of-two scales 2^-e with e over 20 binades and integer x: exact
    (each group's product is an integer times its scale; the fp32 sums of
    at most 4 K terms per group stay exact on the 2^-28 grid below 2^24 of
    it for these sizes)."""
    m, n = 260, 1024
    say(f"f4 wide scales K={K}")
    rng = np.random.default_rng(40 + K)
    S = syn.random_signs(K, m, n, seed=41 + K)
    A = np.ldexp(1.0, -rng.integers(1, 21, size=(K, m, n // 128))).astype(np.float32)
    x = syn.exact_activations(1, n, seed=42 + K)[0]
    d, packed = pack_on_gpu(S, A, "f32")
    y = gemv(d, packed, x, "bf16")
    want = oracle.product(S, A, x)
    E = oracle.bound(S, A, x)
    assert oracle.max_error_ratio(y, want, E) <= 1e-6


@pytest.mark.parametrize("bad", [np.nan, np.inf, -np.inf])
def test_f4_nonfinite_activation_gives_nan(bad):
    say(f"f4 non-finite {bad}")
    K, m, n = 2, 200, 512
    S = syn.random_signs(K, m, n, seed=5)
    A = syn.exact_alpha(K, m, n // 128, seed=6).astype(np.float16)
    x = syn.exact_activations(1, n, seed=7)[0]
    x[300] = bad
    d, packed = pack_on_gpu(S, A, "f16")
    y = gemv(d, packed, x, "bf16")
    assert np.all(np.isnan(y))
    # the next call on finite input is clean again
    x[300] = 1.0
    y = gemv(d, packed, x, "bf16")
    assert np.array_equal(y, oracle.product(S, A, x))


@pytest.mark.parametrize("cfg", [2, 3, 4])
def test_f4_workloads_tolerance(cfg):
    w = syn.WORKLOADS[cfg]
    dt, xdt = w["alpha_dtype"], w["x_dtype"]
    for li, (name, m, n) in enumerate(w["linears"]):
        if cfg == 4 and name in ("k_proj", "v_proj", "up_proj"):
            continue  # same shapes as q_proj / gate_proj
        say(f"f4 config {cfg} {name} {m}x{n}")
        W = syn.weight(m, n, syn.weight_seed(cfg, li))
        x = syn.activations(1, n, syn.act_seed(cfg, li), xdt)[0]
        d, packed, signs, alpha = bw.quantize_and_pack(to_dev(W), w["K"], bw.MBOK_F16)
        del signs, alpha
        y = gemv(d, packed, x, xdt, guard=3)
        rng = np.random.default_rng(li)
        rows = np.unique(np.r_[rng.choice(m, 256, replace=False), np.arange(m - 64, m)])
        S, A, _ = oracle.residual_binarize(W[rows], w["K"], alpha_dtype=dt)
        ratio = oracle.max_error_ratio(y[rows], oracle.product(S, A, x), oracle.bound(S, A, x))
        say(f"  err/bound {ratio:.3e}")
        assert ratio <= TOL, (name, ratio)
        assert np.array_equal(y, gemv(d, packed, x, xdt))  # deterministic
        del packed
        torch.cuda.empty_cache()
