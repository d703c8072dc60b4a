"""GPU parity of the transposed decode product dx = W_hat^T g (mbok_gemvt)
against the oracle's product_transposed, through the C ABI.

Bars (as for the forward product): in the exact regime (integer g in [-8, 8],
scales 2^-e, e in 4..8, so every partial sum is a multiple of 2^-8 far below
2^24 of them) equal values; on the workloads' Gaussian inputs
|dx - dx_ref| <= 1e-3 * sum_i |W_hat[i, j]| |g_i| for every column.  Both
with the sliced workspace path and without a workspace.  Full-size layers are
checked on sampled column groups, which the oracle quantizes on their own
(groups are independent).
"""
import numpy as np
import pytest
import torch

import boolean_weight_amd as bw
import mbok_synth as syn
import oracle
from gpu_util import DEV, alpha_enum, np_alpha, pack_on_gpu, say, to_dev, x_to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bw.load_library()
    yield
    torch.cuda.synchronize()


def gemvt(d, packed, g: np.ndarray, g_dtype: str, workspace=True, guard: int = 0) -> np.ndarray:
    gt = x_to_dev(g.reshape(-1), g_dtype)
    canary = -12345.5
    buf = torch.full((d.n + 2 * guard,), canary, dtype=torch.float32, device=DEV)
    dx = buf[guard:guard + d.n]
    bw.mbok_gemvt(d, packed, gt, dx, workspace=workspace)
    out = buf.cpu().numpy()
    if guard:
        assert np.all(out[:guard] == canary) and np.all(out[guard + d.n:] == canary)
    return out[guard:guard + d.n].astype(np.float64)


EXACT_SHAPES = [(1, 128), (63, 256), (64, 128), (65, 384), (130, 1024), (256, 4096),
                (200, 5120), (70, 13824), (4096, 256)]


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("m,n", EXACT_SHAPES)
@pytest.mark.parametrize("ws", [True, None])
def test_gemvt_exact_regime(m, n, K, ws):
    for dt, gdt in (("f16", "bf16"), ("f32", "f32")):
        say(f"gemvt exact m={m} n={n} K={K} {dt}/{gdt} workspace={ws}")
        S = syn.random_signs(K, m, n, seed=m * 5 + n + K)
        A = syn.exact_alpha(K, m, n // 128, seed=m + 3 * K).astype(np_alpha(dt))
        g = syn.exact_activations(1, m, seed=m + K + 7)[0]
        d, packed = pack_on_gpu(S, A, dt)
        dx = gemvt(d, packed, g, gdt, workspace=ws, guard=9)
        want = oracle.product_transposed(S, A, g)
        assert np.array_equal(dx, want), np.max(np.abs(dx - want))


def test_gemvt_one_hot_rows():
    """A one-hot g returns a row of W_hat exactly."""
    say("gemvt one-hot rows")
    K, m, n = 3, 130, 384
    S = syn.random_signs(K, m, n, seed=15)
    A = syn.exact_alpha(K, m, 3, seed=16).astype(np.float16)
    d, packed = pack_on_gpu(S, A, "f16")
    What = oracle.dequantize(S, A)
    for i in (0, 1, 63, 64, 65, 127, 129):
        g = np.zeros(m, dtype=np.float32)
        g[i] = 1.0
        assert np.array_equal(gemvt(d, packed, g, "f32"), What[i]), i


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_gemvt_workloads_tolerance(cfg):
    """Full pipeline on the device (quantize, pack, transposed product) at
    the workload shapes; the oracle quantizes sampled column groups."""
    w = syn.WORKLOADS[cfg]
    dt, gdt = w["alpha_dtype"], w["x_dtype"]
    for li, (name, m, n) in enumerate(w["linears"]):
        say(f"gemvt config {cfg} {name} {m}x{n} K={w['K']}")
        W = syn.weight(m, n, syn.weight_seed(cfg, li))
        g = syn.activations(1, m, syn.act_seed(cfg, li) + 500, gdt)[0]
        d, packed, signs, alpha = bw.quantize_and_pack(to_dev(W), w["K"], alpha_enum(dt))
        del signs, alpha
        dx = gemvt(d, packed, g, gdt, guard=3)
        G = n // 128
        groups = sorted({0, G - 1, int(np.random.default_rng(li).integers(0, G))})
        for gi in groups:
            cols = slice(128 * gi, 128 * gi + 128)
            S, A, _ = oracle.residual_binarize(W[:, cols], w["K"], alpha_dtype=dt)
            want = oracle.product_transposed(S, A, g)
            E = oracle.bound_transposed(S, A, g)
            ratio = oracle.max_error_ratio(dx[cols], want, E)
            assert ratio <= TOL, (name, gi, ratio)
        assert np.array_equal(dx, gemvt(d, packed, g, gdt))  # deterministic
        assert np.allclose(gemvt(d, packed, g, gdt, workspace=None), dx, rtol=0, atol=1e-5 *
                           np.max(np.abs(dx)))
        del packed
        torch.cuda.empty_cache()


def test_gemvt_workspace_sizes_and_garbage():
    """The workspace serves any shape whatever it holds beforehand."""
    say("gemvt workspace garbage")
    shapes = [(4096, 4096, 2), (300, 11008, 3), (11008, 4096, 3), (64, 13824, 1), (1, 128, 1)]
    need = max(bw.mbok_gemvt_workspace_bytes(bw.mbok_desc_init(m, n, K, bw.MBOK_F16))
               for m, n, K in shapes)
    ws = torch.full((need // 4 + 64,), float("nan"), dtype=torch.float32, device=DEV)
    for m, n, K in shapes:
        S = syn.random_signs(K, m, n, seed=m + n)
        A = syn.exact_alpha(K, m, n // 128, seed=K).astype(np.float16)
        g = syn.exact_activations(1, m, seed=3)[0]
        d, packed = pack_on_gpu(S, A, "f16")
        dx = gemvt(d, packed, g, "bf16", workspace=ws)
        assert np.array_equal(dx, oracle.product_transposed(S, A, g)), (m, n, K)
