"""The hot-path entry points under HIP graph capture.

A serving loop records the products into a HIP graph once and replays it.
Each case here computes the product eagerly, checks it against the oracle
(exact regime: integer activations, power-of-two scales), captures the same
call into a graph, and replays the graph several times with eager library
work and synchronizations between the replays.  Every replay must write the
eager result again, bit for bit (the output is cleared before each replay, so
a replay that writes nothing fails).  The library records no memset, no
allocation and no synchronization, so a captured call is just its kernels.
"""
import numpy as np
import pytest
import torch

import boolean_weight_amd as bw
import mbok_synth as syn
import oracle
from gpu_util import DEV, pack_on_gpu, say, to_dev, x_to_dev

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bw.load_library()
    yield
    torch.cuda.synchronize()


def capture(fn):
    """Warm fn up on a side stream, then record it into a graph."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def check_replays(g, out: torch.Tensor, expect: np.ndarray, other):
    """Replay g REPLAYS times; `other` is eager library work run in between."""
    for r in range(REPLAYS):
        out.fill_(-31.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = out.cpu().numpy()
        assert np.array_equal(got, expect), f"replay {r} differs from the eager result"
        other()
        torch.cuda.synchronize()


def exact_layer(K, m, n, seed):
    S = syn.random_signs(K, m, n, seed=seed)
    A = syn.exact_alpha(K, m, n // 128, seed=seed + 1).astype(np.float16)
    return S, A


def test_graph_gemv():
    K, m, n = 3, 1000, 1024
    say(f"graph gemv m={m} n={n} K={K}")
    S, A = exact_layer(K, m, n, 301)
    d, packed = pack_on_gpu(S, A, "f16")
    x = syn.exact_activations(1, n, seed=303)
    xt = x_to_dev(x.reshape(-1), "bf16")
    y = torch.empty(m, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(1, bw.mbok_gemv_workspace_bytes(d)), dtype=torch.uint8, device=DEV)
    bw.mbok_gemv(d, packed, xt, y, workspace=ws)
    eager = y.cpu().numpy()
    assert np.array_equal(eager.astype(np.float64), oracle.product(S, A, x)[0])
    g = capture(lambda: bw.mbok_gemv(d, packed, xt, y, workspace=ws))
    # in between: the same layer on other activations into another buffer
    x2 = x_to_dev(syn.exact_activations(1, n, seed=304).reshape(-1), "bf16")
    y2 = torch.empty_like(y)
    check_replays(g, y, eager, lambda: bw.mbok_gemv(d, packed, x2, y2, workspace=ws))


@pytest.mark.parametrize("T,variant", [(2, None), (4, "f4g"), (5, None), (300, None)])
def test_graph_gemm(T, variant, monkeypatch):
    """T = 2 runs the two-token matrix-core kernel, T = 4 with
    MBOK_SKINNY_VARIANT=f4g the one-product-per-group kernel, T = 5 the bf16
    +-1 few-token kernel, T = 300 the prefill kernel."""
    if variant:
        monkeypatch.setenv("MBOK_SKINNY_VARIANT", variant)
    K, m, n = 3, 513, 640
    say(f"graph gemm T={T} {variant} m={m} n={n} K={K}")
    S, A = exact_layer(K, m, n, 311 + T)
    d, packed = pack_on_gpu(S, A, "f16")
    X = syn.exact_activations(T, n, seed=313 + T)
    Xt = x_to_dev(X, "bf16").view(T, n)
    Y = torch.empty((T, m), dtype=torch.float32, device=DEV)
    bw.mbok_gemm(d, packed, Xt, Y)
    eager = Y.cpu().numpy()
    assert np.array_equal(eager.astype(np.float64), oracle.product(S, A, X))
    g = capture(lambda: bw.mbok_gemm(d, packed, Xt, Y))
    X2 = x_to_dev(syn.exact_activations(T, n, seed=317 + T), "bf16").view(T, n)
    Y2 = torch.empty_like(Y)
    check_replays(g, Y, eager, lambda: bw.mbok_gemm(d, packed, X2, Y2))


def test_graph_gemvt():
    """The transposed product with its workspace (slices, then the reduce kernel)."""
    K, m, n = 2, 768, 1024
    say(f"graph gemvt m={m} n={n} K={K}")
    S, A = exact_layer(K, m, n, 321)
    d, packed = pack_on_gpu(S, A, "f16")
    gv = syn.exact_activations(1, m, seed=323).reshape(-1)
    gt = x_to_dev(gv, "bf16")
    dx = torch.empty(n, dtype=torch.float32, device=DEV)
    ws = torch.empty(max(1, bw.mbok_gemvt_workspace_bytes(d)), dtype=torch.uint8, device=DEV)
    bw.mbok_gemvt(d, packed, gt, dx, workspace=ws)
    eager = dx.cpu().numpy()
    assert np.array_equal(eager.astype(np.float64), oracle.product_transposed(S, A, gv))
    g = capture(lambda: bw.mbok_gemvt(d, packed, gt, dx, workspace=ws))
    g2 = x_to_dev(syn.exact_activations(1, m, seed=324).reshape(-1), "bf16")
    dx2 = torch.empty_like(dx)
    check_replays(g, dx, eager, lambda: bw.mbok_gemvt(d, packed, g2, dx2, workspace=ws))


def test_graph_svid_gemv():
    K, m, n = 2, 512, 512
    say(f"graph svid gemv m={m} n={n} K={K}")
    S = syn.random_signs(K, m, n, seed=331)
    rng = np.random.default_rng(332)
    SO = (2.0 ** -rng.integers(3, 7, size=(K, m))).astype(np.float16)
    SI = (2.0 ** -rng.integers(3, 7, size=(K, n))).astype(np.float16)
    d = bw.mbok_desc_init(m, n, K, bw.MBOK_F16)
    packed = torch.empty(bw.mbok_packed_bytes(d), dtype=torch.uint8, device=DEV)
    bw.mbok_svid_pack(d, to_dev(S), to_dev(SO), packed)
    s_in = to_dev(SI)
    x = syn.exact_activations(1, n, seed=333).reshape(-1)
    xt = x_to_dev(x, "bf16")
    y = torch.empty(m, dtype=torch.float32, device=DEV)
    bw.mbok_svid_gemv(d, packed, s_in, xt, y)
    eager = y.cpu().numpy()
    assert np.array_equal(eager.astype(np.float64), oracle.svid_product(S, SO, SI, x))
    g = capture(lambda: bw.mbok_svid_gemv(d, packed, s_in, xt, y))
    x2 = x_to_dev(syn.exact_activations(1, n, seed=334).reshape(-1), "bf16")
    y2 = torch.empty_like(y)
    check_replays(g, y, eager, lambda: bw.mbok_svid_gemv(d, packed, s_in, x2, y2))
