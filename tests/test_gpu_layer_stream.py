"""The LLaMA-13B-shaped decoder layer exactly as it is measured per token:
four launches (q|k|v fused 15360 x 5120, o 5120 x 5120, gate|up fused
27648 x 5120, down 5120 x 13824; K = 3), each on its own seeded weight.

  * tolerance: quantized and packed on the device, the four products
    captured in one HIP graph and replayed; every replay is checked against
    the eager result bit for bit, and sampled rows of every launch (plus the
    whole last row block) against the oracle, which quantizes those rows
    itself;
  * exact regime at the two fused shapes (random signs, power-of-two scales,
    integer activations): every 7th row and the last row block equal the
    oracle's values.  At 27648 rows the decode kernel walks 6 or 7 tiles per
    workgroup.
"""
import numpy as np
import pytest
import torch

import boolean_weight_amd as bw
import mbok_synth as syn
import oracle
from gpu_util import DEV, gemv, pack_on_gpu, say, to_dev, x_to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-3
REPLAYS = 3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bw.load_library()
    yield
    torch.cuda.synchronize()


def _rows(m: int, count: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    r = set(rng.choice(m, size=count, replace=False).tolist())
    r |= set(range(m - 64, m)) | {0, 63, 64}
    return np.array(sorted(r))


def test_layer_stream_graph_tolerance():
    launches = []
    for li, (name, m, n) in enumerate(syn.LAYER_STREAM_13B):
        say(f"layer stream setup {name} {m}x{n} K=3")
        W = syn.weight(m, n, syn.weight_seed(4, li))
        x = syn.activations(1, n, syn.act_seed(4, li), "bf16")[0]
        d, packed, signs, alpha = bw.quantize_and_pack(to_dev(W), 3, bw.MBOK_F16)
        del signs, alpha
        y = torch.empty(m, dtype=torch.float32, device=DEV)
        launches.append((name, W, x, d, packed, x_to_dev(x, "bf16"), y))
    torch.cuda.empty_cache()

    def layer():
        for (_, _, _, d, packed, xt, y) in launches:
            bw.mbok_gemv(d, packed, xt, y)

    say("layer stream eager")
    layer()
    torch.cuda.synchronize()
    eager = [y.cpu().numpy().copy() for (*_, y) in launches]
    for li, (name, W, x, d, packed, xt, y) in enumerate(launches):
        say(f"layer stream oracle {name}")
        rows = _rows(d.m, 256, 400 + li)
        S, A, _ = oracle.residual_binarize(W[rows], 3, alpha_dtype="f16")
        ratio = oracle.max_error_ratio(eager[li][rows], oracle.product(S, A, x),
                                       oracle.bound(S, A, x))
        assert ratio <= TOL, (name, ratio)

    say("layer stream graph capture")
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        layer()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer()
    torch.cuda.synchronize()
    for r in range(REPLAYS):
        say(f"layer stream replay {r}")
        for (*_, y) in launches:
            y.fill_(-31.5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for li, (*_, y) in enumerate(launches):
            assert np.array_equal(y.cpu().numpy(), eager[li]), (launches[li][0], r)
        layer()  # eager work between replays
        torch.cuda.synchronize()
    del g


@pytest.mark.parametrize("li", [0, 2], ids=["qkv_15360x5120", "gate_up_27648x5120"])
def test_fused_launch_exact_regime(li):
    name, m, n = syn.LAYER_STREAM_13B[li]
    K = 3
    say(f"fused exact {name} {m}x{n} K={K}")
    S = syn.random_signs(K, m, n, seed=500 + li)
    A = syn.exact_alpha(K, m, n // 128, seed=510 + li).astype(np.float16)
    x = syn.exact_activations(1, n, seed=520 + li)[0]
    d, packed = pack_on_gpu(S, A, "f16")
    y = gemv(d, packed, x, "bf16", guard=9)
    rows = np.unique(np.r_[np.arange(0, m, 7), np.arange(m - 64, m)])
    want = oracle.product(S[:, rows], A[:, rows], x)
    assert np.array_equal(y[rows], want), np.max(np.abs(y[rows] - want))
    del packed
    torch.cuda.empty_cache()
