"""mbok_gemvt_noalloc: the transposed product with the library's static
scratch in place of a caller workspace, for callers that cannot allocate.

Through the C ABI, two calls in a row (the second on a smaller input), each
compared bit for bit with mbok_gemvt given a workspace (the same kernels and
slicing) and, in the exact regime (integer g, power-of-two scales), with the
oracle's values.  The first shape needs the largest scratch any accepted
shape needs (n = 65408: two slice groups of 65408 partial sums).  A third
step records the call into a HIP graph and replays it with eager calls on
other shapes in between, so the shared scratch is overwritten between
replays."""
import ctypes

import numpy as np
import pytest
import torch

import boolean_weight_amd as bw
import mbok_synth as syn
import oracle
from gpu_util import DEV, pack_on_gpu, say, x_to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bw.load_library()
    yield
    torch.cuda.synchronize()


def _case(K, m, n, seed):
    S = syn.random_signs(K, m, n, seed=seed)
    A = syn.exact_alpha(K, m, n // 128, seed=seed + 1).astype(np.float16)
    g = syn.exact_activations(1, m, seed=seed + 2)[0]
    d, packed = pack_on_gpu(S, A, "f16")
    return S, A, g, d, packed, x_to_dev(g, "bf16")


def _noalloc(d, packed, gt):
    """One call through the raw C ABI on the current stream."""
    dx = torch.full((d.n,), -31.5, dtype=torch.float32, device=DEV)
    st = bw.load_library().mbok_gemvt_noalloc(
        ctypes.byref(d), packed.data_ptr(), gt.data_ptr(), bw.MBOK_BF16, dx.data_ptr(),
        torch.cuda.current_stream().cuda_stream)
    assert st == 0, bw.mbok_status_str(st)
    return dx


def _with_workspace(d, packed, gt):
    need = bw.mbok_gemvt_workspace_bytes(d)
    ws = torch.full((max(need, 256),), 0x55, dtype=torch.uint8, device=DEV)
    dx = torch.full((d.n,), -31.5, dtype=torch.float32, device=DEV)
    bw.mbok_gemvt(d, packed, gt, dx, workspace=ws)
    return dx


def test_noalloc_matches_workspace_call_twice():
    shapes = [(2, 300, 65408, 801), (3, 4096, 4096, 802)]  # second call smaller
    needs = [bw.mbok_gemvt_workspace_bytes(bw.mbok_desc_init(m, n, K, bw.MBOK_F16))
             for K, m, n, _ in shapes]
    assert needs[0] == 2 * 65408 * 4 and 0 < needs[1] < needs[0]
    assert needs[0] <= bw.mbok_gemvt_scratch_bytes()
    for K, m, n, seed in shapes:
        say(f"gemvt noalloc m={m} n={n} K={K}")
        S, A, g, d, packed, gt = _case(K, m, n, seed)
        got = _noalloc(d, packed, gt)
        ref = _with_workspace(d, packed, gt)
        torch.cuda.synchronize()
        got, ref = got.cpu().numpy(), ref.cpu().numpy()
        assert np.array_equal(got, ref), (m, n, K)
        assert np.array_equal(got.astype(np.float64), oracle.product_transposed(S, A, g)), (m, n, K)
        del packed
    torch.cuda.empty_cache()


def test_noalloc_graph_replays():
    say("gemvt noalloc graph")
    S, A, g, d, packed, gt = _case(3, 11008, 4096, 811)
    S2, A2, g2, d2, packed2, gt2 = _case(2, 300, 65408, 812)
    assert bw.mbok_gemvt_workspace_bytes(d) > 0
    want = oracle.product_transposed(S, A, g)
    want2 = oracle.product_transposed(S2, A2, g2)
    dx = torch.empty(d.n, dtype=torch.float32, device=DEV)

    def call():
        st = bw.load_library().mbok_gemvt_noalloc(
            ctypes.byref(d), packed.data_ptr(), gt.data_ptr(), bw.MBOK_BF16, dx.data_ptr(),
            torch.cuda.current_stream().cuda_stream)
        assert st == 0, bw.mbok_status_str(st)

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        call()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    gr = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gr):
        call()
    torch.cuda.synchronize()
    for r in range(3):
        dx.fill_(-31.5)
        torch.cuda.synchronize()
        gr.replay()
        torch.cuda.synchronize()
        assert np.array_equal(dx.cpu().numpy().astype(np.float64), want), r
        # another shape in between overwrites the shared scratch
        other = _noalloc(d2, packed2, gt2)
        torch.cuda.synchronize()
        assert np.array_equal(other.cpu().numpy().astype(np.float64), want2), r
    del gr
