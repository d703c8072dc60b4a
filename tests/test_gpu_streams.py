"""Products enqueued on two streams at once.

The library keeps no device state between calls: scratch memory is a
workspace the caller passes in (the binding keeps one per stream), and the
kernels use no atomics.  So the decode, transposed, few-token and prefill
products enqueued on two streams at the same time must give the same bits as
the same calls run one after another on one stream.
"""
import os

import numpy as np
import pytest
import torch

import boolean_weight_amd as bw
import mbok_synth as syn
from gpu_util import DEV, pack_on_gpu, say, x_to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bw.load_library()
    yield
    torch.cuda.synchronize()


def _layer(K, m, n, seed):
    S = syn.random_signs(K, m, n, seed=seed)
    A = syn.exact_alpha(K, m, n // 128, seed=seed + 1).astype(np.float16)
    return pack_on_gpu(S, A, "f16")


def _jobs(tag):
    """The calls of one stream: (name, output tensor, function enqueuing it)."""
    seed = 700 if tag == "a" else 800
    d1, p1 = _layer(2, 4096, 4096, seed)
    d2, p2 = _layer(3, 1000, 2048, seed + 10)
    x = x_to_dev(syn.activations(1, 4096, seed + 20, "bf16")[0], "bf16")
    g = x_to_dev(syn.activations(1, 4096, seed + 21, "bf16")[0], "bf16")
    X2 = x_to_dev(syn.activations(2, 2048, seed + 24, "bf16"), "bf16")
    X5 = x_to_dev(syn.activations(5, 2048, seed + 22, "bf16"), "bf16")
    X300 = x_to_dev(syn.activations(300, 2048, seed + 23, "bf16"), "bf16")
    y = torch.empty(4096, dtype=torch.float32, device=DEV)
    dx = torch.empty(4096, dtype=torch.float32, device=DEV)
    Y2 = torch.empty((2, 1000), dtype=torch.float32, device=DEV)
    Y5 = torch.empty((5, 1000), dtype=torch.float32, device=DEV)
    Y300 = torch.empty((300, 1000), dtype=torch.float32, device=DEV)
    keep = (d1, p1, d2, p2, x, g, X2, X5, X300)  # keep the inputs alive
    return keep, [
        ("gemv", y, lambda: bw.mbok_gemv(d1, p1, x, y)),
        ("gemvt", dx, lambda: bw.mbok_gemvt(d1, p1, g, dx)),
        ("gemm2", Y2, lambda: bw.mbok_gemm(d2, p2, X2, Y2)),
        ("gemm5", Y5, lambda: bw.mbok_gemm(d2, p2, X5, Y5)),
        ("gemm300", Y300, lambda: bw.mbok_gemm(d2, p2, X300, Y300)),
    ]


@pytest.mark.parametrize("variant", ["stream", "split"])
def test_two_streams_give_the_sequential_bits(variant):
    say(f"two streams, decode variant {variant}")
    old = os.environ.get("MBOK_GEMV_VARIANT")
    os.environ["MBOK_GEMV_VARIANT"] = variant
    try:
        keep_a, jobs_a = _jobs("a")
        keep_b, jobs_b = _jobs("b")
        torch.cuda.synchronize()
        # one after another on the current stream
        want = {}
        for tag, jobs in (("a", jobs_a), ("b", jobs_b)):
            for name, out, fn in jobs:
                out.fill_(-1.0)
                fn()
                torch.cuda.synchronize()
                want[(tag, name)] = out.clone()
        # both streams at once, several rounds, calls interleaved on the host
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        for rnd in range(3):
            for _, out, _ in jobs_a + jobs_b:
                out.fill_(-2.0)
            s1.wait_stream(torch.cuda.current_stream())
            s2.wait_stream(torch.cuda.current_stream())
            for (_, _, fa), (_, _, fb) in zip(jobs_a, jobs_b):
                with torch.cuda.stream(s1):
                    fa()
                with torch.cuda.stream(s2):
                    fb()
            torch.cuda.synchronize()
            for tag, jobs in (("a", jobs_a), ("b", jobs_b)):
                for name, out, _ in jobs:
                    assert torch.equal(out, want[(tag, name)]), (rnd, tag, name)
        del keep_a, keep_b
    finally:
        if old is None:
            os.environ.pop("MBOK_GEMV_VARIANT", None)
        else:
            os.environ["MBOK_GEMV_VARIANT"] = old


def _device_layer(K, m, n, seed):
    """A layer packed from signs and scales drawn on the GPU (the comparison
    below is the library against itself, so no host copy is needed)."""
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    d = bw.mbok_desc_init(m, n, K)
    signs = (torch.randint(0, 2, (K, m, n), generator=gen, device=DEV, dtype=torch.int8) * 2 - 1)
    alpha = torch.rand((K, m, n // 128), generator=gen, device=DEV).to(torch.float16)
    packed = torch.empty(bw.mbok_packed_bytes(d), dtype=torch.uint8, device=DEV)
    bw.mbok_pack(d, signs, alpha, packed)
    torch.cuda.synchronize()
    return d, packed


def test_explicit_stream_workspace_grows():
    """Calls given an explicit stream (a torch stream, then its raw handle)
    while the current stream is another one: the binding's cached workspace
    for that stream is allocated on it and replaced when a larger shape needs
    more than it holds, and every result equals the same call on the current
    stream."""
    say("explicit-stream workspace: split decode, 16 KB then 3.2 MB workspace")
    old = os.environ.get("MBOK_GEMV_VARIANT")
    os.environ["MBOK_GEMV_VARIANT"] = "split"
    try:
        small = _device_layer(2, 1000, 2048, 910)
        large = _device_layer(1, 400000, 4096, 920)
        assert bw.mbok_gemv_workspace_bytes(small[0]) < (1 << 20) < \
            bw.mbok_gemv_workspace_bytes(large[0])
        xs = [x_to_dev(syn.activations(1, d.n, 930 + i, "bf16")[0], "bf16")
              for i, (d, _) in enumerate((small, large))]
        want = []
        for (d, p), x in zip((small, large), xs):
            y = torch.empty(d.m, dtype=torch.float32, device=DEV)
            bw.mbok_gemv(d, p, x, y)
            torch.cuda.synchronize()
            want.append(y.clone())
        s = torch.cuda.Stream()
        for handle in (s, s.cuda_stream):
            for i in (0, 1, 0, 1):
                (d, p), x = (small, large)[i], xs[i]
                y = torch.full((d.m,), -3.0, dtype=torch.float32, device=DEV)
                s.wait_stream(torch.cuda.current_stream())
                bw.mbok_gemv(d, p, x, y, stream=handle)
                torch.cuda.current_stream().wait_stream(s)
                torch.cuda.synchronize()
                assert torch.equal(y, want[i]), (type(handle).__name__, i)
    finally:
        if old is None:
            os.environ.pop("MBOK_GEMV_VARIANT", None)
        else:
            os.environ["MBOK_GEMV_VARIANT"] = old
