"""Checkpoint and resume of a packed layer.

A layer is fully described by its descriptor fields and its packed buffer
(sign bits, then scales, in the documented MBOK_LAYOUT_L64 order), so saving
those two and loading them into fresh device memory must give the same
output bits from every product: decode, transposed, few-token and prefill.
The saved buffer is also checked byte for byte against the oracle's packing
of the same signs and scales, so a checkpoint holds the documented format and
not whatever the device happened to write.
"""
import numpy as np
import pytest
import torch

import boolean_weight_amd as bw
import mbok_synth as syn
from gpu_util import DEV, pack_on_gpu, say, x_to_dev
from oracle import mbok_oracle as orc

pytestmark = pytest.mark.gpu

FIELDS = ("m", "n", "K", "group", "alpha_dtype", "layout")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bw.load_library()
    yield
    torch.cuda.synchronize()


def _products(d, packed, x, g, X5, X300):
    y = torch.empty(d.m, dtype=torch.float32, device=DEV)
    dx = torch.empty(d.n, dtype=torch.float32, device=DEV)
    Y5 = torch.empty((5, d.m), dtype=torch.float32, device=DEV)
    Y300 = torch.empty((300, d.m), dtype=torch.float32, device=DEV)
    bw.mbok_gemv(d, packed, x, y)
    bw.mbok_gemvt(d, packed, g, dx)
    bw.mbok_gemm(d, packed, X5, Y5)
    bw.mbok_gemm(d, packed, X300, Y300)
    torch.cuda.synchronize()
    return {"gemv": y, "gemvt": dx, "gemm5": Y5, "gemm300": Y300}


@pytest.mark.parametrize("K,m,n,dt", [(3, 1000, 2048, "f16"), (2, 4096, 4096, "f32")])
def test_save_and_reload_gives_the_same_bits(tmp_path, K, m, n, dt):
    say(f"checkpoint K={K} m={m} n={n} alpha {dt}")
    S = syn.random_signs(K, m, n, seed=1200 + K)
    A = syn.exact_alpha(K, m, n // 128, seed=1300 + K)
    A = A.astype(np.float16 if dt == "f16" else np.float32)
    d, packed = pack_on_gpu(S, A, dt)
    x = x_to_dev(syn.activations(1, n, 1400, "bf16")[0], "bf16")
    g = x_to_dev(syn.activations(1, m, 1401, "bf16")[0], "bf16")
    X5 = x_to_dev(syn.activations(5, n, 1402, "bf16"), "bf16")
    X300 = x_to_dev(syn.activations(300, n, 1403, "bf16"), "bf16")
    before = _products(d, packed, x, g, X5, X300)

    path = tmp_path / "layer.pt"
    torch.save({"desc": {f: int(getattr(d, f)) for f in FIELDS},
                "packed": packed.cpu()}, path)
    del packed
    torch.cuda.synchronize()

    ck = torch.load(path, weights_only=True)
    host = ck["packed"].numpy()
    assert np.array_equal(host, orc.pack(S, A, dt)), "checkpoint differs from the documented layout"
    fd = ck["desc"]
    d2 = bw.mbok_desc_init(fd["m"], fd["n"], fd["K"], fd["alpha_dtype"])
    assert {f: int(getattr(d2, f)) for f in FIELDS} == fd
    # into fresh memory at another (16-byte aligned) address
    big = torch.zeros(host.size + 4096, dtype=torch.uint8, device=DEV)
    packed2 = big[1024:1024 + host.size]
    packed2.copy_(ck["packed"].to(DEV))
    after = _products(d2, packed2, x, g, X5, X300)
    for name in before:
        assert torch.equal(before[name], after[name]), name
