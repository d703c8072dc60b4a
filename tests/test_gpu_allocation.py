"""GPU parity of the residual energies (mbok_residual_energy) and the mixed-K
decoder layer they drive (kernel allocation under a bit budget), through the
C ABI.

Bars: row energies bit-identical to the oracle's (exact sums rounded once);
layer energies equal to the exactly rounded sum of the row energies; the
library's allocation from device energies equal to the oracle's allocation
from its own energies on the same seeded weights; each linear of the mixed
layer within the product tolerance on sampled rows.  Inputs are seeded
N(0, 0.02) weights; nothing the device computes is fed to the oracle.
"""
import math

import numpy as np
import pytest
import torch

import boolean_weight_amd as bw
import mbok_synth as syn
import oracle
from gpu_util import DEV, alpha_enum, gemv, say, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bw.load_library()
    yield
    torch.cuda.synchronize()


def energies_on_gpu(W: np.ndarray, K: int, dt: str, ldw: int | None = None):
    m, n = W.shape
    d = bw.mbok_desc_init(m, n, K, alpha_enum(dt))
    if ldw is not None and ldw > n:
        Wbig = np.full((m, ldw), np.nan, dtype=np.float32)  # padding is never read
        Wbig[:, :n] = W
        Wt = to_dev(Wbig)
    else:
        Wt = to_dev(W)
    rows = torch.full((K + 1, m), -1.0, dtype=torch.float64, device=DEV)
    layer = torch.full((K + 1,), -1.0, dtype=torch.float64, device=DEV)
    bw.mbok_residual_energy(d, Wt, rows, layer)
    return rows.cpu().numpy(), layer.cpu().numpy()


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("dt", ["f16", "f32"])
def test_energy_matches_oracle_small(K, dt):
    say(f"residual energy K={K} {dt}")
    W = syn.weight(37, 640, seed=800 + K)
    W[2, :9] = 0.0
    W[3, 5:11] = -0.0
    W[5, 128:256] = 0.0
    W[6, :] = 0.0                 # a whole zero row
    rows, layer = energies_on_gpu(W, K, dt)
    rows_ref, layer_ref = oracle.residual_energies(W, K, alpha_dtype=dt)
    assert np.array_equal(rows, rows_ref), np.argwhere(rows != rows_ref)[:5]
    assert np.array_equal(layer, layer_ref), (layer, layer_ref)


@pytest.mark.parametrize("n", [128, 256 * 128, 130 * 128])
def test_energy_group_counts(n):
    """One group per row, more groups than quads per workgroup (64), and a
    count that leaves some quads a second group."""
    say(f"residual energy n={n}")
    W = syn.weight(3, n, seed=810)
    rows, layer = energies_on_gpu(W, 2, "f16", ldw=n + 64)
    rows_ref, layer_ref = oracle.residual_energies(W, 2, alpha_dtype="f16")
    assert np.array_equal(rows, rows_ref) and np.array_equal(layer, layer_ref)


def test_energy_workload_sampled_rows():
    """The seven linears of the LLaMA-13B-shaped layer, K up to 4: sampled
    rows against the oracle; each layer energy is the exactly rounded sum of
    the row energies; energies fall with every kernel."""
    w = syn.WORKLOADS[4]
    for li, (name, m, n) in enumerate(w["linears"]):
        say(f"residual energy config 4 {name} {m}x{n} K=4")
        W = syn.weight(m, n, syn.weight_seed(4, li))
        rows, layer = energies_on_gpu(W, 4, "f16")
        sample = np.array(sorted({0, m - 1, *np.random.default_rng(li).choice(m, 6).tolist()}))
        rows_ref, _ = oracle.residual_energies(W[sample], 4, alpha_dtype="f16")
        assert np.array_equal(rows[:, sample], rows_ref), name
        for k in range(5):
            assert layer[k] == math.fsum(rows[k].tolist()), (name, k)
        assert np.all(np.diff(layer) < 0), name


def _small_layer(scale_rows: int):
    """The seven linears of the 13B-shaped layer with their column counts and
    `scale_rows` rows each (the oracle computes these whole)."""
    w = syn.WORKLOADS[4]
    out = []
    for li, (name, m, n) in enumerate(w["linears"]):
        out.append((name, syn.weight(scale_rows, n, syn.weight_seed(4, li) + 50)))
    return out


@pytest.mark.parametrize("avg", [1.5, 2.25, 3.0])
def test_allocation_from_device_energies_matches_oracle(avg):
    """Energies on the device, allocation in the library, against the
    oracle's energies and allocation of the same weights."""
    say(f"allocation avg={avg}")
    layer = _small_layer(12)
    Ws = [to_dev(W) for _, W in layer]
    K_dev, en_dev = bw.allocate_for_budget(Ws, avg, kmax=4)
    sizes, errors = [], []
    for _, W in layer:
        _, lay = oracle.residual_energies(W, 4, alpha_dtype="f16")
        sizes.append(W.size)
        errors.append(lay[1:].tolist())
    for (name, _), e_dev, e_ref in zip(layer, en_dev, errors):
        assert e_dev[1:] == e_ref, name
    want = oracle.allocate_kernels(errors, sizes, int(avg * sum(sizes)), 4)
    assert tuple(K_dev) == want, (K_dev, want)


def test_mixed_k_layer_product():
    """The 13B-shaped layer at 2.5 kernels per weight: the library allocates K
    per linear from device energies; every linear is then quantized with its
    K, packed and multiplied on the device, and sampled rows are checked
    against the oracle's own quantization and product."""
    w = syn.WORKLOADS[4]
    Ws = [syn.weight(m, n, syn.weight_seed(4, li)) for li, (name, m, n) in enumerate(w["linears"])]
    Wd = [to_dev(W) for W in Ws]
    say("mixed-K layer: allocation at 2.5 kernels per weight")
    K_alloc, energies = bw.allocate_for_budget(Wd, 2.5, kmax=4)
    sizes = [W.size for W in Ws]
    assert sum(k * s for k, s in zip(K_alloc, sizes)) <= int(2.5 * sum(sizes))
    assert len(set(K_alloc)) > 1, K_alloc  # the budget really mixes K
    for li, ((name, m, n), K) in enumerate(zip(w["linears"], K_alloc)):
        say(f"mixed-K layer {name} {m}x{n} K={K}")
        d, packed, signs, alpha = bw.quantize_and_pack(Wd[li], K, bw.MBOK_F16)
        del signs, alpha
        x = syn.activations(1, n, syn.act_seed(4, li), "bf16")[0]
        y = gemv(d, packed, x, "bf16")
        rows = np.array(sorted({0, m - 1, *np.random.default_rng(li).choice(m, 128).tolist()}))
        S, A, _ = oracle.residual_binarize(Ws[li][rows], K, alpha_dtype="f16")
        ratio = oracle.max_error_ratio(y[rows], oracle.product(S, A, x), oracle.bound(S, A, x))
        assert ratio <= TOL, (name, K, ratio)
        del packed
        torch.cuda.empty_cache()
