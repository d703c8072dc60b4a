"""GPU parity of the alternating least-squares refit (mbok_refit) against the
oracle's refit, through the C ABI.

Bar: signs identical and scales bit-identical in their dtype.  The oracle
solves each group's normal equations on rationals and rounds once; the
device solves them exactly (integer Gram matrix and adjugate, exact float64
pair sums, a quotient rounded to odd) and must land on the same value.
Inputs: the oracle's own greedy signs and scales for seeded N(0, 0.02)
weights (never the device's), plus constructed groups for the tie, singular
and fixed-point cases.  Full-size layers are checked on sampled rows, which
the oracle refits on their own (rows are independent).
"""
import time

import numpy as np
import pytest
import torch

import boolean_weight_amd as bw
import mbok_synth as syn
import oracle
from gpu_util import DEV, alpha_enum, np_alpha, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    bw.load_library()
    yield
    torch.cuda.synchronize()


def refit_on_gpu(W: np.ndarray, S0: np.ndarray, A0: np.ndarray, dt: str, rounds: int,
                 ldw: int | None = None):
    K, m, n = S0.shape
    d = bw.mbok_desc_init(m, n, K, alpha_enum(dt))
    if ldw is not None and ldw > n:
        Wbig = np.full((m, ldw), np.nan, dtype=np.float32)  # padding is never read
        Wbig[:, :n] = W
        Wt = to_dev(Wbig)
    else:
        Wt = to_dev(W.astype(np.float32))
    signs = to_dev(S0.astype(np.int8))
    alpha = to_dev(A0.astype(np_alpha(dt)))
    bw.mbok_refit(d, Wt, signs, alpha, rounds)
    return signs.cpu().numpy(), alpha.cpu().numpy()


def assert_same(S, A, S_ref, A_ref, what):
    assert np.array_equal(S, S_ref), (what, np.argwhere(S != S_ref)[:5])
    bad = np.argwhere(A.view(np.uint8 if A.dtype == np.uint8 else
                             (np.uint16 if A.dtype == np.float16 else np.uint32))
                      != A_ref.view(np.uint16 if A_ref.dtype == np.float16 else np.uint32))
    assert bad.size == 0, (what, bad[:5], A[tuple(bad[0])], A_ref[tuple(bad[0])])


@pytest.mark.parametrize("K", [1, 2, 3, 4])
@pytest.mark.parametrize("dt", ["f16", "f32"])
@pytest.mark.parametrize("rounds", [0, 2])
def test_refit_matches_oracle_small(K, dt, rounds):
    m = 20 if K == 4 else 37
    say(f"refit small K={K} {dt} rounds={rounds} m={m}")
    W = syn.weight(m, 384, seed=700 + 10 * K + rounds)
    W[2, :9] = 0.0
    W[3, 5:11] = -0.0
    W[5, 128:256] = 0.0  # a whole zero group
    S0, A0, _ = oracle.residual_binarize(W, K, alpha_dtype=dt)
    S_ref, A_ref = oracle.refit(W, S0, A0, rounds=rounds, alpha_dtype=dt)
    S, A = refit_on_gpu(W, S0, A0, dt, rounds)
    assert_same(S, A, S_ref, A_ref, f"K={K} {dt} rounds={rounds}")
    if K >= 2 and rounds > 0:
        assert not np.array_equal(S, S0)  # the sign step moved some weights


def test_refit_after_device_greedy():
    """The whole quantizer on the device (greedy, then refit) against the
    oracle's (greedy, then refit) from the same W."""
    say("refit chained after the device greedy, 70x512 K=3 f16")
    W = syn.weight(70, 512, seed=711)
    d = bw.mbok_desc_init(70, 512, 3, bw.MBOK_F16)
    Wt = to_dev(W)
    signs = torch.empty((3, 70, 512), dtype=torch.int8, device=DEV)
    alpha = torch.empty((3, 70, 4), dtype=torch.float16, device=DEV)
    bw.mbok_residual_binarize(d, Wt, signs, alpha)
    bw.mbok_refit(d, Wt, signs, alpha, 2)
    S0, A0, _ = oracle.residual_binarize(W, 3, alpha_dtype="f16")
    S_ref, A_ref = oracle.refit(W, S0, A0, rounds=2)
    assert_same(signs.cpu().numpy(), alpha.cpu().numpy(), S_ref, A_ref, "chain")


def test_refit_row_stride():
    say("refit with ldw > n")
    W = syn.weight(33, 256, seed=712)
    S0, A0, _ = oracle.residual_binarize(W, 2, alpha_dtype="f16")
    S_ref, A_ref = oracle.refit(W, S0, A0, rounds=1)
    S, A = refit_on_gpu(W, S0, A0, "f16", 1, ldw=384)
    assert_same(S, A, S_ref, A_ref, "ldw")


def _walsh(n):
    H = np.array([[1]], dtype=np.int64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


def test_refit_constructed_groups():
    """Rows built so that the steps meet their special cases: an exact Walsh
    decomposition (a fixed point), constant groups (singular Gram matrix for
    K = 2), a zero row, least-squares scales exactly halfway between fp16
    values (normal and subnormal), a weight halfway between two levels, and
    weights on two equal levels (the pattern-index tie)."""
    say("refit constructed groups K=2 f16")
    rng = np.random.default_rng(713)
    H = _walsh(128)
    h = H[5]  # orthogonal to the all-ones row
    plus = np.flatnonzero(h > 0)
    m, n, K = 6, 256, 2
    Wd = np.zeros((m, n), dtype=np.float64)
    S0 = np.ones((K, m, n), dtype=np.int8)
    A0 = np.zeros((K, m, n // 128), dtype=np.float16)

    def ones_and_h(i, g, c1, c2):
        cols = slice(128 * g, 128 * g + 128)
        S0[1, i, cols] = h
        Wd[i, cols] = c1 + c2 * h
        A0[0, i, g], A0[1, i, g] = np.float16(c1), np.float16(c2)

    # row 0: exact decomposition 2^-5 S1 + 2^-7 S2 with orthogonal patterns
    for g in range(2):
        r = rng.choice(128, size=2, replace=False)
        dsg = rng.choice([-1, 1], size=128)
        for k, c in enumerate((2.0 ** -5, 2.0 ** -7)):
            S0[k, 0, 128 * g:128 * g + 128] = H[r[k]] * dsg
            Wd[0, 128 * g:128 * g + 128] += c * H[r[k]] * dsg
            A0[k, 0, g] = c
    # row 1: constant groups with equal sign rows (singular), greedy scales
    Wd[1, :128] = 0.03125
    Wd[1, 128:] = -0.0078125
    A0[0, 1, 0], A0[0, 1, 1] = 0.03125, 0.0078125
    S0[:, 1, 128:] = -1
    # row 2: zeros (singular for K = 2; every level is 0)
    # row 3: the scales (c1, c2) of signs (1, h) sit halfway between fp16
    # neighbours (normal, and subnormal for c2 of group 1): they round to the
    # even one.  In group 1 the rounding of c1 exceeds c2, so the sign step
    # then puts every weight on the level a1 + a2 and the Gram matrix turns
    # singular: the scales stay.
    ones_and_h(3, 0, 1 + 2.0 ** -11, 2.0 ** -3 + 2.0 ** -14)
    ones_and_h(3, 1, 0.25 + 2.0 ** -13, 3 * 2.0 ** -25)
    # row 4, group 0: scales (2^-5, 2^-7); one weight moved down to the
    # midpoint c1 of the levels c1 +- c2 and one moved up by c2, so that the
    # least-squares scales stay (c1, c2): the first takes the larger level
    ones_and_h(4, 0, 2.0 ** -5, 2.0 ** -7)
    Wd[4, plus[0]] = 2.0 ** -5
    Wd[4, plus[1]] = 2.0 ** -5 + 2 * 2.0 ** -7
    # row 4, group 1: c1 = c2, so the weights 0 lie on the two equal levels
    # (+1, -1) and (-1, +1): the larger pattern index, (-1, +1), wins
    ones_and_h(4, 1, 2.0 ** -6, 2.0 ** -6)
    # row 5: Gaussian, greedy start
    Wd[5] = rng.normal(0, 0.02, size=n)
    W = Wd.astype(np.float32)
    assert np.array_equal(W[:5].astype(np.float64), Wd[:5])  # constructed rows exact
    S0[:, 5:], A0[:, 5:], _ = oracle.residual_binarize(W[5:], K, alpha_dtype="f16")
    S_ref, A_ref = oracle.refit(W, S0, A0, rounds=2)
    # the constructed outcomes, as derived above
    assert np.array_equal(S_ref[:, 0], S0[:, 0]) and np.array_equal(A_ref[:, 0], A0[:, 0])
    assert A_ref[:, 3].astype(np.float64).T.tolist() == [[1.0, 0.125], [0.25, 2.0 ** -23]]
    assert np.all(S_ref[1, 3, 128:] == 1)
    assert S_ref[:, 4, plus[0]].tolist() == [1, 1]
    zeros = np.flatnonzero(h < 0) + 128
    assert np.all(S_ref[0, 4, zeros] == -1) and np.all(S_ref[1, 4, zeros] == 1)
    S, A = refit_on_gpu(W, S0, A0, "f16", 2)
    assert_same(S, A, S_ref, A_ref, "constructed")


def test_refit_rejects_rounds_out_of_range():
    say("refit argument checks")
    W = syn.weight(4, 128, seed=714)
    d = bw.mbok_desc_init(4, 128, 2, bw.MBOK_F16)
    signs = torch.ones((2, 4, 128), dtype=torch.int8, device=DEV)
    alpha = torch.zeros((2, 4, 1), dtype=torch.float16, device=DEV)
    for r in (-1, bw.MBOK_MAX_REFIT_ROUNDS + 1):
        with pytest.raises(bw.MbokError) as e:
            bw.mbok_refit(d, to_dev(W), signs, alpha, r)
        assert e.value.status == -1
    assert int(signs.min().item()) == 1 and float(alpha.abs().max().item()) == 0.0


@pytest.mark.parametrize("cfg,li", [(2, 0), (3, 0), (3, 2), (1, 0)])
def test_refit_workloads_sampled(cfg, li):
    """Full-size layers: the device's greedy + refit, checked on sampled rows
    against the oracle's greedy + refit of those rows."""
    w = syn.WORKLOADS[cfg]
    dt, K = w["alpha_dtype"], w["K"]
    name, m, n = w["linears"][li]
    say(f"refit config {cfg} {name} {m}x{n} K={K} {dt}")
    W = syn.weight(m, n, syn.weight_seed(cfg, li))
    d = bw.mbok_desc_init(m, n, K, alpha_enum(dt))
    Wt = to_dev(W)
    signs = torch.empty((K, m, n), dtype=torch.int8, device=DEV)
    alpha = torch.empty((K, m, n // 128), dtype=bw.alpha_torch_dtype(d.alpha_dtype), device=DEV)
    bw.mbok_residual_binarize(d, Wt, signs, alpha)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    bw.mbok_refit(d, Wt, signs, alpha, 2)
    torch.cuda.synchronize()
    say(f"  refit of {m}x{n} took {1e3 * (time.perf_counter() - t0):.2f} ms (first call)")
    rng = np.random.default_rng(cfg * 100 + li)
    rows = np.array(sorted(set(rng.choice(m, size=min(8, m), replace=False).tolist()) | {0, m - 1}))
    S0, A0, _ = oracle.residual_binarize(W[rows], K, alpha_dtype=dt)
    S_ref, A_ref = oracle.refit(W[rows], S0, A0, rounds=2, alpha_dtype=dt)
    assert_same(signs.cpu().numpy()[:, rows], alpha.cpu().numpy()[:, rows], S_ref, A_ref, name)
    del signs, alpha, Wt
    torch.cuda.empty_cache()
