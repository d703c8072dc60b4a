"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Each check takes the oracle module `o` as an argument and raises
AssertionError when the oracle disagrees with the fact it checks.  The checks
are used twice: by test_oracle_pins.py on the real oracle, and by
test_oracle_mutations.py on copies of the oracle with a planted mistake, to
show that each plausible mistake is caught by at least one pin.

None of these checks re-types the oracle's formulas: each one reaches the
expected value by another route (a hand-worked fixture, an exact rational
computation, a least-squares solve, an exhaustive sign search, an integer
matmul, a constructed matrix with a known decomposition, direct indexing).
"""
from __future__ import annotations

import os
from fractions import Fraction

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))


# ----------------------------------------------------------------- helpers

def _ulp16(v: float) -> float:
    """Spacing of IEEE fp16 values around |v| (normal or subnormal)."""
    v = abs(v)
    if v < 2.0 ** -14:
        return 2.0 ** -24
    e = int(np.floor(np.log2(v)))
    return 2.0 ** (e - 10)


def rne_fraction(q: Fraction, mant_bits: int, emin: int) -> Fraction:
    """Round a positive rational to the nearest value with `mant_bits` bits of
    significand (incl. the leading one) and minimum normal exponent `emin`,
    ties to even.  Written from the definition of IEEE rounding."""
    assert q >= 0
    if q == 0:
        return Fraction(0)
    e = q.numerator.bit_length() - q.denominator.bit_length()
    if Fraction(2) ** e > q:
        e -= 1
    e = max(e, emin)
    quantum = Fraction(2) ** (e - (mant_bits - 1))
    n = q / quantum
    lo = n.numerator // n.denominator
    rem = n - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return lo * quantum


def read_golden(name: str = "hand_worked.txt"):
    """Parse a file of tests/golden/ into {section: {key: list}}."""
    out, cur = {}, None
    with open(os.path.join(HERE, "golden", name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            if line.startswith("["):
                cur = out.setdefault(line.strip("[]"), {})
                continue
            key, val = (s.strip() for s in line.split("=", 1))
            if "|" in val:
                cur[key] = [[float(v) for v in r.split()] for r in val.split("|")]
            else:
                cur[key] = [float(v) for v in val.split()]
    return out


def walsh_hadamard(n: int) -> np.ndarray:
    """Sylvester construction of the n x n +-1 Hadamard matrix (n a power of 2)."""
    H = np.array([[1]], dtype=np.int64)
    while H.shape[0] < n:
        H = np.block([[H, H], [H, -H]])
    return H


# ------------------------------------------------------------ scale rounding

def pin_round_alpha_rne(o):
    """The storage rounding equals exact IEEE round-to-nearest-even, including
    exact midpoints and fp16 subnormals."""
    rng = np.random.default_rng(5)
    vals = list(rng.uniform(1e-5, 0.2, size=300))
    # exact fp16 midpoints: an fp16 value plus half its spacing
    for v in (0.015625, 0.01171875, 0.3, 2.0 ** -13, 3 * 2.0 ** -20):
        v16 = float(np.float16(v))
        vals.append(v16 + _ulp16(v16) / 2)
        vals.append(v16 + _ulp16(v16) / 2 * (1 + 2.0 ** -40))
    for v in vals:
        got16 = Fraction(float(o.round_alpha(np.array([v]), "f16")[0]))
        want16 = rne_fraction(Fraction(v), 11, -14)
        assert got16 == want16, (v, got16, want16)
        got32 = Fraction(float(o.round_alpha(np.array([v]), "f32")[0]))
        want32 = rne_fraction(Fraction(v), 24, -126)
        assert got32 == want32, (v, got32, want32)


# ------------------------------------------------------------- quantizer

def pin_hand_worked(o):
    """Hand-worked examples in tests/golden/hand_worked.txt (group size 4)."""
    for name, ex in read_golden().items():
        K = int(ex["K"][0])
        W = np.array([ex["W"]], dtype=np.float32)
        for dt in ("f32", "f16"):
            S, A, R = o.residual_binarize(W, K, group=4, alpha_dtype=dt)
            for k in range(K):
                assert S[k, 0].tolist() == [int(v) for v in ex[f"B{k + 1}"]], (name, k, S[k, 0])
                assert float(A[k, 0, 0]) == ex["alpha"][k], (name, k, A[k, 0, 0])
            assert R[0].tolist() == ex["R"], (name, R[0])
            What = o.dequantize(S, A, group=4)
            assert What[0].tolist() == ex["W_hat"], (name, What[0])
            x = np.array(ex["x"])
            y = o.product(S, A, x, group=4)
            assert y.tolist() == ex["y"], (name, y)
            E = o.bound(S, A, x, group=4)
            assert E.tolist() == ex["bound"], (name, E)


def pin_sign_step(o):
    """I1: every sign agrees with the residual it was taken from, and exact
    zeros of either sign map to +1."""
    rng = np.random.default_rng(11)
    W = rng.normal(0, 0.02, size=(24, 256)).astype(np.float32)
    W[0, :7] = 0.0
    W[1, :5] = -0.0
    W[2, 128:131] = -0.0
    S, A, R, chain = o.residual_binarize(W, 3, alpha_dtype="f16", return_chain=True)
    for k in range(3):
        Rp = chain[k]
        assert set(np.unique(S[k]).tolist()) <= {-1, 1}
        assert np.all(S[k].astype(np.float64) * Rp >= 0), k
        assert np.all(S[k][Rp == 0] == 1), k
    assert np.all(S[0, 1, :5] == 1) and np.all(S[0, 0, :7] == 1)


def pin_scale_is_least_squares(o):
    """I2: for fixed signs the stored scale is the least-squares optimum
    (numpy lstsq on the group), rounded once; and it is no worse than its
    neighbouring fp16 values."""
    rng = np.random.default_rng(12)
    W = rng.normal(0, 0.02, size=(6, 384)).astype(np.float32)
    S, A, R, chain = o.residual_binarize(W, 3, alpha_dtype="f16", return_chain=True)
    for k in range(3):
        Rp = chain[k]
        for i in range(W.shape[0]):
            for g in range(3):
                cols = slice(128 * g, 128 * g + 128)
                s = S[k, i, cols].astype(np.float64)[:, None]
                c_star = np.linalg.lstsq(s, Rp[i, cols], rcond=None)[0][0]
                a = float(A[k, i, g])
                assert abs(c_star - a) <= _ulp16(a) / 2 * (1 + 1e-9) + 1e-15, (k, i, g, c_star, a)

                def energy(c):
                    return sum((Fraction(float(r)) - Fraction(c) * int(b)) ** 2
                               for r, b in zip(Rp[i, cols], S[k, i, cols]))
                e0 = energy(a)
                up = float(np.nextafter(np.float16(a), np.float16(np.inf)))
                dn = float(np.nextafter(np.float16(a), np.float16(0)))
                assert e0 <= energy(up) and e0 <= energy(dn), (k, i, g)


def pin_residual_chain(o):
    """I3: |R_k|^2 = |R_{k-1}|^2 - G (2 alpha a - alpha^2) per group, exactly,
    so the residual energy never rises; and W = W_hat + R_K exactly (Q7)."""
    rng = np.random.default_rng(13)
    W = rng.normal(0, 0.02, size=(5, 256)).astype(np.float32)
    # a small entry: exact as long as the residual's bits span <= 53 (W fp32,
    # scales near 2^-6); float64 carries the residual, so entries below about
    # 2^-30 would be rounded once (the same rounding on both sides)
    W[0, 3] = 1e-7
    for dt in ("f16", "f32"):
        S, A, R, chain = o.residual_binarize(W, 3, alpha_dtype=dt, return_chain=True)
        for i in range(W.shape[0]):
            for g in range(2):
                cols = range(128 * g, 128 * g + 128)
                prev = None
                for k in range(4):
                    Rk = [Fraction(float(chain[k][i, j])) for j in cols]
                    en = sum(r * r for r in Rk)
                    if k > 0:
                        alpha = Fraction(float(A[k - 1, i, g]))
                        a = sum(abs(r) for r in Rprev) / 128
                        assert en == prev - 128 * (2 * alpha * a - alpha * alpha), (dt, i, g, k)
                        assert en <= prev
                    prev, Rprev = en, Rk
        # exact reconstruction, via rationals
        for i in range(W.shape[0]):
            for j in range(0, 256, 7):
                w_hat = sum(Fraction(float(A[k, i, j // 128])) * int(S[k, i, j]) for k in range(3))
                assert Fraction(float(W[i, j])) == w_hat + Fraction(float(R[i, j])), (dt, i, j)


def pin_levels(o):
    """I4: a row-group of W_hat takes at most 2^K distinct values (exactly
    2^K for generic Gaussian data)."""
    rng = np.random.default_rng(14)
    W = rng.normal(0, 0.02, size=(8, 512)).astype(np.float32)
    for K in (1, 2, 3):
        S, A, R = o.residual_binarize(W, K, alpha_dtype="f16")
        What = o.dequantize(S, A)
        for i in range(8):
            for g in range(4):
                lv = np.unique(What[i, 128 * g:128 * g + 128])
                assert len(lv) == 2 ** K, (K, i, g, len(lv))


def pin_single_kernel_textbook(o):
    """I5: with K = 1 the result is the textbook single-scale binarization
    W_hat = (||W_g||_1 / G) sign(W_g) per row-group."""
    rng = np.random.default_rng(15)
    W = rng.normal(0, 0.02, size=(9, 256)).astype(np.float32)
    W[3, 10] = 0.0
    S, A, R = o.residual_binarize(W, 1, alpha_dtype="f32")
    What = o.dequantize(S, A)
    for i in range(9):
        for g in range(2):
            wg = W[i, 128 * g:128 * g + 128].astype(np.float64)
            scale = np.float32(np.linalg.norm(wg, ord=1) / 128)
            sgn = np.sign(wg)
            sgn[sgn == 0] = 1
            want = np.float64(scale) * sgn
            got = What[i, 128 * g:128 * g + 128]
            assert np.allclose(got, want, rtol=2 ** -23, atol=0), (i, g)


def pin_constructed_walsh(o):
    """I6: W = c1 S1 + c2 S2 + c3 S3 built from mutually orthogonal +-1
    patterns (distinct Walsh-Hadamard rows times a random +-1 vector) with
    dyadic c1 > c2 + c3, c2 > c3 > 0 is recovered exactly: the signs are the
    S_k, the scales are the c_k and the residual is zero."""
    H = walsh_hadamard(128)
    rng = np.random.default_rng(16)
    m, G, K = 6, 3, 3
    c = [2.0 ** -5 + 2.0 ** -8, 2.0 ** -7 + 2.0 ** -9, 2.0 ** -8 + 2.0 ** -10]
    W = np.zeros((m, 128 * G))
    Strue = np.zeros((K, m, 128 * G), dtype=np.int64)
    for i in range(m):
        for g in range(G):
            rows = rng.choice(128, size=K, replace=False)
            d = rng.choice([-1, 1], size=128)
            for k in range(K):
                Strue[k, i, 128 * g:128 * g + 128] = H[rows[k]] * d
    for k in range(K):
        W += c[k] * Strue[k]
    W = W.astype(np.float32)
    assert np.all(W.astype(np.float64) == sum(c[k] * Strue[k] for k in range(K)))
    for dt in ("f16", "f32"):
        S, A, R = o.residual_binarize(W, K, alpha_dtype=dt)
        assert np.array_equal(S.astype(np.int64), Strue), dt
        for k in range(K):
            assert np.all(A[k].astype(np.float64) == c[k]), (dt, k)
        assert np.all(R == 0), dt


def pin_exhaustive_search(o):
    """I7: with K = 1 and groups of 4 and 8, an exhaustive search over all
    2^G sign patterns, each with its least-squares scale, finds the oracle's
    signs and scale."""
    rng = np.random.default_rng(17)
    for G in (4, 8):
        W = rng.normal(0, 0.02, size=(10, 2 * G)).astype(np.float32)
        S, A, R = o.residual_binarize(W, 1, group=G, alpha_dtype="f32")
        pats = np.array([[1 if (p >> t) & 1 else -1 for t in range(G)]
                         for p in range(2 ** G)], dtype=np.float64)
        for i in range(10):
            for g in range(2):
                w = W[i, G * g:G * g + G].astype(np.float64)
                c = pats @ w / G                 # LS scale for each pattern
                err = ((w[None, :] - c[:, None] * pats) ** 2).sum(axis=1)
                # (s, c) and (-s, -c) fit equally well; the sign lives in B,
                # so only nonnegative scales are candidates
                err[c < 0] = np.inf
                best = int(np.argmin(err))
                assert np.array_equal(pats[best], S[0, i, G * g:G * g + G]), (G, i, g)
                assert float(A[0, i, g]) == float(np.float32(c[best])), (G, i, g)


def pin_gaussian_statistics(o):
    """I8: for Gaussian W the K = 1 relative residual tends to sqrt(1 - 2/pi)
    ~ 0.603; K = 2 and 3 fall in bands measured on the same construction."""
    W = np.random.default_rng(18).normal(0, 0.02, size=(128, 1024)).astype(np.float32)
    want = {1: np.sqrt(1 - 2 / np.pi), 2: 0.359, 3: 0.239}
    for K in (1, 2, 3):
        S, A, R = o.residual_binarize(W, K, alpha_dtype="f16")
        ratio = np.linalg.norm(R) / np.linalg.norm(W.astype(np.float64))
        assert abs(ratio - want[K]) < 0.012, (K, ratio)


# ---------------------------------------------------------------- product

def pin_integer_matmul(o):
    """P1: K = 1 and alpha = 1 reduce the product to the +-1 matrix times x,
    an exact int64 matmul for integer x."""
    rng = np.random.default_rng(21)
    S = rng.choice(np.array([-1, 1], dtype=np.int8), size=(1, 37, 384))
    A = np.ones((1, 37, 3), dtype=np.float32)
    X = rng.integers(-8, 9, size=(5, 384))
    Y = o.product(S, A, X.astype(np.float32))
    want = X.astype(np.int64) @ S[0].astype(np.int64).T
    assert np.array_equal(Y, want.astype(np.float64))


def pin_fraction_bruteforce(o):
    """P2: on tiny shapes the float64 product equals the exact rational triple
    loop (to 1e-12 of the bound in general, exactly in the exact regime)."""
    rng = np.random.default_rng(22)
    for K in (1, 2, 3):
        S = rng.choice(np.array([-1, 1], dtype=np.int8), size=(K, 3, 256))
        A = rng.uniform(0.001, 0.05, size=(K, 3, 2)).astype(np.float16)
        X = rng.standard_normal((2, 256)).astype(np.float32)
        Y = o.product(S, A, X)
        E = o.bound(S, A, X)
        Yf = o.product_fraction(S, A, X)
        for t in range(2):
            for i in range(3):
                assert abs(Fraction(float(Y[t, i])) - Yf[t][i]) <= Fraction(1e-12) * Fraction(float(E[t, i]))
        Ae = np.ldexp(1.0, -rng.integers(4, 9, size=(K, 3, 2))).astype(np.float32)
        Xe = rng.integers(-8, 9, size=(2, 256)).astype(np.float32)
        Ye = o.product(S, Ae, Xe)
        Yfe = o.product_fraction(S, Ae, Xe)
        for t in range(2):
            for i in range(3):
                assert Fraction(float(Ye[t, i])) == Yfe[t][i]


def pin_one_hot_and_all_ones(o):
    """P3: x = e_j gives y_i = sum_k alpha_k[i, j div 128] b_k[i, j] (direct
    indexing), and x = 1 on group g gives
    y_i = sum_k alpha_k[i, g] (2 popcount_k - 128).  These fix group
    alignment, scale indexing and operand orientation."""
    rng = np.random.default_rng(23)
    K, m, n = 3, 7, 512
    S = rng.choice(np.array([-1, 1], dtype=np.int8), size=(K, m, n))
    A = rng.uniform(0.001, 0.05, size=(K, m, n // 128)).astype(np.float16)
    for j in (0, 1, 127, 128, 300, 511):
        x = np.zeros(n)
        x[j] = 1.0
        y = o.product(S, A, x)
        for i in range(m):
            want = sum(float(A[k, i, j // 128]) * int(S[k, i, j]) for k in range(K))
            assert y[i] == want, (j, i)
    for g in range(4):
        x = np.zeros(n)
        x[128 * g:128 * g + 128] = 1.0
        y = o.product(S, A, x)
        for i in range(m):
            want = 0.0
            for k in range(K):
                pc = int(np.count_nonzero(S[k, i, 128 * g:128 * g + 128] > 0))
                want += float(A[k, i, g]) * (2 * pc - 128)
            assert y[i] == want, (g, i)


def pin_linearity(o):
    """P4: in the exact regime the product is additive over kernels and
    linear in x, to the last bit."""
    rng = np.random.default_rng(24)
    K, m, n = 3, 9, 384
    S = rng.choice(np.array([-1, 1], dtype=np.int8), size=(K, m, n))
    A = np.ldexp(1.0, -rng.integers(4, 9, size=(K, m, 3))).astype(np.float32)
    x1 = rng.integers(-8, 9, size=n).astype(np.float32)
    x2 = rng.integers(-8, 9, size=n).astype(np.float32)
    y = o.product(S, A, x1)
    parts = sum(o.product(S[k:k + 1], A[k:k + 1], x1) for k in range(K))
    assert np.array_equal(y, parts)
    assert np.array_equal(o.product(S, A, x1 + x2), y + o.product(S, A, x2))


def pin_bound(o):
    """The error scale E = sum_j |W_hat_ij| |x_j| dominates |y|, equals |y|
    when every term has the same sign, and equals |W_hat_ij| for x = e_j."""
    rng = np.random.default_rng(25)
    K, m, n = 2, 6, 256
    S = rng.choice(np.array([-1, 1], dtype=np.int8), size=(K, m, n))
    A = rng.uniform(0.001, 0.05, size=(K, m, 2)).astype(np.float16)
    X = rng.standard_normal((3, n))
    assert np.all(o.bound(S, A, X) >= np.abs(o.product(S, A, X)))
    Sp = np.ones((1, m, n), dtype=np.int8)
    Ap = A[:1]
    xp = np.abs(X[0])
    assert np.allclose(o.bound(Sp, Ap, xp), o.product(Sp, Ap, xp), rtol=1e-15)
    x = np.zeros(n)
    x[130] = -2.0
    e = o.bound(S, A, x)
    for i in range(m):
        w = sum(float(A[k, i, 1]) * int(S[k, i, 130]) for k in range(K))
        assert e[i] == 2.0 * abs(w)


def pin_error_ratio_hand_worked(o):
    """The tolerance's acceptance figure on the hand-worked cases of
    tests/golden/error_ratio.txt: the largest |y_dev - y_ref| / E, exact
    equality required where E = 0, and inf for a mismatch there or for a
    non-finite result."""
    cases = read_golden("error_ratio.txt")
    assert sorted(cases) == ["A", "B", "C", "D", "E", "F"]
    for name, c in cases.items():
        got = o.max_error_ratio(np.array(c["y_dev"]), np.array(c["y_ref"]), np.array(c["E"]))
        want = c["figure"][0]
        if np.isinf(want):
            assert got == np.inf, (name, got)
        else:
            assert got == want, (name, got, want)


def pin_error_ratio_decides_tolerance(o):
    """Against the tolerance written out element by element: a device result
    made from the reference plus a perturbation of exactly r * E (r drawn per
    entry, either sign) has figure max(r); the figure is <= 1e-3 exactly when
    every entry meets |diff| <= 1e-3 E; scaling y_dev - y_ref and E together
    leaves it unchanged."""
    rng = np.random.default_rng(27)
    for _ in range(20):
        T, m = rng.integers(1, 4), rng.integers(1, 40)
        E = rng.uniform(0.5, 4.0, size=(T, m)).round(3)
        E[rng.random(size=(T, m)) < 0.2] = 0.0
        Y_ref = rng.normal(size=(T, m)).round(3)
        r = rng.uniform(0.0, 2e-3, size=(T, m))
        sgn = rng.choice([-1.0, 1.0], size=(T, m))
        # powers of two keep Y_ref + sgn r E - Y_ref = sgn r E exact
        E = np.ldexp(1.0, np.round(np.log2(np.maximum(E, 1e-9))).astype(int)) * (E > 0)
        r = np.ldexp(np.floor(r * 2.0 ** 20), -20)
        Y_ref = np.ldexp(np.round(Y_ref * 2.0 ** 10), -10)
        Y_dev = Y_ref + sgn * r * E
        got = o.max_error_ratio(Y_dev, Y_ref, E)
        pos = E > 0
        want = float(np.max(r[pos])) if np.any(pos) else 0.0
        assert got == want, (got, want)
        ok = all(abs(Y_dev[t, i] - Y_ref[t, i]) <= 1e-3 * E[t, i]
                 for t in range(T) for i in range(m))
        assert (got <= 1e-3) == ok
        assert o.max_error_ratio(Y_ref + 4 * (Y_dev - Y_ref), Y_ref, 4 * E) == got
    # a single bad entry anywhere is found
    Y_ref = np.zeros((3, 50))
    E = np.ones((3, 50))
    for t, i in ((0, 0), (2, 49), (1, 17)):
        Y_dev = Y_ref.copy()
        Y_dev[t, i] = -0.5
        assert o.max_error_ratio(Y_dev, Y_ref, E) == 0.5


# ----------------------------------------------------------------- layout

def pin_pack_roundtrip(o):
    """P5: unpack(pack(S, A)) gives back S and A, with clean padding, for
    ragged m and every K."""
    rng = np.random.default_rng(26)
    for K, m, n, dt in ((1, 1, 128, "f32"), (2, 65, 256, "f16"), (3, 130, 384, "f16"),
                        (4, 64, 128, "f32")):
        S = rng.choice(np.array([-1, 1], dtype=np.int8), size=(K, m, n))
        A = rng.uniform(0.001, 0.05, size=(K, m, n // 128)).astype(
            np.float16 if dt == "f16" else np.float32)
        buf = o.pack(S, A, dt)
        assert buf.size == o.packed_nbytes(m, n, K, dt)
        S2, A2, clean = o.unpack(buf, m, n, K, dt)
        assert np.array_equal(S, S2) and np.array_equal(A, A2) and clean


def pin_layout_single_bit(o):
    """The header's addressing rule, evaluated by hand for single +1 entries:
    chunk ((rb G + g) K + k) 64 + r; within it, for column j = 128g + 32w +
    4q + e, byte 4w + e and bit q; the scale of (i, g, k) at value index
    ((rb G + g) K + k) 64 + r after the sign region."""
    K, m, n = 3, 130, 384
    G = n // 128
    m_pad = 192
    for (k, i, j) in ((0, 0, 0), (2, 129, 383), (1, 64, 130), (0, 63, 255), (2, 5, 9),
                      (1, 7, 1), (0, 9, 4), (2, 3, 32 + 29), (1, 100, 256 + 127)):
        S = -np.ones((K, m, n), dtype=np.int8)
        S[k, i, j] = 1
        A = np.zeros((K, m, G), dtype=np.float32)
        A[k, i, j // 128] = 1.5
        buf = o.pack(S, A, "f32")
        nbits = K * m_pad * n // 8
        rb, r, g = i // 64, i % 64, j // 128
        chunk = ((rb * G + g) * K + k) * 64 + r
        jj = j % 128
        w, q, e = jj // 32, (jj % 32) // 4, jj % 4
        byte = chunk * 16 + 4 * w + e
        nz = np.flatnonzero(buf[:nbits])
        assert nz.tolist() == [byte], ((k, i, j), nz[:4], byte)
        assert buf[byte] == 1 << q
        sc = buf[nbits:].view(np.float32)
        assert np.flatnonzero(sc).tolist() == [chunk] and sc[chunk] == 1.5


# ----------------------------------------------------------------- refit

def _cramer(Gm, r):
    """Exact solution of Gm a = r (Fractions) by Cramer's rule, the
    determinants expanded over all permutations; None when det Gm = 0."""
    from itertools import permutations

    K = len(r)

    def det(M):
        tot = Fraction(0)
        for p in permutations(range(K)):
            inv = sum(1 for x in range(K) for y in range(x + 1, K) if p[x] > p[y])
            term = Fraction(-1 if inv % 2 else 1)
            for x in range(K):
                term *= M[x][p[x]]
            tot += term
        return tot

    d = det(Gm)
    if d == 0:
        return None
    out = []
    for c in range(K):
        M = [[r[x] if y == c else Gm[x][y] for y in range(K)] for x in range(K)]
        out.append(det(M) / d)
    return out


def _ls_exact_by_cramer(w, b):
    """Normal equations of one group written with integer dot products."""
    bi = b.astype(np.int64)
    Gm = [[Fraction(int(bi[k] @ bi[l])) for l in range(len(bi))] for k in range(len(bi))]
    wf = [Fraction(float(v)) for v in w]
    r = [sum((f * int(s) for f, s in zip(wf, bi[k])), Fraction(0)) for k in range(len(bi))]
    return _cramer(Gm, r)


def _group_energy(w, b, a):
    """Exact squared error of one group for signs b (K, n) and scales a."""
    af = [Fraction(float(v)) for v in a]
    return sum((Fraction(float(w[j])) - sum(af[k] * int(b[k, j]) for k in range(len(af)))) ** 2
               for j in range(len(w)))


def _nearest_by_sort(w, a):
    """Vectorised nearest-level signs: all 2^K levels, ordered per weight by
    (distance, -level, -pattern index) with np.lexsort."""
    K = len(a)
    idx = np.arange(2 ** K)
    pats = np.array([[1 if (p >> k) & 1 else -1 for k in range(K)] for p in idx])
    lev = pats.astype(np.float64) @ np.asarray(a, dtype=np.float64)
    dist = np.abs(np.asarray(w, dtype=np.float64)[:, None] - lev[None, :])
    out = np.empty((K, len(w)), dtype=np.int64)
    for j in range(len(w)):
        order = np.lexsort((-idx, -lev, dist[j]))
        out[:, j] = pats[order[0]]
    return out


def pin_refit_hand_worked(o):
    """R1: the hand-worked alternating refit of tests/golden/hand_worked_refit.txt
    (K = 2, group of 4, one round, fp16 scales)."""
    for name, ex in read_golden("hand_worked_refit.txt").items():
        K, rounds = int(ex["K"][0]), int(ex["rounds"][0])
        W = np.array([ex["W"]], dtype=np.float32)
        S0, A0, _ = o.residual_binarize(W, K, group=4, alpha_dtype="f16")
        assert [float(v) for v in A0[:, 0, 0]] == ex["greedy_alpha"], (name, A0[:, 0, 0])
        assert _group_energy(W[0], S0[:, 0], A0[:, 0, 0]) == Fraction(ex["energy_greedy"][0])
        # the exact least-squares scales the fixture derives by hand
        q = _ls_exact_by_cramer(W[0], S0[:, 0])
        assert q == [Fraction(int(n), int(d)) for n, d in zip(ex["ls_num"], ex["ls_den"])], q
        S, A = o.refit(W, S0, A0, rounds=rounds, group=4, alpha_dtype="f16")
        assert A.dtype == np.float16
        for k in range(K):
            assert S[k, 0].tolist() == [int(v) for v in ex[f"B{k + 1}"]], (name, k, S[k, 0])
        assert [float(v) for v in A[:, 0, 0]] == ex["alpha"], (name, A[:, 0, 0])
        assert _group_energy(W[0], S[:, 0], A[:, 0, 0]) == Fraction(ex["energy"][0])


def pin_refit_scale_step(o):
    """R2: with rounds = 0 only the scale step runs: the signs are kept and
    every scale is the exact least-squares solution (Cramer's rule on
    rationals) rounded once to the dtype (IEEE rounding written out), and lies
    within half an ulp of numpy's lstsq solution."""
    rng = np.random.default_rng(31)
    for K, dt, mant, emin in ((2, "f16", 11, -14), (3, "f16", 11, -14), (3, "f32", 24, -126)):
        W = rng.normal(0, 0.02, size=(3, 256)).astype(np.float32)
        S0, A0, _ = o.residual_binarize(W, K, alpha_dtype=dt)
        S, A = o.refit(W, S0, A0, rounds=0, alpha_dtype=dt)
        assert np.array_equal(S, S0)
        for i in range(3):
            for g in range(2):
                cols = slice(128 * g, 128 * g + 128)
                q = _ls_exact_by_cramer(W[i, cols], S0[:, i, cols])
                ls = np.linalg.lstsq(S0[:, i, cols].T.astype(np.float64),
                                     W[i, cols].astype(np.float64), rcond=None)[0]
                for k in range(K):
                    want = rne_fraction(abs(q[k]), mant, emin) * (1 if q[k] >= 0 else -1)
                    got = float(A[k, i, g])
                    assert Fraction(got) == want, (K, dt, i, g, k, got, float(want))
                    ulp = _ulp16(got) if dt == "f16" else abs(got) * 2.0 ** -23
                    assert abs(ls[k] - got) <= ulp / 2 * (1 + 1e-6) + 1e-12, (K, dt, i, g, k)


def pin_refit_sign_step(o):
    """R3: after one round the signs are the nearest-level patterns for the
    scales of the first scale step (rounds = 0), found by a sorted search over
    all 2^K levels, and the final scales are the rounded least-squares
    solution for those signs."""
    rng = np.random.default_rng(32)
    K = 3
    W = rng.normal(0, 0.02, size=(2, 256)).astype(np.float32)
    S0, A0, _ = o.residual_binarize(W, K, alpha_dtype="f16")
    _, A1 = o.refit(W, S0, A0, rounds=0)
    S, A = o.refit(W, S0, A0, rounds=1)
    changed = 0
    for i in range(2):
        for g in range(2):
            cols = slice(128 * g, 128 * g + 128)
            want = _nearest_by_sort(W[i, cols], A1[:, i, g])
            assert np.array_equal(S[:, i, cols], want), (i, g)
            changed += int(np.sum(np.any(want != S0[:, i, cols], axis=0)))
            q = _ls_exact_by_cramer(W[i, cols], S[:, i, cols])
            for k in range(K):
                assert Fraction(float(A[k, i, g])) == \
                    rne_fraction(abs(q[k]), 11, -14) * (1 if q[k] >= 0 else -1)
    assert changed > 0  # the sign step did move some weights


def pin_refit_ties(o):
    """R4: the tie readings of the two steps on constructed groups.  Scale
    step: a least-squares scale that falls exactly halfway between fp16 (or
    fp32) values rounds to the even one, also in the subnormal range.  Sign
    step: a weight halfway between two levels takes the larger level; equal
    levels go to the larger pattern index sum_k [b_k = +1] 2^k."""
    # K = 1: the scale is the mean |w|; each row is a constant group of 4
    # (the last row sits 2^-40 above the midpoint of 0 and the smallest fp16
    # subnormal: it must round up, which a rounding at fp16's normal
    # precision first and to the subnormal grid second gets wrong)
    rows = [(1 + 2.0 ** -11, "f16", 1.0), (1 + 3 * 2.0 ** -11, "f16", 1 + 2 * 2.0 ** -10),
            (2.0 ** -24 + 2.0 ** -25, "f16", 2.0 ** -23), (2.0 ** -25, "f16", 0.0),
            (3 * 2.0 ** -26, "f16", 2.0 ** -24),
            ([2.0 ** -25 + 2.0 ** -38] + [2.0 ** -25] * 3, "f16", 2.0 ** -24)]
    for v, dt, want in rows:
        W = np.array([v if isinstance(v, list) else [v] * 4], dtype=np.float32)
        assert W[0].astype(np.float64).tolist() == (v if isinstance(v, list) else [v] * 4)
        S0 = np.ones((1, 1, 4), dtype=np.int8)
        A0 = np.zeros((1, 1, 1), dtype=np.float16)
        _, A = o.refit(W, S0, A0, rounds=0, group=4, alpha_dtype=dt)
        assert float(A[0, 0, 0]) == want, (v, float(A[0, 0, 0]), want)
    # fp32 tie: mean of {1, 1 + 2^-23} over a group of 2 is 1 + 2^-24
    W = np.array([[1.0, 1 + 2.0 ** -23]], dtype=np.float32)
    _, A = o.refit(W, np.ones((1, 1, 2), dtype=np.int8), np.zeros((1, 1, 1), np.float32),
                   rounds=0, group=2, alpha_dtype="f32")
    assert float(A[0, 0, 0]) == 1.0
    # sign step ties, straight on the oracle's nearest-level rule
    w = np.array([0.5, 0.0, -0.5, 1.0, 0.25, -1.0])
    for a in ([0.5, 0.25], [0.25, 0.25], [0.5, 0.0], [0.5, 0.25, 0.125]):
        got = o._nearest_levels(w, np.array(a))
        assert np.array_equal(got.astype(np.int64), _nearest_by_sort(w, a)), a
    got = o._nearest_levels(np.array([0.5, 0.0]), np.array([0.5, 0.25]))
    assert got[:, 0].tolist() == [1, 1] and got[:, 1].tolist() == [1, -1]
    got = o._nearest_levels(np.array([0.0]), np.array([0.25, 0.25]))
    assert got[:, 0].tolist() == [-1, 1]


def pin_refit_single_kernel(o):
    """R5: with K = 1 the refit changes nothing: the least-squares scale of
    sign(w) is mean |w| and the nearest of +-a to w is sign(w) (+a at 0)."""
    rng = np.random.default_rng(33)
    W = rng.normal(0, 0.02, size=(4, 256)).astype(np.float32)
    W[1, 5] = 0.0
    for dt in ("f16", "f32"):
        S0, A0, _ = o.residual_binarize(W, 1, alpha_dtype=dt)
        S, A = o.refit(W, S0, A0, rounds=2, alpha_dtype=dt)
        assert np.array_equal(S, S0) and np.array_equal(A, A0), dt


def pin_refit_walsh_fixed_point(o):
    """R6: the constructed exact decomposition of I6 (orthogonal Walsh sign
    patterns, dyadic scales) is a fixed point of the refit."""
    H = walsh_hadamard(128)
    rng = np.random.default_rng(34)
    c = [2.0 ** -5 + 2.0 ** -8, 2.0 ** -7 + 2.0 ** -9, 2.0 ** -8 + 2.0 ** -10]
    W = np.zeros((2, 256))
    Strue = np.zeros((3, 2, 256), dtype=np.int8)
    for i in range(2):
        for g in range(2):
            rows = rng.choice(128, size=3, replace=False)
            d = rng.choice([-1, 1], size=128)
            for k in range(3):
                Strue[k, i, 128 * g:128 * g + 128] = H[rows[k]] * d
    for k in range(3):
        W += c[k] * Strue[k]
    W = W.astype(np.float32)
    A0 = np.zeros((3, 2, 2), dtype=np.float16)
    for k in range(3):
        A0[k] = c[k]
    S, A = o.refit(W, Strue, A0, rounds=2)
    assert np.array_equal(S, Strue) and np.array_equal(A, A0)


def pin_refit_singular_gram(o):
    """R7: when the Gram matrix B^T B of a group is singular (two equal sign
    rows) the scales are kept, and the sign step keeps the larger pattern."""
    W = np.full((1, 128), 0.03125, dtype=np.float32)
    S0 = np.ones((2, 1, 128), dtype=np.int8)
    A0 = np.array([[[0.03125]], [[0.0]]], dtype=np.float16)
    S, A = o.refit(W, S0, A0, rounds=2)
    assert np.array_equal(S, S0) and np.array_equal(A, A0)


def pin_refit_lowers_error(o):
    """R8: on Gaussian weights the refit (two rounds) never raises a group's
    error by more than the scale rounding can, and lowers the total error
    clearly for K = 2 and 3 (the closed-form scales fit the weight, not the
    residual chain)."""
    rng = np.random.default_rng(35)
    W = rng.normal(0, 0.02, size=(4, 256)).astype(np.float32)
    for K in (2, 3):
        S0, A0, _ = o.residual_binarize(W, K, alpha_dtype="f16")
        S, A = o.refit(W, S0, A0, rounds=2)
        tot0 = tot = Fraction(0)
        for i in range(4):
            for g in range(2):
                cols = slice(128 * g, 128 * g + 128)
                e0 = _group_energy(W[i, cols], S0[:, i, cols], A0[:, i, g])
                e = _group_energy(W[i, cols], S[:, i, cols], A[:, i, g])
                slack = 128 * Fraction(K * _ulp16(float(np.max(np.abs(A[:, i, g]))))) ** 2
                assert e <= e0 + slack, (K, i, g, float(e), float(e0))
                tot0 += e0
                tot += e
        # measured on this seed: 0.935 (K = 2) and 0.818 (K = 3) of the greedy error
        assert tot < {2: Fraction(95, 100), 3: Fraction(85, 100)}[K] * tot0, (K, float(tot / tot0))


# ------------------------------------------------ residual energy, allocation

def pin_energy_walsh(o):
    """E1: the constructed exact decomposition of I6 has closed-form
    residual energies: 128 G (c1^2 + c2^2 + c3^2), 128 G (c2^2 + c3^2),
    128 G c3^2 and 0 per row (orthogonal patterns), and m times that for the
    layer."""
    H = walsh_hadamard(128)
    rng = np.random.default_rng(41)
    m, G, K = 3, 2, 3
    c = [2.0 ** -5 + 2.0 ** -8, 2.0 ** -7 + 2.0 ** -9, 2.0 ** -8 + 2.0 ** -10]
    W = np.zeros((m, 128 * G))
    for i in range(m):
        for g in range(G):
            rows = rng.choice(128, size=K, replace=False)
            d = rng.choice([-1, 1], size=128)
            for k in range(K):
                W[i, 128 * g:128 * g + 128] += c[k] * H[rows[k]] * d
    W = W.astype(np.float32)
    rows, layer = o.residual_energies(W, K, alpha_dtype="f16")
    want = [128 * G * sum(Fraction(ck) ** 2 for ck in c[k:]) for k in range(K + 1)]
    for k in range(K + 1):
        assert all(Fraction(float(v)) == want[k] for v in rows[k]), (k, rows[k], float(want[k]))
        assert Fraction(float(layer[k])) == m * want[k], (k, layer[k])


def pin_energy_single_kernel(o):
    """E2: with one kernel the residual energy of a group has the closed form
    |w|^2 - 128 (2 alpha a - alpha^2) with a = |w|_1 / 128 and alpha the
    stored scale; a row sums its groups exactly and rounds once, the layer
    adds the rounded rows exactly and rounds once."""
    rng = np.random.default_rng(42)
    W = rng.normal(0, 0.02, size=(5, 384)).astype(np.float32)
    S, A, _ = o.residual_binarize(W, 1, alpha_dtype="f16")
    rows, layer = o.residual_energies(W, 1, alpha_dtype="f16")
    total = Fraction(0)
    for i in range(5):
        e0 = Fraction(0)
        e1 = Fraction(0)
        for g in range(3):
            wg = [Fraction(float(v)) for v in W[i, 128 * g:128 * g + 128]]
            sq = sum(v * v for v in wg)
            a = sum(abs(v) for v in wg) / 128
            al = Fraction(float(A[0, i, g]))
            e0 += sq
            e1 += sq - 128 * (2 * al * a - al * al)
        assert rows[0, i] == float(e0) and rows[1, i] == float(e1), i
        total += Fraction(float(rows[1, i]))
    assert layer[1] == float(total)


def pin_energy_decreases(o):
    """E3: greedy kernels never raise the residual energy of a row (each step
    subtracts a least-squares fit), for K up to 4 and both scale dtypes."""
    rng = np.random.default_rng(43)
    W = rng.normal(0, 0.02, size=(4, 256)).astype(np.float32)
    for dt in ("f16", "f32"):
        rows, layer = o.residual_energies(W, 4, alpha_dtype=dt)
        assert np.all(np.diff(rows, axis=0) <= 0) and np.all(np.diff(layer) < 0), dt


def _read_allocations():
    cases = []
    for name, ex in read_golden("allocation.txt").items():
        sizes = [int(v) for v in ex["sizes"]]
        kmax = int(ex["kmax"][0])
        errors = [ex[f"errors_{l}"] for l in range(len(sizes))]
        for key, val in ex.items():
            if key.startswith("budget_"):
                want = tuple(int(v) for v in val)
                cases.append((name, sizes, kmax, errors, int(key[7:]),
                              None if not any(want) else want))
    return cases


def pin_allocation_hand_worked(o):
    """A1: the hand-worked allocations of tests/golden/allocation.txt,
    including the two tie rules and an infeasible budget."""
    for name, sizes, kmax, errors, budget, want in _read_allocations():
        got = o.allocate_kernels(errors, sizes, budget, kmax)
        assert got == want, (name, budget, got, want)


def _knapsack_best(errors, sizes, budget, kmax):
    """Least (error, bits) by dynamic programming over used bits (integers):
    best[b] = least error of the first l weights using exactly b bits."""
    INF = float("inf")
    best = {0: 0.0}
    for l, sz in enumerate(sizes):
        nxt = {}
        for b, e in best.items():
            for K in range(1, kmax + 1):
                nb = b + K * sz
                if nb > budget:
                    continue
                ne = e + float(errors[l][K - 1])
                if ne < nxt.get(nb, INF):
                    nxt[nb] = ne
        best = nxt
    if not best:
        return None
    return min((e, b) for b, e in best.items())


def pin_allocation_knapsack(o):
    """A2: on random instances (unequal sizes, dyadic errors so that float
    sums are exact too) the allocation reaches the least (error, bits) that a
    dynamic program over used bits finds, and stays within the budget."""
    rng = np.random.default_rng(44)
    for trial in range(40):
        L = int(rng.integers(1, 6))
        kmax = int(rng.integers(1, 5))
        sizes = [int(v) for v in rng.integers(1, 9, size=L)]
        errors = []
        for l in range(L):
            e = np.sort(rng.integers(0, 4096, size=kmax))[::-1] / 1024.0
            errors.append(e.tolist())
        budget = int(rng.integers(0, kmax * sum(sizes) + 3))
        got = o.allocate_kernels(errors, sizes, budget, kmax)
        want = _knapsack_best(errors, sizes, budget, kmax)
        if want is None:
            assert got is None, (trial, got)
            continue
        bits = sum(k * s for k, s in zip(got, sizes))
        err = sum(errors[l][got[l] - 1] for l in range(L))
        assert bits <= budget and (err, bits) == want, (trial, got, want)


def pin_allocation_greedy_convex(o):
    """A3: with equal sizes and convex, decreasing errors, adding one kernel
    at a time where it lowers the error most is optimal (separable convex
    allocation), so both reach the same least error."""
    rng = np.random.default_rng(45)
    for trial in range(30):
        L, kmax = int(rng.integers(2, 6)), 4
        errors = []
        for l in range(L):
            steps = np.sort(rng.integers(1, 512, size=kmax - 1))[::-1]  # shrinking gains
            e = [4096.0]
            for st in steps:
                e.append(e[-1] - float(st))
            errors.append([v / 1024.0 for v in e])
        budget = int(rng.integers(L, kmax * L + 1))
        K = [1] * L
        for _ in range(budget - L):
            gains = [(errors[l][K[l] - 1] - errors[l][K[l]]) if K[l] < kmax else -1.0
                     for l in range(L)]
            lbest = int(np.argmax(gains))
            if gains[lbest] <= 0:
                break
            K[lbest] += 1
        got = o.allocate_kernels(errors, [1] * L, budget, kmax)
        assert sum(errors[l][got[l] - 1] for l in range(L)) == \
            sum(errors[l][K[l] - 1] for l in range(L)), (trial, got, K)


def pin_allocation_monotone(o):
    """A4: a larger budget never gives a larger least error."""
    rng = np.random.default_rng(46)
    sizes = [3, 5, 2, 7]
    errors = [sorted(rng.random(4).tolist(), reverse=True) for _ in sizes]
    prev = None
    for budget in range(sum(sizes), 4 * sum(sizes) + 1):
        got = o.allocate_kernels(errors, sizes, budget, 4)
        err = sum((Fraction(errors[l][got[l] - 1]) for l in range(4)), Fraction(0))
        assert prev is None or err <= prev, budget
        prev = err


# ------------------------------------------------------- transposed product

def pin_transposed_integer(o):
    """T1: K = 1 and alpha = 1 reduce the transposed product to an exact
    int64 matmul g^T B; one-hot g gives a row of W_hat."""
    rng = np.random.default_rng(61)
    S = rng.choice(np.array([-1, 1], dtype=np.int8), size=(1, 45, 256))
    A = np.ones((1, 45, 2), dtype=np.float32)
    g = rng.integers(-8, 9, size=45)
    want = g.astype(np.int64) @ S[0].astype(np.int64)
    assert np.array_equal(o.product_transposed(S, A, g), want.astype(np.float64))
    S3 = rng.choice(np.array([-1, 1], dtype=np.int8), size=(3, 7, 384))
    A3 = (2.0 ** -rng.integers(3, 9, size=(3, 7, 3))).astype(np.float16)
    for i in (0, 6):
        e = np.zeros(7)
        e[i] = 1.0
        row = sum(np.repeat(A3[k, i].astype(np.float64), 128) * S3[k, i] for k in range(3))
        assert np.array_equal(o.product_transposed(S3, A3, e), row), i


def pin_transposed_adjoint(o):
    """T2: <W_hat x, g> = <x, W_hat^T g> exactly (rationals): the transposed
    product is the adjoint of the (pinned) forward product; and it is linear
    in g."""
    rng = np.random.default_rng(62)
    K, m, n = 2, 5, 256
    S = rng.choice(np.array([-1, 1], dtype=np.int8), size=(K, m, n))
    A = (2.0 ** -rng.integers(2, 7, size=(K, m, 2))).astype(np.float16)
    x = rng.integers(-8, 9, size=n).astype(np.float64)
    g = rng.integers(-8, 9, size=m).astype(np.float64)
    y = o.product(S, A, x)
    dx = o.product_transposed(S, A, g)
    lhs = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(y, g))
    rhs = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x, dx))
    assert lhs == rhs
    g2 = rng.integers(-8, 9, size=m).astype(np.float64)
    assert np.array_equal(o.product_transposed(S, A, g + 2 * g2),
                          o.product_transposed(S, A, g) + 2 * o.product_transposed(S, A, g2))
    G = np.stack([g, g2])
    assert np.array_equal(o.product_transposed(S, A, G)[1], o.product_transposed(S, A, g2))
    E = o.bound_transposed(S, A, G)
    assert np.all(np.abs(o.product_transposed(S, A, G)) <= E) and E.shape == (2, n)
    # with every term nonnegative the bound is the product itself; flipping
    # the signs of g or of the kernels leaves it unchanged
    Sp = np.ones_like(S)
    gp = np.abs(g)
    assert np.array_equal(o.bound_transposed(Sp, A, gp), o.product_transposed(Sp, A, gp))
    assert np.array_equal(o.bound_transposed(-S, A, -g), o.bound_transposed(S, A, g))


# ---------------------------------------------------------------- SVID

def pin_svid_exact_rank1(o):
    """V1: W = S (.) (a b^T) with positive fp16 vectors a, b of equal norm (b a
    permutation of a; m = n) is recovered exactly by one SVID kernel: |W| is
    the rank-1 a b^T, so sqrt(sigma) u = a and sqrt(sigma) v = b.  A zero row
    and a zero column (a 0 in a and in b) get s = 0 and signs +1."""
    rng = np.random.default_rng(71)
    n = 96
    a = (rng.integers(16, 64, size=n) / 256.0).astype(np.float16)
    a[5] = 0.0
    b = a[rng.permutation(n)]
    S = rng.choice(np.array([-1, 1], dtype=np.int8), size=(n, n))
    W = (S.astype(np.float64) * (a.astype(np.float64)[:, None] * b.astype(np.float64)[None, :]))
    W = W.astype(np.float32)
    zero_col = int(np.flatnonzero(b == 0)[0])
    Sg, SO, SI, R = o.svid_decompose(W, 1, alpha_dtype="f16")
    want_S = S.copy()
    want_S[5, :] = 1
    want_S[:, zero_col] = 1
    assert np.array_equal(Sg[0], want_S)
    assert np.array_equal(SO[0], a) and np.array_equal(SI[0], b)
    assert np.all(R == 0)


def _power_top(M, iters=200):
    """Top singular value of M by plain power iteration on M^T M."""
    v = np.ones(M.shape[1]) / np.sqrt(M.shape[1])
    for _ in range(iters):
        u = M @ v
        v = M.T @ u
        v /= np.linalg.norm(v)
    return float(np.linalg.norm(M @ v))


def pin_top_singular_arpack(o):
    """The iterative (ARPACK) branch of the library SVD, forced on small
    matrices by a size limit of 0, agrees with the dense LAPACK branch and
    with a plain power iteration: sigma to 1e-12, the unit vectors to 1e-9,
    both signed to a nonnegative sum; the exact rank-1 SVID recovery (V1)
    holds through that branch too."""
    rng = np.random.default_rng(74)
    for shape in ((120, 300), (300, 120), (64, 64)):
        M = np.abs(rng.normal(size=shape))
        s_it, u_it, v_it = o._top_singular(M, dense_limit=0)
        s_de, u_de, v_de = o._top_singular(M, dense_limit=M.size)
        assert u_it.shape == (shape[0],) and v_it.shape == (shape[1],)
        assert abs(s_it - s_de) <= 1e-12 * s_de
        assert abs(s_it - _power_top(M)) <= 1e-10 * s_de
        assert np.max(np.abs(u_it - u_de)) <= 1e-9 and np.max(np.abs(v_it - v_de)) <= 1e-9
        assert u_it.sum() >= 0 and v_it.sum() >= 0
        assert abs(np.linalg.norm(M @ v_it) - s_de) <= 1e-10 * s_de
        assert np.max(np.abs(M.T @ u_it - s_de * v_it)) <= 1e-9 * s_de
    saved = o.DENSE_SVD_LIMIT
    try:
        o.DENSE_SVD_LIMIT = 0
        pin_svid_exact_rank1(o)
    finally:
        o.DENSE_SVD_LIMIT = saved


def pin_svid_eckart_young(o):
    """V2: the sign-value split makes W - S (.) (s_out s_in^T) = S (.) (|W| -
    s_out s_in^T), so with the rank-1 SVD of |W| the residual energy is
    |W|_F^2 - sigma_1^2 (Eckart-Young), sigma_1 found here by a plain power
    iteration; the scale vectors are nonnegative (Perron); later kernels
    lower the residual further."""
    rng = np.random.default_rng(72)
    W = rng.normal(0, 0.02, size=(40, 256)).astype(np.float32)
    S, SO, SI, R = o.svid_decompose(W, 3, alpha_dtype="f32")
    W64 = W.astype(np.float64)
    sigma = _power_top(np.abs(W64))
    S1, SO1, SI1, R1 = o.svid_decompose(W, 1, alpha_dtype="f32")
    e1 = float(np.sum(R1 ** 2))
    assert abs(e1 - (np.sum(W64 ** 2) - sigma ** 2)) <= 1e-5 * np.sum(W64 ** 2), e1
    assert np.all(SO >= 0) and np.all(SI >= 0)
    # the successive kernels: each fit lowers the residual
    norms = [np.linalg.norm(W64)]
    for K in (1, 2, 3):
        norms.append(np.linalg.norm(o.svid_decompose(W, K, alpha_dtype="f32")[3]))
    assert norms[0] > norms[1] > norms[2] > norms[3]
    assert np.array_equal(S[:1], S1) and np.array_equal(SO[:1], SO1)


def pin_svid_product_grouped(o):
    """V3: when every s_in^k is constant on each 128-column group, the SVID
    product equals the group-scaled product with alpha_k[i, g] = s_out^k[i]
    * c_g (the pinned product), and the SVID bound matches too."""
    rng = np.random.default_rng(73)
    K, m, n = 2, 9, 384
    S = rng.choice(np.array([-1, 1], dtype=np.int8), size=(K, m, n))
    SO = (2.0 ** -rng.integers(1, 4, size=(K, m))).astype(np.float32)
    cg = (2.0 ** -rng.integers(1, 4, size=(K, 3))).astype(np.float32)
    SI = np.repeat(cg, 128, axis=1)
    A = (SO[:, :, None].astype(np.float64) * cg[:, None, :]).astype(np.float32)
    x = rng.integers(-8, 9, size=n).astype(np.float64)
    assert np.array_equal(o.svid_product(S, SO, SI, x), o.product(S, A, x))
    assert np.array_equal(o.svid_bound(S, SO, SI, x), o.bound(S, A, x))


ALL_PINS = [
    pin_round_alpha_rne, pin_hand_worked, pin_sign_step, pin_scale_is_least_squares,
    pin_residual_chain, pin_levels, pin_single_kernel_textbook, pin_constructed_walsh,
    pin_exhaustive_search, pin_gaussian_statistics, pin_integer_matmul,
    pin_fraction_bruteforce, pin_one_hot_and_all_ones, pin_linearity, pin_bound,
    pin_error_ratio_hand_worked, pin_error_ratio_decides_tolerance,
    pin_pack_roundtrip, pin_layout_single_bit,
    pin_refit_hand_worked, pin_refit_scale_step, pin_refit_sign_step, pin_refit_ties,
    pin_refit_single_kernel, pin_refit_walsh_fixed_point, pin_refit_singular_gram,
    pin_refit_lowers_error,
    pin_energy_walsh, pin_energy_single_kernel, pin_energy_decreases,
    pin_allocation_hand_worked, pin_allocation_knapsack, pin_allocation_greedy_convex,
    pin_allocation_monotone,
    pin_transposed_integer, pin_transposed_adjoint,
    pin_svid_exact_rank1, pin_svid_eckart_young, pin_svid_product_grouped,
    pin_top_singular_arpack,
]
