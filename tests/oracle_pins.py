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
    """Parse tests/golden/hand_worked.txt into {section: {key: list}}."""
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


ALL_PINS = [
    pin_round_alpha_rne, pin_hand_worked, pin_sign_step, pin_scale_is_least_squares,
    pin_residual_chain, pin_levels, pin_single_kernel_textbook, pin_constructed_walsh,
    pin_exhaustive_search, pin_gaussian_statistics, pin_integer_matmul,
    pin_fraction_bruteforce, pin_one_hot_and_all_ones, pin_linearity, pin_bound,
    pin_pack_roundtrip, pin_layout_single_bit,
]
