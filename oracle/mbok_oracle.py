"""CPU oracle for the Multi-Boolean-kernel (MBOK) linear layer.

TEST INFRASTRUCTURE.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this module.  The product path
(boolean_weight_amd and its HIP library) never imports, calls or links it,
and this module imports nothing from the product path.

Plain and slow on purpose: float64 NumPy, math.fsum and fractions.Fraction,
with no blocking, fusion or reordering beyond what each definition states.

Sources (page title, then the section on that page):
  [RN] "Highly Efficient and Effective LLMs with Multi-Boolean Architectures",
       Paper-Notes reading note (zhaoyang97.github.io):
         - 关键设计 / multi-kernel Boolean parameters: W ~ sum_k alpha_k B_k with
           B_k in {-1,+1}^{m x n}; K kernels give 2^K weight levels; Wx splits
           into K Boolean matrix-vector products.
         - 关键设计 / efficient scale optimisation: for fixed B_k the scales have
           a closed-form least-squares solution.
         - 关键设计 / group-wise strategy: an independent scale per group of
           columns; 消融实验 table: group size 128 is the usual choice.
         - 训练策略: kernels are initialised from the pretrained weight by SVD
           or greedy search.
  [GS] gist.science summaries of the same paper ("Successive SVID",
       "Extracción Sucesiva"): each further kernel is fitted to the residual
       error left by the previous ones; SVID approximates a weight by
       sign(W) (.) (s_out s_in^T), s_out s_in^T the rank-1 SVD of |W|
       ("Riformulazione Booleana e SVID", "Descomposición SVID").  The
       Italian summary, section "D.
       Allocazione Automatica dei Kernel": the number of kernels per weight
       is allocated for an average bit budget from residual error,
       importance and size.

Readings taken where the pages are silent:
  * scale structure: one scale per (kernel k, output row i, group g of 128
    consecutive input columns), as the group-wise strategy of [RN];
  * initialisation: greedy residual binarization, i.e. the residual chain of
    [GS] with the sign of the residual and its LS scale;
  * sign(0) = sign(-0.0) = +1 (B has no zero entry; either choice has the same
    squared error);
  * the scale is the exact float64 group mean of |R| (math.fsum, one
    rounding) rounded once, nearest-even, to the storage dtype, and the
    residual update uses that rounded scale, so W = W_hat + R_K exactly;
  * y is produced in fp32 by the device; the oracle keeps float64;
  * refit: the scale step solves the normal equations exactly and rounds
    once; the sign step takes each weight's nearest level (ties: larger
    level, then larger pattern index); a singular Gram matrix keeps the
    scales; rounds alternate (scale, sign) and end with a scale step;
  * allocation: residual energy = exact squared Frobenius norm of R_K, one
    rounding per row and one fsum over rows; importance is 1 for every
    weight (it needs data); the budget is a total of kernel-bits; total
    errors are compared exactly; ties go to fewer bits, then to the first K
    vector in lexicographic order.

parity pins: every function here is pinned in tests/test_oracle_pins.py
against closed forms, constructed examples, brute force (Fraction,
exhaustive sign search) and library routines (numpy lstsq, integer matmul).
"""
from __future__ import annotations

import math
from fractions import Fraction

import numpy as np

GROUP = 128
ROW_BLOCK = 64

_ALPHA_NP = {"f32": np.float32, "f16": np.float16}


def round_alpha(a: np.ndarray, alpha_dtype: str) -> np.ndarray:
    """Round float64 values once, nearest-even, to the scale storage dtype.

    NumPy converts float64 directly to float16 / float32 with one
    round-to-nearest-even step (pinned against an exact Fraction rounding in
    the tests)."""
    return np.asarray(a, dtype=np.float64).astype(_ALPHA_NP[alpha_dtype])


def residual_binarize(W: np.ndarray, K: int, group: int = GROUP,
                      alpha_dtype: str = "f16", return_chain: bool = False):
    """Greedy residual binarization of W (m x n) into K Boolean kernels.

    [RN] 训练策略 (greedy initialisation) with the residual chain of [GS] and
    the closed-form scale of [RN] 关键设计.  For every row i and group g
    (columns group*g .. group*g+group-1), k = 1..K:
        S_k = sign(R_{k-1})         with sign(0) = +1
        a   = fsum(|R_{k-1}|) / group   (exact sum, one rounding)
        A_k = round-to-nearest-even(a) in alpha_dtype
        R_k = R_{k-1} - A_k * S_k   (float64)
    Returns S int8 [K, m, n], A [K, m, n/group] (alpha dtype) and R_K float64
    [m, n]; with return_chain also the list [R_0, ..., R_K].
    """
    W = np.asarray(W)
    m, n = W.shape
    if n % group:
        raise ValueError("n must be a multiple of the group size")
    G = n // group
    R = W.astype(np.float64)
    chain = [R.copy()]
    S = np.empty((K, m, n), dtype=np.int8)
    A = np.empty((K, m, G), dtype=_ALPHA_NP[alpha_dtype])
    for k in range(K):
        Sk = np.where(R >= 0.0, 1, -1).astype(np.int8)
        a = np.empty((m, G), dtype=np.float64)
        absR = np.abs(R)
        for i in range(m):
            row = absR[i]
            for g in range(G):
                a[i, g] = math.fsum(row[g * group:(g + 1) * group].tolist()) / group
        Ak = round_alpha(a, alpha_dtype)
        alpha_cols = np.repeat(Ak.astype(np.float64), group, axis=1)
        R = R - alpha_cols * Sk.astype(np.float64)
        S[k] = Sk
        A[k] = Ak
        chain.append(R.copy())
    if return_chain:
        return S, A, R, chain
    return S, A, R


def _ls_scales_exact(w: np.ndarray, b: np.ndarray):
    """Exact least-squares scales of one group for fixed signs: the solution
    of the normal equations (B^T B) a = B^T w as Fractions, or None when the
    integer Gram matrix B^T B is singular.  w: float values (n_g,), b: +-1
    (K, n_g)."""
    K = b.shape[0]
    wf = [Fraction(float(v)) for v in w]
    G = [[Fraction(int(np.dot(b[k].astype(np.int64), b[l].astype(np.int64)))) for l in range(K)]
         for k in range(K)]
    r = [sum((wf[j] if b[k, j] > 0 else -wf[j] for j in range(len(wf))), Fraction(0))
         for k in range(K)]
    # Gauss-Jordan elimination on Fractions (exact)
    M = [G[k] + [r[k]] for k in range(K)]
    for c in range(K):
        piv = next((i for i in range(c, K) if M[i][c] != 0), None)
        if piv is None:
            return None
        M[c], M[piv] = M[piv], M[c]
        for i in range(K):
            if i != c and M[i][c] != 0:
                f = M[i][c] / M[c][c]
                M[i] = [M[i][j] - f * M[c][j] for j in range(K + 1)]
    return [M[k][K] / M[k][k] for k in range(K)]


def _round_fraction(q: Fraction, alpha_dtype: str) -> float:
    """Nearest-even rounding of an exact rational to the scale dtype."""
    if alpha_dtype == "f32":
        dt, mant = np.float32, 24
    else:
        dt, mant = np.float16, 11
    if q == 0:
        return 0.0
    sign = -1 if q < 0 else 1
    a = abs(q)
    # exponent of the leading bit, clamped to the subnormal range
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    emin = -14 if alpha_dtype == "f16" else -126
    e = max(e, emin)
    quantum = Fraction(2) ** (e - mant + 1)
    t = a / quantum
    n = t.numerator // t.denominator
    rem = t - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    v = float(sign * n * quantum)
    return float(dt(v))  # overflow becomes inf; the value is exact otherwise


def _nearest_levels(w: np.ndarray, a: np.ndarray) -> np.ndarray:
    """Signs (K, n_g) whose level sum_k a_k b_k is nearest to each w, the
    distance taken in float64; ties go to the larger level, then to the
    larger pattern index sum_k [b_k = +1] 2^k."""
    K = a.shape[0]
    best = np.empty((K, w.shape[0]), dtype=np.int8)
    for j in range(w.shape[0]):
        wj = float(w[j])
        choice = None
        for idx in range(2 ** K):
            b = [1 if (idx >> k) & 1 else -1 for k in range(K)]
            lev = 0.0
            for k in range(K):  # exact: K <= 4 values of the scale dtype
                lev += float(a[k]) * b[k]
            key = (abs(wj - lev), -lev, -idx)
            if choice is None or key < choice[0]:
                choice = (key, b)
        best[:, j] = choice[1]
    return best


def refit(W: np.ndarray, S: np.ndarray, A: np.ndarray, rounds: int = 2,
          group: int = GROUP, alpha_dtype: str = "f16"):
    """Alternating refit of the kernels of one layer for the weight itself
    ([RN] 关键设计, efficient scale optimisation: with the B_k fixed the scales
    have a closed-form least-squares solution, and B and alpha are optimised
    in turn, fixing one to update the other).  Per (row, group):
        repeat `rounds` times: alpha-step, then B-step; finally an alpha-step
        alpha-step: alpha = exact solution of (B^T B) alpha = B^T w, rounded
                    once (nearest-even) to the dtype; kept as is when the
                    integer Gram matrix is singular
        B-step:     each weight takes the sign pattern of its nearest level
                    sum_k alpha_k b_k (see _nearest_levels)
    W: (m, n) float32 values; S: (K, m, n) +-1; A: (K, m, G) scales.
    Returns new (S, A)."""
    S = S.copy()
    A = A.astype(np.float64).copy()
    K, m, n = S.shape
    G = n // group
    for i in range(m):
        for g in range(G):
            cols = slice(g * group, (g + 1) * group)
            w = W[i, cols]
            b = S[:, i, cols]
            a = A[:, i, g].copy()
            for step in range(2 * rounds + 1):
                if step % 2 == 0:
                    q = _ls_scales_exact(w, b)
                    if q is not None:
                        a = np.array([_round_fraction(v, alpha_dtype) for v in q])
                else:
                    b = _nearest_levels(w, a)
            S[:, i, cols] = b
            A[:, i, g] = a
    return S, A.astype(np.float16 if alpha_dtype == "f16" else np.float32)


def residual_energies(W: np.ndarray, K: int, group: int = GROUP, alpha_dtype: str = "f16"):
    """Residual energy of the greedy decomposition after k = 0..K kernels
    ([GS-it] "Allocazione Automatica dei Kernel": the allocation weighs the
    residual approximation error of each weight).
        rows[k, i] = the float64 nearest to the exact sum over row i of
                     R_k[i, j]^2 (R_0 = W; R_k as in residual_binarize)
        layer[k]   = fsum over i of rows[k, i]  (exact sum, one rounding)
    Returns rows float64 [K+1, m] and layer float64 [K+1]."""
    _, _, _, chain = residual_binarize(W, K, group, alpha_dtype, return_chain=True)
    m = np.asarray(W).shape[0]
    rows = np.empty((K + 1, m), dtype=np.float64)
    for k in range(K + 1):
        Rk = chain[k]
        for i in range(m):
            rows[k, i] = float(sum((Fraction(float(v)) ** 2 for v in Rk[i]), Fraction(0)))
    layer = np.array([math.fsum(rows[k].tolist()) for k in range(K + 1)])
    return rows, layer


def allocate_kernels(errors, sizes, budget: int, kmax: int):
    """Kernels per weight under a bit budget ([GS-it] "Allocazione Automatica
    dei Kernel": the number of kernels of each weight is chosen for an
    average bit budget, trading residual error against the weight's size;
    the importance term needs data and is left out, i.e. every weight counts
    the same).
        errors[l][K-1]  residual energy of weight l with K kernels
        sizes[l]        entries of weight l (bits per kernel)
        budget          largest total sum_l K_l * sizes[l]
    Every K vector in {1..kmax}^L is tried in lexicographic order; the total
    error is the exact (rational) sum of the float64 errors.  The least error
    wins, then the fewest bits, then the first vector in that order.  Returns
    the tuple of K_l, or None when even K = 1 everywhere exceeds the budget."""
    from itertools import product as cartesian

    L = len(sizes)
    best = None
    for ks in cartesian(range(1, kmax + 1), repeat=L):
        bits = sum(int(k) * int(sz) for k, sz in zip(ks, sizes))
        if bits > budget:
            continue
        err = Fraction(0)
        for l in range(L):
            err = err + Fraction(float(errors[l][ks[l] - 1]))
        key = (err, bits)
        if best is None or key < best[0]:
            best = (key, ks)
    return None if best is None else tuple(best[1])


# Matrices with at most this many entries take the dense LAPACK SVD; larger
# ones take ARPACK.  Read at call time, so a pin can lower it and drive the
# ARPACK branch on a small matrix.
DENSE_SVD_LIMIT = 1 << 22


def _top_singular(M: np.ndarray, dense_limit: int | None = None):
    """Largest singular value of a nonnegative float64 matrix M and its unit
    singular vectors (u, v), signed so that each sums to >= 0.  A library
    SVD: numpy's dense LAPACK SVD up to `dense_limit` entries (default
    DENSE_SVD_LIMIT), above that scipy's ARPACK (scipy.sparse.linalg.svds,
    one triple, tol=0, a start vector of ones, so the result is
    reproducible)."""
    limit = DENSE_SVD_LIMIT if dense_limit is None else dense_limit
    if M.size <= limit:
        U, sv, Vt = np.linalg.svd(M, full_matrices=False)
        sigma, u, v = float(sv[0]), U[:, 0], Vt[0]
    else:
        from scipy.sparse.linalg import svds
        Ua, sa, Vta = svds(M, k=1, tol=0, v0=np.ones(min(M.shape)))
        sigma, u, v = float(sa[0]), Ua[:, 0], Vta[0, :]
    if u.sum() < 0:
        u = -u
    if v.sum() < 0:
        v = -v
    return sigma, u, v


def svid_decompose(W: np.ndarray, K: int, alpha_dtype: str = "f16"):
    """Successive sign-value-independent decomposition (gist.science
    summaries, "Riformulazione Booleana e SVID" / "Successive SVID" /
    "Descomposición SVID"): a weight is approximated by sign(W) (.) (s_out
    s_in^T) with s_out s_in^T the rank-1 SVD of |W|, and every further kernel
    is fitted the same way to the residual left by the previous ones.  For
    k = 1..K, in float64:
        S_k   = sign(R_{k-1})  (sign(0) = +1),   R_0 = W
        sigma, u, v = the top singular triple of |R_{k-1}|
        s_out = sqrt(sigma) u,  s_in = sqrt(sigma) v, each rounded once to
                alpha_dtype (nearest-even)
        R_k   = R_{k-1} - S_k (.) (s_out s_in^T)   (rounded s, one rounding
                per entry)
    Returns S int8 [K, m, n], s_out [K, m] and s_in [K, n] (alpha dtype) and
    R_K float64 [m, n]."""
    W = np.asarray(W)
    m, n = W.shape
    R = W.astype(np.float64)
    S = np.empty((K, m, n), dtype=np.int8)
    SO = np.empty((K, m), dtype=_ALPHA_NP[alpha_dtype])
    SI = np.empty((K, n), dtype=_ALPHA_NP[alpha_dtype])
    for k in range(K):
        Sk = np.where(R >= 0.0, 1, -1).astype(np.int8)
        sigma, u, v = _top_singular(np.abs(R))
        root = math.sqrt(sigma)
        SO[k] = round_alpha(root * u, alpha_dtype)
        SI[k] = round_alpha(root * v, alpha_dtype)
        outer = SO[k].astype(np.float64)[:, None] * SI[k].astype(np.float64)[None, :]
        R = R - Sk.astype(np.float64) * outer
        S[k] = Sk
    return S, SO, SI, R


def svid_dequantize(S: np.ndarray, SO: np.ndarray, SI: np.ndarray) -> np.ndarray:
    """W_hat = sum_k S_k (.) (s_out^k s_in^k^T) in float64."""
    K, m, n = S.shape
    What = np.zeros((m, n), dtype=np.float64)
    for k in range(K):
        What += S[k].astype(np.float64) * (SO[k].astype(np.float64)[:, None] *
                                           SI[k].astype(np.float64)[None, :])
    return What


def svid_product(S, SO, SI, X):
    """Y = X . W_hat^T for the SVID representation, i.e. y = sum_k s_out^k
    (.) (S_k (s_in^k (.) x)), in float64; a 1-D x gives a 1-D y."""
    X = np.asarray(X, dtype=np.float64)
    one = X.ndim == 1
    X2 = X[None, :] if one else X
    Y = X2 @ svid_dequantize(S, SO, SI).T
    return Y[0] if one else Y


def svid_bound(S, SO, SI, X):
    """E[t, i] = sum_j |W_hat[i, j]| |X[t, j]| for the SVID representation."""
    X = np.asarray(X, dtype=np.float64)
    one = X.ndim == 1
    X2 = X[None, :] if one else X
    E = np.abs(X2) @ np.abs(svid_dequantize(S, SO, SI)).T
    return E[0] if one else E


def dequantize(S: np.ndarray, A: np.ndarray, group: int = GROUP) -> np.ndarray:
    """W_hat[i, j] = sum_k A_k[i, j // group] * S_k[i, j] in float64 ([RN]
    关键设计: W ~ sum_k alpha_k B_k, with group-wise alpha)."""
    K, m, n = S.shape
    What = np.zeros((m, n), dtype=np.float64)
    for k in range(K):
        alpha_cols = np.repeat(np.asarray(A[k], dtype=np.float64), group, axis=1)
        What += alpha_cols * S[k].astype(np.float64)
    return What


def product(S: np.ndarray, A: np.ndarray, X: np.ndarray,
            group: int = GROUP) -> np.ndarray:
    """Y = X . W_hat^T in float64: Y[t, i] = sum_j W_hat[i, j] X[t, j].

    X is [T, n] (a 1-D x is treated as T = 1 and a 1-D y is returned)."""
    X = np.asarray(X, dtype=np.float64)
    one = X.ndim == 1
    X2 = X[None, :] if one else X
    Y = X2 @ dequantize(S, A, group).T
    return Y[0] if one else Y


def bound(S: np.ndarray, A: np.ndarray, X: np.ndarray,
          group: int = GROUP) -> np.ndarray:
    """E[t, i] = sum_j |W_hat[i, j]| |X[t, j]|: the scale of the accepted error."""
    X = np.asarray(X, dtype=np.float64)
    one = X.ndim == 1
    X2 = X[None, :] if one else X
    E = np.abs(X2) @ np.abs(dequantize(S, A, group)).T
    return E[0] if one else E


def product_transposed(S: np.ndarray, A: np.ndarray, Gr: np.ndarray,
                       group: int = GROUP) -> np.ndarray:
    """DX = Gr . W_hat in float64: DX[t, j] = sum_i W_hat[i, j] Gr[t, i], the
    activation gradient of the layer (the Boolean-domain training of [GS]
    propagates gradients through the same weights; [RN] 关键设计: the product
    splits into K Boolean products).  Gr is [T, m]; a 1-D g gives a 1-D dx."""
    Gr = np.asarray(Gr, dtype=np.float64)
    one = Gr.ndim == 1
    G2 = Gr[None, :] if one else Gr
    D = G2 @ dequantize(S, A, group)
    return D[0] if one else D


def bound_transposed(S: np.ndarray, A: np.ndarray, Gr: np.ndarray,
                     group: int = GROUP) -> np.ndarray:
    """E[t, j] = sum_i |W_hat[i, j]| |Gr[t, i]|: the scale of the accepted
    error of the transposed product."""
    Gr = np.asarray(Gr, dtype=np.float64)
    one = Gr.ndim == 1
    G2 = Gr[None, :] if one else Gr
    E = np.abs(G2) @ np.abs(dequantize(S, A, group))
    return E[0] if one else E


def product_fraction(S: np.ndarray, A: np.ndarray, X: np.ndarray,
                     group: int = GROUP):
    """Exact rational Y[t][i] by the triple loop (tiny shapes only)."""
    K, m, n = S.shape
    T = X.shape[0]
    Af = [[[Fraction(float(A[k, i, g])) for g in range(n // group)]
           for i in range(m)] for k in range(K)]
    Y = []
    for t in range(T):
        row = []
        for i in range(m):
            acc = Fraction(0)
            for j in range(n):
                w = Fraction(0)
                for k in range(K):
                    w += Af[k][i][j // group] * int(S[k, i, j])
                acc += w * Fraction(float(X[t, j]))
            row.append(acc)
        Y.append(row)
    return Y


def max_error_ratio(Y_dev: np.ndarray, Y_ref: np.ndarray, E: np.ndarray) -> float:
    """The acceptance figure of the tolerance: max over entries of
    |Y_dev - Y_ref| / E, where E is the bound sum_j |W_hat_ij| |x_j|; a result
    is accepted when this is at most 1e-3.  An entry with E == 0 must match
    exactly (+0 equals -0), else the figure is inf; a non-finite difference
    (NaN or inf in Y_dev) satisfies no bound and also gives inf."""
    Y_dev = np.asarray(Y_dev, dtype=np.float64)
    Y_ref = np.asarray(Y_ref, dtype=np.float64)
    E = np.asarray(E, dtype=np.float64)
    diff = np.abs(Y_dev - Y_ref)
    if not np.all(np.isfinite(diff)):
        return math.inf
    zero = E == 0
    if np.any(diff[zero] != 0):
        return math.inf
    if not np.any(~zero):
        return 0.0
    return float(np.max(diff[~zero] / E[~zero]))


# --------------------------------------------------------------------------
# Packed layout MBOK_LAYOUT_L64, written from its specification in the
# library header: sign chunks of 16 bytes at chunk index
# ((rb*G + g)*K + k)*64 + r (rb = i // 64, r = i % 64); byte 4w + e of a
# chunk, bit q, is column 128g + 32w + 4q + e; bit 1 = +1.  Then the scales in
# the same (rb, g, k, r) order, in the scale dtype.  Padding rows are zero.
# --------------------------------------------------------------------------

def packed_nbytes(m: int, n: int, K: int, alpha_dtype: str) -> int:
    m_pad = -(-m // ROW_BLOCK) * ROW_BLOCK
    G = n // GROUP
    return K * m_pad * n // 8 + K * m_pad * G * np.dtype(_ALPHA_NP[alpha_dtype]).itemsize


def pack(S: np.ndarray, A: np.ndarray, alpha_dtype: str) -> np.ndarray:
    """Pack int8 signs [K, m, n] and scales [K, m, G] into the L64 byte buffer."""
    K, m, n = S.shape
    G = n // GROUP
    m_pad = -(-m // ROW_BLOCK) * ROW_BLOCK
    RB = m_pad // ROW_BLOCK
    nbits = K * m_pad * n // 8
    buf = np.zeros(packed_nbytes(m, n, K, alpha_dtype), dtype=np.uint8)
    # bit value per (k, i, j): 1 for +1 (entries >= 0), 0 for -1; padding rows 0
    b = np.zeros((K, m_pad, n), dtype=np.uint8)
    b[:, :m, :] = (S >= 0)
    # column 128g + 32w + 4q + e -> byte 4w + e of chunk (i, g, k), bit q
    cols = b.reshape(K, m_pad, G, 4, 8, 4)                # [k, i, g, w, q, e]
    cols = cols.transpose(0, 1, 2, 3, 5, 4)               # [k, i, g, w, e, q]
    by = np.packbits(cols, axis=-1, bitorder="little")    # [k, i, g, w, e]
    by = by.reshape(K, RB, ROW_BLOCK, G, 16)              # [k, rb, r, g, 4w+e]
    buf[:nbits] = by.transpose(1, 3, 0, 2, 4).reshape(-1)  # [rb, g, k, r, byte]
    scale_dt = _ALPHA_NP[alpha_dtype]
    a = np.zeros((K, m_pad, G), dtype=scale_dt)
    a[:, :m, :] = A
    a = a.reshape(K, RB, ROW_BLOCK, G).transpose(1, 3, 0, 2)  # [rb, g, k, r]
    buf[nbits:] = np.ascontiguousarray(a).reshape(-1).view(np.uint8)
    return buf


def unpack(buf: np.ndarray, m: int, n: int, K: int, alpha_dtype: str):
    """Read an L64 buffer back into int8 signs [K, m, n] and scales [K, m, G].

    Also returns whether every padding bit and padding scale is zero."""
    buf = np.asarray(buf, dtype=np.uint8)
    G = n // GROUP
    m_pad = -(-m // ROW_BLOCK) * ROW_BLOCK
    RB = m_pad // ROW_BLOCK
    nbits = K * m_pad * n // 8
    if buf.size != packed_nbytes(m, n, K, alpha_dtype):
        raise ValueError("packed buffer has the wrong size")
    by = buf[:nbits].reshape(RB, G, K, ROW_BLOCK, 4, 4)   # [rb, g, k, r, w, e]
    by = by.transpose(2, 0, 3, 1, 4, 5)                   # [k, rb, r, g, w, e]
    bits = np.unpackbits(by[..., None], axis=-1, bitorder="little")  # [..., w, e, q]
    bits = bits.transpose(0, 1, 2, 3, 4, 6, 5)            # [k, rb, r, g, w, q, e]
    bits = bits.reshape(K, m_pad, n)                      # column 128g+32w+4q+e
    S = np.where(bits[:, :m, :] == 1, 1, -1).astype(np.int8)
    scale_dt = _ALPHA_NP[alpha_dtype]
    sc = buf[nbits:].view(scale_dt).reshape(RB, G, K, ROW_BLOCK)
    sc = sc.transpose(2, 0, 3, 1).reshape(K, m_pad, G)   # [k, i, g]
    A = np.ascontiguousarray(sc[:, :m, :])
    pad_clean = bool(np.all(bits[:, m:, :] == 0) and np.all(sc[:, m:, :] == 0))
    return S, A, pad_clean
