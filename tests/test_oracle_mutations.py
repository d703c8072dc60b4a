"""Planted mistakes in the oracle must be caught by its pins.

Each case edits the source text of one oracle function (a dropped term, a
wrong sign, a transposed operand, an off-by-one, a wrong bit order ...),
executes the edited function into a fresh copy of the oracle module, and runs
every pin of oracle_pins.py against that copy.  The case passes when at least
one pin fails.  All of this happens on the CPU; the real oracle is untouched.
"""
import importlib.util
import inspect
import os

import pytest

import oracle_pins as P

ORACLE_FILE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                           "oracle", "mbok_oracle.py")

# (case id, function, exact text in its source, replacement)
MUTATIONS = [
    ("sign_tie_to_minus_one", "residual_binarize",
     "np.where(R >= 0.0, 1, -1)", "np.where(R > 0.0, 1, -1)"),
    ("sign_flipped", "residual_binarize",
     "np.where(R >= 0.0, 1, -1)", "np.where(R >= 0.0, -1, 1)"),
    ("scale_from_original_weight", "residual_binarize",
     "absR = np.abs(R)", "absR = np.abs(W.astype(np.float64))"),
    ("scale_of_signed_residual", "residual_binarize",
     "absR = np.abs(R)", "absR = R"),
    ("scale_divisor_off_by_one", "residual_binarize",
     ".tolist()) / group", ".tolist()) / (group - 1)"),
    ("residual_uses_unrounded_scale", "residual_binarize",
     "alpha_cols = np.repeat(Ak.astype(np.float64), group, axis=1)",
     "alpha_cols = np.repeat(a, group, axis=1)"),
    ("residual_not_updated", "residual_binarize",
     "R = R - alpha_cols * Sk.astype(np.float64)", "R = R"),
    ("scale_double_rounded", "round_alpha",
     "np.asarray(a, dtype=np.float64).astype(_ALPHA_NP[alpha_dtype])",
     "np.asarray(a, dtype=np.float64).astype(np.float32).astype(_ALPHA_NP[alpha_dtype])"),
    ("scale_truncated", "round_alpha",
     "np.asarray(a, dtype=np.float64).astype(_ALPHA_NP[alpha_dtype])",
     "np.asarray(a, dtype=np.float64).astype(np.float32)"),
    ("dequantize_columns_tiled", "dequantize",
     "np.repeat(np.asarray(A[k], dtype=np.float64), group, axis=1)",
     "np.tile(np.asarray(A[k], dtype=np.float64), (1, group))"),
    ("dequantize_drops_last_kernel", "dequantize",
     "for k in range(K):", "for k in range(K - 1):"),
    ("dequantize_sign_inverted", "dequantize",
     "What += alpha_cols", "What -= alpha_cols"),
    ("product_transposed_operand", "product",
     "Y = X2 @ dequantize(S, A, group).T", "Y = dequantize(S, A, group) @ X2.T"),
    ("bound_without_abs_x", "bound",
     "E = np.abs(X2) @", "E = X2 @"),
    ("pack_msb_first", "pack",
     'axis=-1, bitorder="little")', 'axis=-1, bitorder="big")'),
    ("pack_kernel_group_swapped", "pack",
     "by.transpose(1, 3, 0, 2, 4)", "by.transpose(1, 0, 3, 2, 4)"),
    ("pack_scales_natural_order", "pack",
     "a = a.reshape(K, RB, ROW_BLOCK, G).transpose(1, 3, 0, 2)",
     "a = a.reshape(K, RB, ROW_BLOCK, G)"),
    ("unpack_msb_first", "unpack",
     'axis=-1, bitorder="little")', 'axis=-1, bitorder="big")'),
    ("unpack_bit_means_minus", "unpack",
     "np.where(bits[:, :m, :] == 1, 1, -1)", "np.where(bits[:, :m, :] == 1, -1, 1)"),
    ("refit_rhs_unsigned", "_ls_scales_exact",
     "wf[j] if b[k, j] > 0 else -wf[j]", "abs(wf[j])"),
    ("refit_gram_diagonal_only", "_ls_scales_exact",
     "Fraction(int(np.dot(b[k].astype(np.int64), b[l].astype(np.int64))))",
     "Fraction(len(wf) if k == l else 0)"),
    ("refit_pivot_not_divided", "_ls_scales_exact",
     "return [M[k][K] / M[k][k] for k in range(K)]", "return [M[k][K] for k in range(K)]"),
    ("refit_round_ties_odd", "_round_fraction",
     "(rem == Fraction(1, 2) and n % 2 == 1)", "(rem == Fraction(1, 2) and n % 2 == 0)"),
    ("refit_round_no_subnormal_clamp", "_round_fraction",
     "e = max(e, emin)", "e = e"),
    ("refit_round_truncates", "_round_fraction",
     "if rem > Fraction(1, 2) or", "if False and"),
    ("refit_level_tie_to_smaller", "_nearest_levels",
     "key = (abs(wj - lev), -lev, -idx)", "key = (abs(wj - lev), lev, -idx)"),
    ("refit_pattern_tie_to_smaller_index", "_nearest_levels",
     "key = (abs(wj - lev), -lev, -idx)", "key = (abs(wj - lev), -lev, idx)"),
    ("refit_level_sign_dropped", "_nearest_levels",
     "lev += float(a[k]) * b[k]", "lev += float(a[k])"),
    ("refit_steps_swapped", "refit",
     "if step % 2 == 0:", "if step % 2 == 1:"),
    ("refit_one_round_short", "refit",
     "for step in range(2 * rounds + 1):", "for step in range(2 * rounds - 1):"),
    ("refit_no_final_scale_step", "refit",
     "for step in range(2 * rounds + 1):", "for step in range(2 * rounds):"),
    ("refit_singular_zeroes_scales", "refit",
     "if q is not None:\n                        a = np.array([_round_fraction(v, alpha_dtype) for v in q])",
     "a = np.array([_round_fraction(v, alpha_dtype) for v in q]) if q is not None else 0 * a"),
    ("energy_of_abs_not_square", "residual_energies",
     "(Fraction(float(v)) ** 2 for v in Rk[i])", "(abs(Fraction(float(v))) for v in Rk[i])"),
    ("energy_one_kernel_late", "residual_energies",
     "Rk = chain[k]", "Rk = chain[min(k + 1, K)]"),
    ("energy_layer_drops_last_row", "residual_energies",
     "math.fsum(rows[k].tolist())", "math.fsum(rows[k][:-1].tolist())"),
    ("allocation_ignores_budget", "allocate_kernels",
     "if bits > budget:", "if False:"),
    ("allocation_ties_to_more_bits", "allocate_kernels",
     "key = (err, bits)", "key = (err, -bits)"),
    ("allocation_ties_to_last_vector", "allocate_kernels",
     "if best is None or key < best[0]:", "if best is None or key <= best[0]:"),
    ("allocation_size_ignored", "allocate_kernels",
     "bits = sum(int(k) * int(sz) for k, sz in zip(ks, sizes))", "bits = sum(int(k) for k in ks)"),
    ("allocation_error_of_wrong_kernel", "allocate_kernels",
     "err = err + Fraction(float(errors[l][ks[l] - 1]))",
     "err = err + Fraction(float(errors[l][min(ks[l], kmax - 1)]))"),
    ("transposed_uses_forward_orientation", "product_transposed",
     "D = G2 @ dequantize(S, A, group)", "D = (dequantize(S, A, group) @ G2.T).T"),
    ("transposed_bound_without_abs_g", "bound_transposed",
     "E = np.abs(G2) @", "E = G2 @"),
    ("svid_sign_tie_to_minus_one", "svid_decompose",
     "np.where(R >= 0.0, 1, -1)", "np.where(R > 0.0, 1, -1)"),
    ("svid_of_signed_residual", "svid_decompose",
     "_top_singular(np.abs(R))", "_top_singular(R)"),
    ("svid_sigma_not_split", "svid_decompose",
     "root = math.sqrt(sigma)", "root = sigma"),
    ("svid_in_vector_misordered", "svid_decompose",
     "SI[k] = round_alpha(root * v, alpha_dtype)", "SI[k] = round_alpha(root * v[::-1], alpha_dtype)"),
    ("svid_vectors_swapped", "svid_decompose",
     "SO[k] = round_alpha(root * u, alpha_dtype)\n        SI[k] = round_alpha(root * v, alpha_dtype)",
     "SO[k] = round_alpha(root * v, alpha_dtype)\n        SI[k] = round_alpha(root * u, alpha_dtype)"),
    ("svid_residual_not_updated", "svid_decompose",
     "R = R - Sk.astype(np.float64) * outer", "R = R"),
    ("svid_product_transposed_scales", "svid_dequantize",
     "SO[k].astype(np.float64)[:, None] *", "SO[k].astype(np.float64)[::-1, None] *"),
    ("error_ratio_min_for_max", "max_error_ratio",
     "return float(np.max(diff[~zero] / E[~zero]))", "return float(np.min(diff[~zero] / E[~zero]))"),
    ("error_ratio_abs_dropped", "max_error_ratio",
     "diff = np.abs(Y_dev - Y_ref)", "diff = Y_dev - Y_ref"),
    ("error_ratio_zero_bound_unchecked", "max_error_ratio",
     "if np.any(diff[zero] != 0):", "if False:"),
    ("error_ratio_zero_mask_dropped", "max_error_ratio",
     "zero = E == 0", "zero = E < 0"),
    ("error_ratio_relative_to_reference", "max_error_ratio",
     "return float(np.max(diff[~zero] / E[~zero]))",
     "return float(np.max(diff[~zero] / np.abs(Y_ref[~zero])))"),
    ("error_ratio_nan_passes", "max_error_ratio",
     "if not np.all(np.isfinite(diff)):", "if False:"),
    ("error_ratio_first_row_only", "max_error_ratio",
     "diff = np.abs(Y_dev - Y_ref)", "diff = np.abs(Y_dev - Y_ref); diff[..., 1:] = 0"),
    ("arpack_vectors_swapped", "_top_singular",
     "sigma, u, v = float(sa[0]), Ua[:, 0], Vta[0, :]", "sigma, u, v = float(sa[0]), Vta[0, :], Ua[:, 0]"),
    ("arpack_of_transpose", "_top_singular",
     "svds(M, k=1", "svds(M.T, k=1"),
    ("arpack_smallest_triple", "_top_singular",
     "svds(M, k=1, tol=0,", "svds(M, k=1, which='SM', tol=0,"),
]


def _mutated_oracle(func: str, old: str, new: str):
    spec = importlib.util.spec_from_file_location("mbok_oracle_mutant", ORACLE_FILE)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    src = inspect.getsource(getattr(mod, func))
    assert old in src, f"mutation text not found in {func}: {old!r}"
    exec(compile(src.replace(old, new, 1), ORACLE_FILE, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("case", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistake_is_caught(case):
    _, func, old, new = case
    mod = _mutated_oracle(func, old, new)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin(mod)
        except Exception as e:  # an assertion or a crash both expose the mistake
            caught.append(f"{pin.__name__}: {type(e).__name__}")
    assert caught, f"no pin caught the planted mistake {case[0]}"


def test_unmutated_copy_passes_every_pin():
    spec = importlib.util.spec_from_file_location("mbok_oracle_copy", ORACLE_FILE)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    for pin in P.ALL_PINS:
        pin(mod)
