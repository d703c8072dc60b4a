"""Seeded synthetic inputs for the MBOK linear layer.

This module only draws random numbers and shapes them; it holds none of the
method's arithmetic (no signs, scales, residuals or products).  Both the CPU
oracle and the HIP path receive their inputs from here, so the two sides see
identical data.

Workloads (all synthetic; no checkpoint or dataset is read):
  * W ~ N(0, 0.02) in fp32 (0.02 is the standard deviation), standing in for
    LLaMA-7B / LLaMA-13B linear weights of the same shapes.
  * x ~ N(0, 1), rounded to bf16 (nearest-even) where the workload is bf16,
    kept fp32 otherwise.
  * "exact" inputs for bit-exact checks: integer activations in [-8, 8] and
    power-of-two scales 2^-e, e in {4..8}, with uniformly random +-1 signs;
    "spread" scales 2^-e with e in {2..13} for the two-term prefill product.
Generator: numpy.random.default_rng(seed) (PCG64).
"""
from __future__ import annotations

import numpy as np

GROUP = 128

# The five workloads.  "linears" lists (name, m_out, n_in); K is the number of
# Boolean kernels used for throughput; T lists token counts.
WORKLOADS = {
    1: dict(name="single linear 256x512", linears=[("w", 256, 512)], K=2,
            T=[1], x_dtype="f32", alpha_dtype="f32"),
    2: dict(name="LLaMA-7B attention projection 4096x4096",
            linears=[("q_proj", 4096, 4096)], K=2, T=[1], x_dtype="bf16",
            alpha_dtype="f16"),
    3: dict(name="LLaMA-7B MLP gate/up 11008x4096 and down 4096x11008",
            linears=[("gate_proj", 11008, 4096), ("up_proj", 11008, 4096),
                     ("down_proj", 4096, 11008)],
            K=3, T=[1, 4, 16], x_dtype="bf16", alpha_dtype="f16"),
    4: dict(name="LLaMA-13B decoder layer, seven linears",
            linears=[("q_proj", 5120, 5120), ("k_proj", 5120, 5120),
                     ("v_proj", 5120, 5120), ("o_proj", 5120, 5120),
                     ("gate_proj", 13824, 5120), ("up_proj", 13824, 5120),
                     ("down_proj", 5120, 13824)],
            K=3, T=[1], x_dtype="bf16", alpha_dtype="f16"),
    5: dict(name="prefill GEMM 11008x4096, 2048 tokens",
            linears=[("gate_proj", 11008, 4096)], K=3, T=[2048],
            x_dtype="bf16", alpha_dtype="f16"),
}


# The LLaMA-13B-shaped layer as it runs per token: q|k|v and gate|up share
# their input and run as one launch each (rows stacked), then o and down.
# Launch li draws its weight from weight_seed(4, li) and its activations from
# act_seed(4, li).
LAYER_STREAM_13B = [("qkv_proj", 3 * 5120, 5120), ("o_proj", 5120, 5120),
                    ("gate_up_proj", 2 * 13824, 5120), ("down_proj", 5120, 13824)]


def weight_seed(config: int, layer: int = 0) -> int:
    return 1000 + 10 * config + layer


def act_seed(config: int, layer: int = 0) -> int:
    return 2000 + 10 * config + layer


def weight(m: int, n: int, seed: int, std: float = 0.02) -> np.ndarray:
    """fp32 [m, n] drawn from N(0, std^2)."""
    rng = np.random.default_rng(seed)
    return rng.normal(0.0, std, size=(m, n)).astype(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest-even); returns the uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    nan = np.isnan(np.asarray(a, dtype=np.float32))
    out = rounded.astype(np.uint16)
    out[nan] = 0x7FC0
    return out


def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to the fp32 values they denote (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def activations(T: int, n: int, seed: int, dtype: str = "bf16") -> np.ndarray:
    """fp32 [T, n] ~ N(0, 1); for dtype 'bf16' every value is bf16-representable."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(size=(T, n)).astype(np.float32)
    if dtype == "bf16":
        x = bf16_to_f32(bf16_bits(x))
    elif dtype != "f32":
        raise ValueError(dtype)
    return x


def random_signs(K: int, m: int, n: int, seed: int) -> np.ndarray:
    """int8 [K, m, n] of uniformly random +1 / -1."""
    rng = np.random.default_rng(seed)
    return (rng.integers(0, 2, size=(K, m, n), dtype=np.int8) * 2 - 1).astype(np.int8)


def exact_alpha(K: int, m: int, groups: int, seed: int) -> np.ndarray:
    """fp32 [K, m, groups] of 2^-e with e uniform in {4,...,8}."""
    rng = np.random.default_rng(seed)
    e = rng.integers(4, 9, size=(K, m, groups))
    return np.ldexp(np.float32(1.0), -e).astype(np.float32)


def spread_alpha(K: int, m: int, groups: int, seed: int, lo: int = 2, hi: int = 13) -> np.ndarray:
    """fp32 [K, m, groups] of 2^-e with e uniform in {lo,...,hi}: power-of-two
    scales spread over many binades (levels with up to hi - lo + 1 significant
    bits)."""
    rng = np.random.default_rng(seed)
    e = rng.integers(lo, hi + 1, size=(K, m, groups))
    return np.ldexp(np.float32(1.0), -e).astype(np.float32)


def exact_activations(T: int, n: int, seed: int) -> np.ndarray:
    """fp32 [T, n] of integers uniform in [-8, 8]."""
    rng = np.random.default_rng(seed)
    return rng.integers(-8, 9, size=(T, n)).astype(np.float32)
