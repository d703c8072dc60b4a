"""Helpers for the GPU parity tests: device transfers and run-once checks.

Expected values always come from the oracle on inputs drawn by mbok_synth;
nothing produced by the HIP path is ever fed to the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import boolean_weight_amd as bw
import mbok_synth as syn

DEV = "cuda:0"


def say(msg: str):
    """Name the case before a GPU step (flushed, so a lost box still shows it)."""
    print(msg, flush=True)
    sys.stdout.flush()


def alpha_enum(dt: str) -> int:
    return bw.MBOK_F16 if dt == "f16" else bw.MBOK_F32


def np_alpha(dt: str):
    return np.float16 if dt == "f16" else np.float32


def to_dev(a: np.ndarray, dtype=None) -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def x_to_dev(x: np.ndarray, x_dtype: str) -> torch.Tensor:
    """x values (already representable in x_dtype) to a device tensor."""
    if x_dtype == "bf16":
        bits = syn.bf16_bits(x)
        return torch.from_numpy(bits.view(np.int16)).to(DEV).view(torch.bfloat16)
    return to_dev(x.astype(np.float32))


def pack_on_gpu(S: np.ndarray, A: np.ndarray, dt: str):
    K, m, n = S.shape
    d = bw.mbok_desc_init(m, n, K, alpha_enum(dt))
    packed = torch.empty(bw.mbok_packed_bytes(d), dtype=torch.uint8, device=DEV)
    bw.mbok_pack(d, to_dev(S), to_dev(A.astype(np_alpha(dt))), packed)
    return d, packed


def gemv(d, packed, x: np.ndarray, x_dtype: str, guard: int = 0) -> np.ndarray:
    """Run mbok_gemv; with guard > 0, y sits between canary words that must
    survive the call unchanged."""
    xt = x_to_dev(x.reshape(-1), x_dtype)
    canary = -12345.5
    yb = torch.full((d.m + 2 * guard,), canary, dtype=torch.float32, device=DEV)
    y = yb[guard:guard + d.m]
    bw.mbok_gemv(d, packed, xt, y)
    out = yb.cpu().numpy()
    if guard:
        assert np.all(out[:guard] == canary) and np.all(out[guard + d.m:] == canary), \
            "mbok_gemv wrote outside y"
    return out[guard:guard + d.m].astype(np.float64)


def gemm(d, packed, X: np.ndarray, ldx: int | None = None, ldy: int | None = None) -> np.ndarray:
    T, n = X.shape
    ldx = ldx or n
    ldy = ldy or d.m
    Xp = np.zeros((T, ldx), dtype=np.float32)
    Xp[:, :n] = X
    Xt = x_to_dev(Xp, "bf16").view(T, ldx)
    canary = -777.25
    Yb = torch.full((T, ldy), canary, dtype=torch.float32, device=DEV)
    bw.mbok_gemm(d, packed, Xt[:, :ldx], Yb)
    out = Yb.cpu().numpy()
    if ldy > d.m:
        assert np.all(out[:, d.m:] == canary), "mbok_gemm wrote into the row padding of Y"
    return out[:, :d.m].astype(np.float64)
