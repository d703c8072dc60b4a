"""The part's own ceilings (libmbok_ceilings.so), for measurement only.

Each function times one microbenchmark kernel as a HIP graph of back-to-back
launches with HIP events on the launching stream:
  launch_floor_us(grid, block)      -- interval of an empty kernel
  read_bandwidth(bytes, ...)        -- GB/s of a 16-byte-load read stream over
                                       a rotating pool of at least 1 GiB
  mfma_rate(kind)                   -- TFLOP/s of independent matrix-core
                                       products (bf16, or fp4 x fp8 scaled)
None of this is on the product path; bench.py reports the MBOK kernels
against these figures beside the nameplate ones.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None

MFMA_BF16, MFMA_F4F8, MFMA_F4F8_LANE_SCALES = 0, 1, 2
# flops of one product of each kind (2 per multiply-add)
_MFMA_FLOPS = {MFMA_BF16: 2 * 32 * 32 * 16, MFMA_F4F8: 2 * 16 * 16 * 128,
               MFMA_F4F8_LANE_SCALES: 2 * 16 * 16 * 128}


def load():
    global _LIB
    if _LIB is not None:
        return _LIB
    path = os.path.join(_HERE, "libmbok_ceilings.so")
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: run __graft_entry__.build() first")
    lib = ctypes.CDLL(path)
    V, I, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.mbok_ceiling_empty.argtypes = [I, I, V]
    lib.mbok_ceiling_marker.argtypes = [V]
    lib.mbok_ceiling_spin.argtypes = [I, V, V]
    lib.mbok_ceiling_spin.restype = I
    lib.mbok_ceiling_read.argtypes = [V, SZ, V, I, I, V]
    lib.mbok_ceiling_mfma.argtypes = [I, V, I, I, I, V]
    for f in (lib.mbok_ceiling_empty, lib.mbok_ceiling_marker, lib.mbok_ceiling_read,
              lib.mbok_ceiling_mfma):
        f.restype = I
    _LIB = lib
    return lib


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _check(rc: int, what: str):
    if rc != 0:
        raise RuntimeError(f"{what} failed ({rc})")


def _graph_us(fn, calls: int, reps: int = 5) -> float:
    """Mean microseconds per call of fn(i), i = 0..calls-1, captured in one
    HIP graph and replayed reps times (the first replay untimed)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn(0)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(calls):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / (reps * calls)


def launch_floor_us(grid: int = 256, block: int = 512, calls: int = 400) -> float:
    lib = load()
    return _graph_us(lambda i: _check(lib.mbok_ceiling_empty(grid, block, _stream()), "empty"),
                     calls)


def read_bandwidth(nbytes: int, pool_bytes: int = 1 << 30, grid: int = 1024,
                   block: int = 1024) -> dict:
    """Read-stream rate over copies of an nbytes buffer cycled through a pool
    of at least pool_bytes (so each read comes from HBM, not the 256 MB
    Infinity Cache).  Returns us per call and GB/s."""
    lib = load()
    nbytes = (nbytes + 15) // 16 * 16
    ncopy = max(2, -(-pool_bytes // nbytes))
    pool = torch.empty((ncopy, nbytes), dtype=torch.uint8, device="cuda")
    pool.fill_(1)
    out = torch.empty(grid, dtype=torch.float32, device="cuda")
    us = _graph_us(lambda i: _check(lib.mbok_ceiling_read(pool[i].data_ptr(), nbytes,
                                                          out.data_ptr(), grid, block,
                                                          _stream()), "read"), ncopy)
    del pool
    return {"bytes": nbytes, "us": us, "GB/s": nbytes / (us * 1e-6) / 1e9,
            "grid": grid, "block": block, "pool_copies": ncopy}


def mfma_rate(kind: int = MFMA_BF16, iters: int = 4000, grid: int = 1024,
              block: int = 256) -> dict:
    """TFLOP/s of independent products of `kind`: four chains per wavefront,
    grid x block threads."""
    lib = load()
    out = torch.empty(grid, dtype=torch.float32, device="cuda")
    us = _graph_us(lambda i: _check(lib.mbok_ceiling_mfma(kind, out.data_ptr(), iters, grid,
                                                          block, _stream()), "mfma"), 4, reps=3)
    products = grid * (block // 64) * iters * 4
    return {"kind": kind, "us": us, "TFLOP/s": products * _MFMA_FLOPS[kind] / (us * 1e-6) / 1e12,
            "grid": grid, "block": block}
