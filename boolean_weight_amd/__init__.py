"""Python binding of the MBOK C ABI (include/mbok.h): argument marshalling only.

Every step of the layer runs in the HIP library libmbok.so built in this
directory; this module turns torch tensors into device pointers and sizes,
checks that the buffers are large enough and on the GPU (the C ABI receives
plain pointers and cannot check sizes), and raises MbokError on a nonzero
status.  There is no CPU fallback: without the built library every call
raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

__all__ = [
    "MBOK_F32", "MBOK_F16", "MBOK_BF16", "MBOK_GROUP", "MBOK_MAX_K", "MBOK_MAX_T",
    "MbokError", "mbok_desc", "library_path", "load_library",
    "mbok_desc_init", "mbok_packed_bytes", "mbok_alpha_bytes", "mbok_residual_binarize",
    "mbok_refit", "MBOK_MAX_REFIT_ROUNDS", "mbok_residual_energy", "mbok_allocate_kernels",
    "mbok_pack", "mbok_gemv", "mbok_gemv_workspace_bytes", "mbok_gemm", "mbok_gemm_precise",
    "mbok_status_str",
    "mbok_gemvt", "mbok_gemvt_workspace_bytes", "mbok_gemvt_noalloc", "mbok_gemvt_scratch_bytes",
    "mbok_svid_workspace_bytes", "mbok_svid_decompose", "mbok_svid_pack",
    "mbok_svid_gemv_workspace_bytes", "mbok_svid_gemv", "MBOK_MAX_SVID_ITERS",
    "mbok_version", "workspace_for",
    "alpha_torch_dtype", "quantize_and_pack", "allocate_for_budget",
]

MBOK_F32, MBOK_F16, MBOK_BF16 = 0, 1, 2
MBOK_GROUP = 128
MBOK_ROW_BLOCK = 64
MBOK_MAX_K = 4
MBOK_MAX_T = 65536
MBOK_LAYOUT_L64 = 1
MBOK_MAX_REFIT_ROUNDS = 64
MBOK_MAX_SVID_ITERS = 1000

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB = None


class MbokError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {mbok_status_str(status)} ({status})")


class mbok_desc(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("n", ctypes.c_int32), ("K", ctypes.c_int32),
                ("group", ctypes.c_int32), ("alpha_dtype", ctypes.c_int32),
                ("layout", ctypes.c_int32)]

    def __repr__(self):
        return (f"mbok_desc(m={self.m}, n={self.n}, K={self.K}, group={self.group}, "
                f"alpha_dtype={self.alpha_dtype}, layout={self.layout})")


def library_path() -> str:
    return os.environ.get("MBOK_LIBRARY", os.path.join(_HERE, "libmbok.so"))


def load_library() -> ctypes.CDLL:
    """Load libmbok.so (once).  Raises RuntimeError if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    path = library_path()
    if not os.path.exists(path):
        raise RuntimeError(f"MBOK HIP library not built: {path} is missing "
                           "(run `python -m boolean_weight_amd.build`)")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    D = ctypes.POINTER(mbok_desc)
    sigs = {
        "mbok_desc_init": (ctypes.c_int, [D, I32, I32, I32, I32]),
        "mbok_packed_bytes": (SZ, [D]),
        "mbok_alpha_bytes": (SZ, [D]),
        "mbok_residual_binarize": (ctypes.c_int, [D, P, I64, P, P, P, P]),
        "mbok_refit": (ctypes.c_int, [D, P, I64, P, P, I32, P]),
        "mbok_residual_energy": (ctypes.c_int, [D, P, I64, P, P, P]),
        "mbok_allocate_kernels": (ctypes.c_int, [I32, P, P, I32, I64, P]),
        "mbok_pack": (ctypes.c_int, [D, P, P, P, P]),
        "mbok_gemv_workspace_bytes": (SZ, [D]),
        "mbok_gemv": (ctypes.c_int, [D, P, P, I32, P, P, P]),
        "mbok_gemm": (ctypes.c_int, [D, P, P, I32, I64, I64, P, I64, P]),
        "mbok_gemm_precise": (ctypes.c_int, [D, P, P, I32, I64, I64, P, I64, P]),
        "mbok_gemvt_workspace_bytes": (SZ, [D]),
        "mbok_gemvt": (ctypes.c_int, [D, P, P, I32, P, P, P]),
        "mbok_gemvt_scratch_bytes": (SZ, []),
        "mbok_gemvt_noalloc": (ctypes.c_int, [D, P, P, I32, P, P]),
        "mbok_svid_workspace_bytes": (SZ, [D]),
        "mbok_svid_decompose": (ctypes.c_int, [D, P, I64, P, P, P, I32, P, P]),
        "mbok_svid_pack": (ctypes.c_int, [D, P, P, P, P]),
        "mbok_svid_gemv_workspace_bytes": (SZ, [D]),
        "mbok_svid_gemv": (ctypes.c_int, [D, P, P, P, I32, P, P, P]),
        "mbok_status_str": (ctypes.c_char_p, [ctypes.c_int]),
        "mbok_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


# ------------------------------------------------------------------ helpers

def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _dev(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on the GPU (the library takes device pointers)")
    return t


def _nbytes_from(t: torch.Tensor) -> int:
    """Bytes addressable from t.data_ptr() to the end of its storage."""
    st = t.untyped_storage()
    return st.nbytes() - (t.data_ptr() - st.data_ptr())


def _check(status: int, where: str):
    if status != 0:
        raise MbokError(status, where)


def alpha_torch_dtype(alpha_dtype: int) -> torch.dtype:
    return {MBOK_F32: torch.float32, MBOK_F16: torch.float16}[alpha_dtype]


def _x_dtype(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return MBOK_BF16
    if t.dtype == torch.float32:
        return MBOK_F32
    raise ValueError(f"activations must be bfloat16 or float32, got {t.dtype}")


# ---------------------------------------------------------------- the C ABI

def mbok_status_str(status: int) -> str:
    return load_library().mbok_status_str(int(status)).decode()


def mbok_version() -> str:
    return load_library().mbok_version().decode()


def mbok_desc_init(m: int, n: int, K: int, alpha_dtype: int = MBOK_F16) -> mbok_desc:
    d = mbok_desc()
    _check(load_library().mbok_desc_init(ctypes.byref(d), m, n, K, alpha_dtype), "mbok_desc_init")
    return d


def mbok_packed_bytes(d: mbok_desc) -> int:
    return int(load_library().mbok_packed_bytes(ctypes.byref(d)))


def mbok_alpha_bytes(d: mbok_desc) -> int:
    return int(load_library().mbok_alpha_bytes(ctypes.byref(d)))


def mbok_residual_binarize(d: mbok_desc, W: torch.Tensor, signs: torch.Tensor,
                           alpha: torch.Tensor, flag: torch.Tensor | None = None,
                           stream=None) -> None:
    """W fp32 [m, ldw] -> signs int8 [K, m, n] and alpha [K, m, n/128]."""
    _dev(W, "W"), _dev(signs, "signs"), _dev(alpha, "alpha")
    if W.dtype != torch.float32 or W.dim() != 2 or W.shape[0] != d.m or W.shape[1] < d.n:
        raise ValueError("W must be float32 [m, >= n]")
    if W.stride(1) != 1:
        raise ValueError("W rows must be contiguous")
    ldw = W.stride(0)
    if _nbytes_from(W) < ((d.m - 1) * ldw + d.n) * 4:
        raise ValueError("W buffer too small")
    if signs.dtype != torch.int8 or _nbytes_from(signs) < d.K * d.m * d.n:
        raise ValueError("signs must be int8 with K*m*n elements")
    if alpha.dtype != alpha_torch_dtype(d.alpha_dtype) or _nbytes_from(alpha) < mbok_alpha_bytes(d):
        raise ValueError("alpha has the wrong dtype or size")
    fptr = None
    if flag is not None:
        _dev(flag, "flag")
        if flag.dtype != torch.int32 or flag.numel() < 1:
            raise ValueError("flag must be int32 with >= 1 element")
        fptr = flag.data_ptr()
    _check(load_library().mbok_residual_binarize(
        ctypes.byref(d), W.data_ptr(), ldw, signs.data_ptr(), alpha.data_ptr(), fptr,
        _stream(stream)), "mbok_residual_binarize")


def mbok_refit(d: mbok_desc, W: torch.Tensor, signs: torch.Tensor, alpha: torch.Tensor,
               rounds: int = 2, stream=None) -> None:
    """Alternating least-squares refit of signs int8 [K, m, n] and alpha
    [K, m, n/128] (both updated in place) for W fp32 [m, ldw]."""
    _dev(W, "W"), _dev(signs, "signs"), _dev(alpha, "alpha")
    if W.dtype != torch.float32 or W.dim() != 2 or W.shape[0] != d.m or W.shape[1] < d.n:
        raise ValueError("W must be float32 [m, >= n]")
    if W.stride(1) != 1:
        raise ValueError("W rows must be contiguous")
    ldw = W.stride(0)
    if _nbytes_from(W) < ((d.m - 1) * ldw + d.n) * 4:
        raise ValueError("W buffer too small")
    if signs.dtype != torch.int8 or not signs.is_contiguous() or \
            _nbytes_from(signs) < d.K * d.m * d.n:
        raise ValueError("signs must be contiguous int8 with K*m*n elements")
    if alpha.dtype != alpha_torch_dtype(d.alpha_dtype) or not alpha.is_contiguous() \
            or _nbytes_from(alpha) < mbok_alpha_bytes(d):
        raise ValueError("alpha has the wrong dtype or size")
    _check(load_library().mbok_refit(ctypes.byref(d), W.data_ptr(), ldw, signs.data_ptr(),
                                     alpha.data_ptr(), int(rounds), _stream(stream)),
           "mbok_refit")


def mbok_residual_energy(d: mbok_desc, W: torch.Tensor, row_energy: torch.Tensor,
                         layer_energy: torch.Tensor, stream=None) -> None:
    """Residual energies of the greedy chain after 0..K kernels: row_energy
    float64 [K+1, m] and layer_energy float64 [K+1] (both overwritten)."""
    _dev(W, "W"), _dev(row_energy, "row_energy"), _dev(layer_energy, "layer_energy")
    if W.dtype != torch.float32 or W.dim() != 2 or W.shape[0] != d.m or W.shape[1] < d.n:
        raise ValueError("W must be float32 [m, >= n]")
    if W.stride(1) != 1:
        raise ValueError("W rows must be contiguous")
    ldw = W.stride(0)
    if _nbytes_from(W) < ((d.m - 1) * ldw + d.n) * 4:
        raise ValueError("W buffer too small")
    for t, cnt, nm in ((row_energy, (d.K + 1) * d.m, "row_energy"),
                       (layer_energy, d.K + 1, "layer_energy")):
        if t.dtype != torch.float64 or not t.is_contiguous() or t.numel() < cnt:
            raise ValueError(f"{nm} must be contiguous float64 with {cnt} elements")
    _check(load_library().mbok_residual_energy(ctypes.byref(d), W.data_ptr(), ldw,
                                               row_energy.data_ptr(), layer_energy.data_ptr(),
                                               _stream(stream)), "mbok_residual_energy")


def mbok_allocate_kernels(sizes, errors, budget: int) -> list:
    """Kernels per weight under a total bit budget (host only).  sizes: L
    entry counts; errors: L rows of kmax residual energies (K = 1..kmax)."""
    import numpy as np

    sz = np.ascontiguousarray(np.asarray(sizes, dtype=np.int64).reshape(-1))
    er = np.ascontiguousarray(np.asarray(errors, dtype=np.float64))
    if er.ndim != 2 or er.shape[0] != sz.shape[0]:
        raise ValueError("errors must be [L, kmax] with one row per size")
    out = np.zeros(sz.shape[0], dtype=np.int32)
    _check(load_library().mbok_allocate_kernels(
        int(sz.shape[0]), sz.ctypes.data, er.ctypes.data, int(er.shape[1]), int(budget),
        out.ctypes.data), "mbok_allocate_kernels")
    return out.tolist()


def mbok_pack(d: mbok_desc, signs: torch.Tensor, alpha: torch.Tensor, packed: torch.Tensor,
              stream=None) -> None:
    """signs int8 [K, m, n] + alpha [K, m, n/128] -> packed uint8 [mbok_packed_bytes]."""
    _dev(signs, "signs"), _dev(alpha, "alpha"), _dev(packed, "packed")
    if signs.dtype != torch.int8 or not signs.is_contiguous() or signs.numel() < d.K * d.m * d.n:
        raise ValueError("signs must be contiguous int8 with K*m*n elements")
    if alpha.dtype != alpha_torch_dtype(d.alpha_dtype) or not alpha.is_contiguous() \
            or _nbytes_from(alpha) < mbok_alpha_bytes(d):
        raise ValueError("alpha has the wrong dtype or size")
    if _nbytes_from(packed) < mbok_packed_bytes(d):
        raise ValueError("packed buffer too small")
    _check(load_library().mbok_pack(ctypes.byref(d), signs.data_ptr(), alpha.data_ptr(),
                                    packed.data_ptr(), _stream(stream)), "mbok_pack")


def mbok_gemv_workspace_bytes(d: mbok_desc) -> int:
    return int(load_library().mbok_gemv_workspace_bytes(ctypes.byref(d)))


_WORKSPACES: dict = {}


def workspace_for(nbytes: int, device=None, stream=None) -> torch.Tensor | None:
    """A workspace of at least nbytes, kept per (device, stream) so that calls
    which may overlap never share one.

    The tensor is allocated with the target stream current, so torch's caching
    allocator ties its memory to that stream: when a larger request replaces
    it, the old block is reused only in that stream's order, after the work
    already enqueued there that reads it."""
    if nbytes == 0:
        return None
    dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
    key = (dev.index, _stream(stream))
    ws = _WORKSPACES.get(key)
    if ws is None or ws.numel() < nbytes:
        if stream is None:
            target = torch.cuda.current_stream(dev)
        elif isinstance(stream, torch.cuda.Stream):
            target = stream
        else:
            target = torch.cuda.ExternalStream(int(stream), device=dev)
        with torch.cuda.stream(target):
            ws = torch.empty(max(nbytes, 1 << 20), dtype=torch.uint8, device=dev)
        _WORKSPACES[key] = ws
    return ws


def mbok_gemv(d: mbok_desc, packed: torch.Tensor, x: torch.Tensor, y: torch.Tensor,
              workspace: torch.Tensor | None | bool = True, stream=None) -> None:
    """y[m] (fp32, overwritten) = W_hat x for x bf16 / fp32 [n].

    workspace: True (default) uses a cached workspace for this device and
    stream; a tensor is used as given; None/False runs without one."""
    _dev(packed, "packed"), _dev(x, "x"), _dev(y, "y")
    if _nbytes_from(packed) < mbok_packed_bytes(d):
        raise ValueError("packed buffer too small")
    xd = _x_dtype(x)
    if x.numel() < d.n or not x.is_contiguous():
        raise ValueError("x must be contiguous with n elements")
    if y.dtype != torch.float32 or y.numel() < d.m or not y.is_contiguous():
        raise ValueError("y must be contiguous float32 with m elements")
    need = mbok_gemv_workspace_bytes(d)
    if workspace is True:
        workspace = workspace_for(need, y.device, stream)
    elif workspace is False:
        workspace = None
    wptr = None
    if workspace is not None and need > 0:
        _dev(workspace, "workspace")
        if _nbytes_from(workspace) < need:
            raise ValueError("workspace too small")
        wptr = workspace.data_ptr()
    _check(load_library().mbok_gemv(ctypes.byref(d), packed.data_ptr(), x.data_ptr(), xd,
                                    y.data_ptr(), wptr, _stream(stream)), "mbok_gemv")


def mbok_gemvt_workspace_bytes(d: mbok_desc) -> int:
    return int(load_library().mbok_gemvt_workspace_bytes(ctypes.byref(d)))


def mbok_gemvt(d: mbok_desc, packed: torch.Tensor, g: torch.Tensor, dx: torch.Tensor,
               workspace: torch.Tensor | None | bool = True, stream=None) -> None:
    """dx[n] (fp32, overwritten) = W_hat^T g for g bf16 / fp32 [m].

    workspace: True (default) uses a cached workspace for this device and
    stream; a tensor is used as given; None/False runs without one."""
    _dev(packed, "packed"), _dev(g, "g"), _dev(dx, "dx")
    if _nbytes_from(packed) < mbok_packed_bytes(d):
        raise ValueError("packed buffer too small")
    gd = _x_dtype(g)
    if g.numel() < d.m or not g.is_contiguous():
        raise ValueError("g must be contiguous with m elements")
    if dx.dtype != torch.float32 or dx.numel() < d.n or not dx.is_contiguous():
        raise ValueError("dx must be contiguous float32 with n elements")
    need = mbok_gemvt_workspace_bytes(d)
    if workspace is True:
        workspace = workspace_for(need, dx.device, stream)
    elif workspace is False:
        workspace = None
    wptr = None
    if workspace is not None and need > 0:
        _dev(workspace, "workspace")
        if _nbytes_from(workspace) < need:
            raise ValueError("workspace too small")
        wptr = workspace.data_ptr()
    _check(load_library().mbok_gemvt(ctypes.byref(d), packed.data_ptr(), g.data_ptr(), gd,
                                     dx.data_ptr(), wptr, _stream(stream)), "mbok_gemvt")


def mbok_gemvt_scratch_bytes() -> int:
    return int(load_library().mbok_gemvt_scratch_bytes())


def mbok_gemvt_noalloc(d: mbok_desc, packed: torch.Tensor, g: torch.Tensor, dx: torch.Tensor,
                       stream=None) -> None:
    """mbok_gemvt with the library's static scratch instead of a workspace
    (for callers that cannot allocate device memory).  Calls that overlap in
    time on one GPU share that scratch and race."""
    _dev(packed, "packed"), _dev(g, "g"), _dev(dx, "dx")
    if _nbytes_from(packed) < mbok_packed_bytes(d):
        raise ValueError("packed buffer too small")
    gd = _x_dtype(g)
    if g.numel() < d.m or not g.is_contiguous():
        raise ValueError("g must be contiguous with m elements")
    if dx.dtype != torch.float32 or dx.numel() < d.n or not dx.is_contiguous():
        raise ValueError("dx must be contiguous float32 with n elements")
    _check(load_library().mbok_gemvt_noalloc(ctypes.byref(d), packed.data_ptr(), g.data_ptr(),
                                             gd, dx.data_ptr(), _stream(stream)),
           "mbok_gemvt_noalloc")


def mbok_svid_workspace_bytes(d: mbok_desc) -> int:
    return int(load_library().mbok_svid_workspace_bytes(ctypes.byref(d)))


def mbok_svid_gemv_workspace_bytes(d: mbok_desc) -> int:
    return int(load_library().mbok_svid_gemv_workspace_bytes(ctypes.byref(d)))


def mbok_svid_decompose(d: mbok_desc, W: torch.Tensor, signs: torch.Tensor, s_out: torch.Tensor,
                        s_in: torch.Tensor, iters: int = 32, workspace: torch.Tensor | None = None,
                        stream=None) -> None:
    """Successive SVID of W fp32 [m, ldw] into signs int8 [K, m, n], s_out
    [K, m] and s_in [K, n] (scale dtype).  A workspace is allocated when none
    is given."""
    _dev(W, "W"), _dev(signs, "signs"), _dev(s_out, "s_out"), _dev(s_in, "s_in")
    if W.dtype != torch.float32 or W.dim() != 2 or W.shape[0] != d.m or W.shape[1] < d.n:
        raise ValueError("W must be float32 [m, >= n]")
    if W.stride(1) != 1:
        raise ValueError("W rows must be contiguous")
    ldw = W.stride(0)
    if _nbytes_from(W) < ((d.m - 1) * ldw + d.n) * 4:
        raise ValueError("W buffer too small")
    at = alpha_torch_dtype(d.alpha_dtype)
    if signs.dtype != torch.int8 or not signs.is_contiguous() or signs.numel() < d.K * d.m * d.n:
        raise ValueError("signs must be contiguous int8 with K*m*n elements")
    for t, cnt, nm in ((s_out, d.K * d.m, "s_out"), (s_in, d.K * d.n, "s_in")):
        if t.dtype != at or not t.is_contiguous() or t.numel() < cnt:
            raise ValueError(f"{nm} must be contiguous {at} with {cnt} elements")
    need = mbok_svid_workspace_bytes(d)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=W.device)
    _dev(workspace, "workspace")
    if _nbytes_from(workspace) < need:
        raise ValueError("workspace too small")
    _check(load_library().mbok_svid_decompose(
        ctypes.byref(d), W.data_ptr(), ldw, signs.data_ptr(), s_out.data_ptr(), s_in.data_ptr(),
        int(iters), workspace.data_ptr(), _stream(stream)), "mbok_svid_decompose")


def mbok_svid_pack(d: mbok_desc, signs: torch.Tensor, s_out: torch.Tensor, packed: torch.Tensor,
                   stream=None) -> None:
    """signs int8 [K, m, n] + s_out [K, m] -> packed uint8 [mbok_packed_bytes]."""
    _dev(signs, "signs"), _dev(s_out, "s_out"), _dev(packed, "packed")
    if signs.dtype != torch.int8 or not signs.is_contiguous() or signs.numel() < d.K * d.m * d.n:
        raise ValueError("signs must be contiguous int8 with K*m*n elements")
    if s_out.dtype != alpha_torch_dtype(d.alpha_dtype) or not s_out.is_contiguous() or \
            s_out.numel() < d.K * d.m:
        raise ValueError("s_out has the wrong dtype or size")
    if _nbytes_from(packed) < mbok_packed_bytes(d):
        raise ValueError("packed buffer too small")
    _check(load_library().mbok_svid_pack(ctypes.byref(d), signs.data_ptr(), s_out.data_ptr(),
                                         packed.data_ptr(), _stream(stream)), "mbok_svid_pack")


def mbok_svid_gemv(d: mbok_desc, packed: torch.Tensor, s_in: torch.Tensor, x: torch.Tensor,
                   y: torch.Tensor, stream=None) -> None:
    """y[m] (fp32, overwritten) = sum_k s_out^k (.) (B_k (s_in^k (.) x)) for x bf16 / fp32 [n]."""
    _dev(packed, "packed"), _dev(s_in, "s_in"), _dev(x, "x"), _dev(y, "y")
    if _nbytes_from(packed) < mbok_packed_bytes(d):
        raise ValueError("packed buffer too small")
    if s_in.dtype != alpha_torch_dtype(d.alpha_dtype) or not s_in.is_contiguous() or \
            s_in.numel() < d.K * d.n:
        raise ValueError("s_in has the wrong dtype or size")
    xd = _x_dtype(x)
    if x.numel() < d.n or not x.is_contiguous():
        raise ValueError("x must be contiguous with n elements")
    if y.dtype != torch.float32 or y.numel() < d.m or not y.is_contiguous():
        raise ValueError("y must be contiguous float32 with m elements")
    _check(load_library().mbok_svid_gemv(ctypes.byref(d), packed.data_ptr(), s_in.data_ptr(),
                                         x.data_ptr(), xd, y.data_ptr(), None, _stream(stream)),
           "mbok_svid_gemv")


def mbok_gemm(d: mbok_desc, packed: torch.Tensor, X: torch.Tensor, Y: torch.Tensor,
              stream=None) -> None:
    """Y[T, m] (fp32, overwritten) = X W_hat^T for X bf16 [T, n] (row stride ldx)."""
    _gemm_call("mbok_gemm", d, packed, X, Y, stream)


def mbok_gemm_precise(d: mbok_desc, packed: torch.Tensor, X: torch.Tensor, Y: torch.Tensor,
                      stream=None) -> None:
    """mbok_gemm with each prefill weight carried as two bf16 terms (hi + lo)."""
    _gemm_call("mbok_gemm_precise", d, packed, X, Y, stream)


def _gemm_call(name: str, d: mbok_desc, packed: torch.Tensor, X: torch.Tensor, Y: torch.Tensor,
               stream) -> None:
    _dev(packed, "packed"), _dev(X, "X"), _dev(Y, "Y")
    if _nbytes_from(packed) < mbok_packed_bytes(d):
        raise ValueError("packed buffer too small")
    xd = _x_dtype(X)
    if X.dim() != 2 or X.shape[1] < d.n or X.stride(1) != 1:
        raise ValueError("X must be 2-D [T, >= n] with contiguous rows")
    if Y.dtype != torch.float32 or Y.dim() != 2 or Y.shape[0] != X.shape[0] or \
            Y.shape[1] < d.m or Y.stride(1) != 1:
        raise ValueError("Y must be float32 [T, >= m] with contiguous rows")
    T = X.shape[0]
    ldx, ldy = X.stride(0), Y.stride(0)
    if T > 0:
        if _nbytes_from(X) < ((T - 1) * ldx + d.n) * X.element_size():
            raise ValueError("X buffer too small")
        if _nbytes_from(Y) < ((T - 1) * ldy + d.m) * 4:
            raise ValueError("Y buffer too small")
    fn = getattr(load_library(), name)
    _check(fn(ctypes.byref(d), packed.data_ptr(), X.data_ptr(), xd, T, ldx, Y.data_ptr(), ldy,
              _stream(stream)), name)


# ---------------------------------------------------------------- conveniences

def quantize_and_pack(W: torch.Tensor, K: int, alpha_dtype: int = MBOK_F16, stream=None):
    """Greedy residual binarization of a device fp32 W, then packing.

    Returns (desc, packed, signs, alpha); every step runs in the library."""
    m, n = W.shape
    d = mbok_desc_init(m, n, K, alpha_dtype)
    signs = torch.empty((K, m, n), dtype=torch.int8, device=W.device)
    alpha = torch.empty((K, m, n // MBOK_GROUP), dtype=alpha_torch_dtype(alpha_dtype),
                        device=W.device)
    flag = torch.zeros(1, dtype=torch.int32, device=W.device)
    mbok_residual_binarize(d, W, signs, alpha, flag, stream)
    packed = torch.empty(mbok_packed_bytes(d), dtype=torch.uint8, device=W.device)
    mbok_pack(d, signs, alpha, packed, stream)
    if int(flag.item()) != 0:
        raise ValueError("W holds NaN or Inf")
    return d, packed, signs, alpha


def allocate_for_budget(weights, avg_kernels: float, kmax: int = MBOK_MAX_K,
                        alpha_dtype: int = MBOK_F16, stream=None):
    """Kernels per weight for a set of device fp32 weights under an average
    budget of `avg_kernels` kernels per entry: the residual energies of each
    weight's greedy chain (mbok_residual_energy, K = 1..kmax) feed
    mbok_allocate_kernels with budget floor(avg_kernels * total entries).
    Returns (K list, layer energies [L][kmax + 1] as nested lists)."""
    errors, sizes, energies = [], [], []
    for W in weights:
        m, n = W.shape
        d = mbok_desc_init(m, n, kmax, alpha_dtype)
        rows = torch.empty((kmax + 1, m), dtype=torch.float64, device=W.device)
        layer = torch.empty(kmax + 1, dtype=torch.float64, device=W.device)
        mbok_residual_energy(d, W, rows, layer, stream)
        e = layer.cpu().tolist()
        energies.append(e)
        errors.append(e[1:])
        sizes.append(m * n)
    budget = int(avg_kernels * sum(sizes))
    return mbok_allocate_kernels(sizes, errors, budget), energies
