"""W8A8 FP8 linear layer for AMD MI355X (gfx950) — Python binding.

Thin ``ctypes`` wrapper over ``libw8a8.so`` (C ABI in ``include/w8a8.h``).
torch provides device memory and the current HIP stream; every step of the
computation runs in the library's HIP kernels. There is no fallback: if the
library is missing or the device is not gfx950 the calls raise.

The layer is the FP8 "fast-math" linear layer of the Metis-1.6 pages: a
token's BF16 row is quantised to E4M3 with one scale per token and multiplied
with E4M3 weights carrying one scale per output row (Lernex/Metis-1.6-Logos-
FP8, "What --fast-math does" and "What is in FP8").
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "W8A8Error", "lib", "lib_path", "abi_version",
    "quantize_per_token", "w8a8_gemm", "w8a8_linear", "quantize_weight",
]

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_NAME = "libw8a8.so"
_lib = None

_c_i64 = ctypes.c_int64
_c_ptr = ctypes.c_void_p

# name -> (restype, argtypes); mirrors include/w8a8.h
_SIGNATURES = {
    "w8a8_abi_version": (ctypes.c_int, []),
    "w8a8_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "quantize_per_token": (ctypes.c_int, [_c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr]),
    "w8a8_gemm": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, _c_ptr]),
}


class W8A8Error(RuntimeError):
    """A non-zero status from libw8a8.so."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status} ({status_string(status)})")


def lib_path() -> str:
    return os.path.join(_HERE, _LIB_NAME)


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() "
                               "or python -m w8a8_fp8_linear_amd.build")
        handle = ctypes.CDLL(path)
        for name, (res, args) in _SIGNATURES.items():
            f = getattr(handle, name)
            f.restype = res
            f.argtypes = args
        _lib = handle
    return _lib


def abi_version() -> int:
    return lib().w8a8_abi_version()


def status_string(status: int) -> str:
    try:
        return lib().w8a8_status_string(status).decode()
    except Exception:  # pragma: no cover - library not loadable
        return "unknown"


def _check(fn: str, status: int) -> None:
    if status != 0:
        raise W8A8Error(fn, status)


def _stream(t) -> int:
    import torch

    return torch.cuda.current_stream(t.device).cuda_stream


def _want(t, dtype, ndim, name):
    import torch

    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {t.dim()}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be on a GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def quantize_per_token(x, q=None, scale=None):
    """BF16 [M, K] -> (E4M3 codes uint8 [M, K], float32 scales [M]).

    One scale per row: s = fl32(amax / 448); q = E4M3(fl32(x / s)), round to
    nearest even, saturating at 448. Used for activations (per token) and for
    weights (per output row).
    """
    import torch

    _want(x, torch.bfloat16, 2, "x")
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((M,), dtype=torch.float32, device=x.device)
    _want(q, torch.uint8, 2, "q")
    _want(scale, torch.float32, 1, "scale")
    if tuple(q.shape) != (M, K) or tuple(scale.shape) != (M,):
        raise ValueError("output shapes do not match x")
    _check("quantize_per_token",
           lib().quantize_per_token(x.data_ptr(), M, K, q.data_ptr(), scale.data_ptr(), _stream(x)))
    return q, scale


def w8a8_gemm(a_q, a_scale, w_q, w_scale, out=None):
    """y[m, n] = bf16(a_scale[m] * w_scale[n] * sum_k a_q[m, k] * w_q[n, k]) (E4M3 operands)."""
    import torch

    _want(a_q, torch.uint8, 2, "a_q")
    _want(w_q, torch.uint8, 2, "w_q")
    _want(a_scale, torch.float32, 1, "a_scale")
    _want(w_scale, torch.float32, 1, "w_scale")
    M, K = a_q.shape
    N, K2 = w_q.shape
    if K2 != K or a_scale.shape[0] != M or w_scale.shape[0] != N:
        raise ValueError("shape mismatch between a, w and their scales")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device)
    _want(out, torch.bfloat16, 2, "out")
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    _check("w8a8_gemm", lib().w8a8_gemm(a_q.data_ptr(), a_scale.data_ptr(), w_q.data_ptr(), w_scale.data_ptr(),
                                        out.data_ptr(), M, N, K, _stream(a_q)))
    return out


def quantize_weight(w):
    """BF16 weight [out, in] -> (E4M3 [out, in], float32 [out]); the same per-row map."""
    return quantize_per_token(w)


def w8a8_linear(x, w_q, w_scale, out=None):
    """The layer: quantise the BF16 input per token, then the scaled FP8 GEMM."""
    q, s = quantize_per_token(x)
    return w8a8_gemm(q, s, w_q, w_scale, out=out)
