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
    "W8A8Error", "lib", "lib_path", "abi_version", "e4m3_from_f32", "bf16_from_f32",
    "quantize_per_token", "w8a8_gemm", "w8a8_linear", "quantize_weight",
    "moe_route", "moe_gate_up_bf16", "moe_gate_up_swiglu_quant", "moe_down_combine",
    "w8a8_grouped_gemm", "moe_w8a8_grouped", "moe_workspace", "moe_ffn",
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
    "w8a8_gemm_timed": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, _c_ptr,
                                       _c_ptr, _c_ptr]),
    "w8a16_gemm": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, _c_ptr]),
    "fp8_linear_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64]),
    "fp8_linear_single_launch": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, _c_ptr]),
    "fp8_linear": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, ctypes.c_int, _c_ptr,
                                  ctypes.c_size_t, _c_ptr]),
    "fp8_linear_noalloc_max_bytes": (ctypes.c_size_t, []),
    "fp8_linear_noalloc": (ctypes.c_int, [_c_ptr, _c_ptr, _c_ptr, _c_ptr, _c_i64, _c_i64, _c_i64, ctypes.c_int,
                                          _c_ptr]),
    "moe_route_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64, ctypes.c_int]),
    "moe_route": (ctypes.c_int, [_c_ptr, _c_i64, _c_i64, _c_i64, ctypes.c_int, _c_ptr, _c_ptr, _c_ptr, _c_ptr,
                                 _c_ptr, ctypes.c_size_t, _c_ptr]),
    "moe_gate_up_bf16": (ctypes.c_int, [_c_ptr] * 7 + [_c_i64] * 5 + [ctypes.c_int, _c_ptr]),
    "moe_gate_up_swiglu_quant_workspace_bytes": (ctypes.c_size_t, [_c_i64] * 3),
    "moe_gate_up_swiglu_quant": (ctypes.c_int, [_c_ptr] * 10 + [_c_i64] * 5 + [ctypes.c_int, _c_ptr, ctypes.c_size_t,
                                                                           _c_ptr]),
    "e4m3_from_f32": (ctypes.c_int, [_c_ptr, _c_i64, _c_ptr, _c_ptr]),
    "read_probe_sink_words": (ctypes.c_int64, [_c_i64]),
    "read_probe": (ctypes.c_int, [_c_ptr, _c_i64, _c_ptr, _c_ptr]),
    "clock_probe": (ctypes.c_int, [_c_ptr, _c_i64, _c_ptr]),
    "bf16_from_f32": (ctypes.c_int, [_c_ptr, _c_i64, _c_ptr, _c_ptr]),
    "moe_down_combine": (ctypes.c_int, [_c_ptr] * 10 + [_c_i64] * 5 + [ctypes.c_int, _c_ptr]),
    "w8a8_grouped_gemm_workspace_bytes": (ctypes.c_size_t, [_c_i64, _c_i64, _c_i64]),
    "w8a8_grouped_gemm": (ctypes.c_int, [_c_ptr] * 8 + [_c_i64] * 5 + [_c_ptr, ctypes.c_size_t, _c_ptr]),
    "moe_w8a8_workspace_bytes": (ctypes.c_size_t, [_c_i64] * 5),
    "moe_w8a8_grouped": (ctypes.c_int, [_c_ptr] * 11 + [_c_i64] * 5 + [_c_ptr, ctypes.c_size_t, _c_ptr]),
    "mxfp4_quantize": (ctypes.c_int, [_c_ptr, _c_i64, _c_i64, _c_ptr, _c_ptr, _c_ptr]),
    "moe_mxfp4_gate_up_bf16": (ctypes.c_int, [_c_ptr] * 7 + [_c_i64] * 5 + [ctypes.c_int, _c_ptr]),
    "moe_mxfp4_gate_up_swiglu_quant": (ctypes.c_int, [_c_ptr] * 9 + [_c_i64] * 5 + [ctypes.c_int, _c_ptr]),
    "moe_mxfp4_down_combine": (ctypes.c_int, [_c_ptr] * 12 + [_c_i64] * 5 + [ctypes.c_int, _c_ptr]),
    "moe_mxfp4_workspace_bytes": (ctypes.c_size_t, [_c_i64] * 5),
    "moe_mxfp4_grouped": (ctypes.c_int, [_c_ptr] * 11 + [_c_i64] * 5 + [_c_ptr, ctypes.c_size_t, _c_ptr]),
}


class W8A8Error(RuntimeError):
    """A non-zero status from libw8a8.so."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: status {status} ({status_string(status)})")


def lib_path() -> str:
    """The in-tree build, or the library named by ``W8A8_LIB`` (for example a
    host-sanitized build)."""
    return os.environ.get("W8A8_LIB") or os.path.join(_HERE, _LIB_NAME)


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises if it is not built)."""
    global _lib
    if _lib is None:
        path = lib_path()
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build() "
                               "or python -m w8a8_fp8_linear_amd.build")
        # torch first: the library then binds to the HIP runtime torch has
        # loaded (the one its tensors and streams belong to) rather than
        # bringing in a second copy of the runtime
        import torch  # noqa: F401

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


def w8a8_gemm(a_q, a_scale, w_q, w_scale, out=None, events=None):
    """y[m, n] = bf16(a_scale[m] * w_scale[n] * sum_k a_q[m, k] * w_q[n, k]) (E4M3 operands).

    events: optional (start, stop) pair of timing torch.cuda.Event; the
    kernel is then launched through w8a8_gemm_timed, which stamps them with
    its own start and end (start.elapsed_time(stop) is the kernel alone)."""
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
    if events is None:
        _check("w8a8_gemm", lib().w8a8_gemm(a_q.data_ptr(), a_scale.data_ptr(), w_q.data_ptr(),
                                            w_scale.data_ptr(), out.data_ptr(), M, N, K, _stream(a_q)))
        return out
    start, stop = events
    stream = torch.cuda.current_stream(a_q.device)
    for ev in (start, stop):
        if not isinstance(ev, torch.cuda.Event):
            raise TypeError("events must be torch.cuda.Event objects")
        if not ev.cuda_event:  # torch creates the HIP event on its first record
            ev.record(stream)
    _check("w8a8_gemm_timed", lib().w8a8_gemm_timed(a_q.data_ptr(), a_scale.data_ptr(), w_q.data_ptr(),
                                                    w_scale.data_ptr(), out.data_ptr(), M, N, K, stream.cuda_stream,
                                                    start.cuda_event, stop.cuda_event))
    return out


def w8a16_gemm(x, w_q, w_scale, out=None):
    """Default maths: y[m, n] = bf16(w_scale[n] * sum_k x[m, k] * dec(w_q[n, k])), x BF16 (not quantised)."""
    import torch

    _want(x, torch.bfloat16, 2, "x")
    _want(w_q, torch.uint8, 2, "w_q")
    _want(w_scale, torch.float32, 1, "w_scale")
    M, K = x.shape
    N, K2 = w_q.shape
    if K2 != K or w_scale.shape[0] != N:
        raise ValueError("shape mismatch between x, w_q and w_scale")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _want(out, torch.bfloat16, 2, "out")
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    _check("w8a16_gemm", lib().w8a16_gemm(x.data_ptr(), w_q.data_ptr(), w_scale.data_ptr(), out.data_ptr(), M, N, K,
                                          _stream(x)))
    return out


def fp8_linear(x, w_q, w_scale, fast_math=True, out=None, workspace=None):
    """The layer as the model page's runtime picks it: FP8 multiply (per-token
    quantisation + w8a8_gemm) when ``fast_math`` and more than 8 tokens,
    otherwise the default maths (w8a16_gemm)."""
    import torch

    _want(x, torch.bfloat16, 2, "x")
    _want(w_q, torch.uint8, 2, "w_q")
    _want(w_scale, torch.float32, 1, "w_scale")
    M, K = x.shape
    N, K2 = w_q.shape
    if K2 != K or w_scale.shape[0] != N:
        raise ValueError("shape mismatch between x, w_q and w_scale")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _want(out, torch.bfloat16, 2, "out")
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    nbytes = int(lib().fp8_linear_workspace_bytes(M, K))
    if workspace is None and fast_math and M > 8:
        workspace = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=x.device)
    wptr = workspace.data_ptr() if workspace is not None else None
    wlen = workspace.numel() if workspace is not None else 0
    _check("fp8_linear", lib().fp8_linear(x.data_ptr(), w_q.data_ptr(), w_scale.data_ptr(), out.data_ptr(), M, N, K,
                                          1 if fast_math else 0, wptr, wlen, _stream(x)))
    return out


def fp8_linear_noalloc(x, w_q, w_scale, fast_math=True, out=None):
    """fp8_linear with the quantised input in the library's static device
    scratch instead of a workspace: the library allocates nothing. ``out`` is
    allocated here when not given (pass it to allocate nothing at all). Calls
    that overlap on one GPU share the scratch and race."""
    import torch

    _want(x, torch.bfloat16, 2, "x")
    _want(w_q, torch.uint8, 2, "w_q")
    _want(w_scale, torch.float32, 1, "w_scale")
    M, K = x.shape
    N, K2 = w_q.shape
    if K2 != K or w_scale.shape[0] != N:
        raise ValueError("shape mismatch between x, w_q and w_scale")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _want(out, torch.bfloat16, 2, "out")
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    _check("fp8_linear_noalloc", lib().fp8_linear_noalloc(x.data_ptr(), w_q.data_ptr(), w_scale.data_ptr(),
                                                          out.data_ptr(), M, N, K, 1 if fast_math else 0,
                                                          _stream(x)))
    return out


def fp8_linear_single_launch(x, w_q, w_scale, out=None):
    """The FP8 multiply (per-token quantisation + scaled FP8 GEMM) in one launch, M <= 32, K <= 2048;
    bit-identical to quantize_per_token + w8a8_gemm."""
    import torch

    _want(x, torch.bfloat16, 2, "x")
    _want(w_q, torch.uint8, 2, "w_q")
    _want(w_scale, torch.float32, 1, "w_scale")
    M, K = x.shape
    N, K2 = w_q.shape
    if K2 != K or w_scale.shape[0] != N:
        raise ValueError("shape mismatch between x, w_q and w_scale")
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=x.device)
    _want(out, torch.bfloat16, 2, "out")
    if tuple(out.shape) != (M, N):
        raise ValueError("out must be [M, N]")
    _check("fp8_linear_single_launch", lib().fp8_linear_single_launch(
        x.data_ptr(), w_q.data_ptr(), w_scale.data_ptr(), out.data_ptr(), M, N, K, _stream(x)))
    return out


def e4m3_from_f32(v):
    """E4M3 codes (uint8, same shape) of float32 values clamped to +-448: the
    encoding step every quantiser here ends with, run on the device."""
    import torch

    if not isinstance(v, torch.Tensor) or v.dtype != torch.float32 or not v.is_cuda or not v.is_contiguous():
        raise TypeError("v must be a contiguous float32 tensor on a GPU")
    q = torch.empty(v.shape, dtype=torch.uint8, device=v.device)
    _check("e4m3_from_f32", lib().e4m3_from_f32(v.data_ptr(), v.numel(), q.data_ptr(), _stream(v)))
    return q


def bf16_from_f32(v):
    """BF16 (round to nearest even) of float32 values: the rounding every BF16
    result here ends with, run on the device."""
    import torch

    if not isinstance(v, torch.Tensor) or v.dtype != torch.float32 or not v.is_cuda or not v.is_contiguous():
        raise TypeError("v must be a contiguous float32 tensor on a GPU")
    y = torch.empty(v.shape, dtype=torch.bfloat16, device=v.device)
    _check("bf16_from_f32", lib().bf16_from_f32(v.data_ptr(), v.numel(), y.data_ptr(), _stream(v)))
    return y


def clock_probe(n=256, out=None, device="cuda"):
    """Enqueue the shader-clock probe (n one-wave workgroups) on the current
    stream. Returns out, int64 [n, 2]: shader cycles and 100 MHz ticks per
    workgroup over the same span (about 4 us)."""
    import torch

    if out is None:
        out = torch.empty((n, 2), dtype=torch.int64, device=device)
    if out.dtype != torch.int64 or not out.is_cuda or not out.is_contiguous() or out.numel() < 2 * n:
        raise ValueError("out must be a contiguous int64 GPU tensor with at least 2 * n entries")
    _check("clock_probe", lib().clock_probe(out.data_ptr(), n, _stream(out)))
    return out


def clock_ghz(out):
    """Median shader clock in GHz over the workgroups of a clock_probe result
    (a CPU or GPU int64 [n, 2] tensor)."""
    import torch

    v = out.detach().to("cpu", torch.float64).view(-1, 2)
    return float(torch.median(0.1 * v[:, 0] / v[:, 1]))


def read_probe(t, sink=None):
    """Read every byte of the contiguous device tensor t in the decode GEMM's
    launch shape, doing nothing else (the weight stream's read floor). Returns
    the sink: one uint32 XOR word per 32 KB block."""
    import torch

    if not isinstance(t, torch.Tensor) or not t.is_cuda or not t.is_contiguous():
        raise TypeError("t must be a contiguous tensor on a GPU")
    nbytes = t.numel() * t.element_size()
    words = int(lib().read_probe_sink_words(nbytes))
    if sink is None:
        sink = torch.empty(max(words, 4), dtype=torch.int32, device=t.device)
    if sink.numel() < words or sink.dtype != torch.int32:
        raise ValueError("sink must be int32 with at least read_probe_sink_words(bytes) entries")
    _check("read_probe", lib().read_probe(t.data_ptr(), nbytes, sink.data_ptr(), _stream(t)))
    return sink


def quantize_weight(w):
    """BF16 weight [out, in] -> (E4M3 [out, in], float32 [out]); the same per-row map."""
    return quantize_per_token(w)


def w8a8_linear(x, w_q, w_scale, out=None):
    """The layer: quantise the BF16 input per token, then the scaled FP8 GEMM."""
    q, s = quantize_per_token(x)
    return w8a8_gemm(q, s, w_q, w_scale, out=out)


# ---- routed experts -----------------------------------------------------------
#
# Shapes: x_q [T, H] uint8 (E4M3), x_scale [T] f32, topk_ids [T, k] int32,
# topk_w [T, k] f32, w13_q [E, 2I, H] uint8 ([gate; up] rows), w13_scale
# [E, 2I] f32, w2_q [E, H, I] uint8, w2_scale [E, H] f32. Slots are t*k + j;
# "sorted" arrays list the valid slots grouped by expert (stable).


def _check_order(offsets, E: int, topk: int, order: int) -> None:
    """The grouped kernels walk offsets on the device; its length must match the order."""
    want = (topk * E if order else E) + 1
    if order not in (0, 1):
        raise ValueError("order must be 0 (expert-major) or 1 (slot-position-major)")
    if offsets.numel() != want:
        raise ValueError(f"offsets has {offsets.numel()} entries; order {order} with E={E}, topk={topk} "
                         f"needs {want} (route with moe_route(..., order={order}))")


def _moe_dims(x_q, topk_ids, w13_q):
    T, H = x_q.shape
    E, twoI, H2 = w13_q.shape
    if H2 != H or twoI % 2:
        raise ValueError("w13_q must be [E, 2I, H]")
    if topk_ids.shape[0] != T:
        raise ValueError("topk_ids must be [T, k]")
    return T, H, twoI // 2, E, topk_ids.shape[1]


def moe_route(topk_ids, E: int, order: int = 0, with_slot_row: bool = False):
    """Sorted order of the routed slots: (counts [G], offsets [G+1], perm [T*k]) int32,
    plus slot_row [T*k] (slot -> sorted row, -1 if dropped) when ``with_slot_row``.

    order 0: G = E groups by expert; order 1: G = k * E groups keyed
    j * E + e (slot position j, expert e), the order the down projection uses.
    """
    import torch

    _want(topk_ids, torch.int32, 2, "topk_ids")
    T, k = topk_ids.shape
    G = k * E if order else E
    dev = topk_ids.device
    counts = torch.empty(G, dtype=torch.int32, device=dev)
    offsets = torch.empty(G + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    slot_row = torch.empty(T * k, dtype=torch.int32, device=dev) if with_slot_row else None
    nbytes = max(int(lib().moe_route_workspace_bytes(T, k, E, order)), 16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check("moe_route", lib().moe_route(topk_ids.data_ptr(), T, k, E, order, counts.data_ptr(), offsets.data_ptr(),
                                        perm.data_ptr(), slot_row.data_ptr() if with_slot_row else None,
                                        ws.data_ptr(), nbytes, _stream(topk_ids)))
    if with_slot_row:
        return counts, offsets, perm, slot_row
    return counts, offsets, perm


def moe_gate_up_bf16(x_q, x_scale, perm, offsets, w13_q, w13_scale, topk: int, order: int = 0):
    """Sorted-slot gate/up rows in BF16: [T*k, 2I] (perm/offsets made with ``order``)."""
    import torch

    T, H = x_q.shape
    E, twoI, _ = w13_q.shape
    _check_order(offsets, E, topk, order)
    gu = torch.empty((T * topk, twoI), dtype=torch.bfloat16, device=x_q.device)
    _check("moe_gate_up_bf16", lib().moe_gate_up_bf16(
        x_q.data_ptr(), x_scale.data_ptr(), perm.data_ptr(), offsets.data_ptr(), w13_q.data_ptr(),
        w13_scale.data_ptr(), gu.data_ptr(), T, H, twoI // 2, E, topk, order, _stream(x_q)))
    return gu


def moe_gate_up_swiglu_quant(x_q, x_scale, perm, offsets, w13_q, w13_scale, topk: int, order: int = 0,
                             dst_row=None, workspace=None, return_h=False):
    """Requantised h = silu(g) * u: (h_q uint8 [T*k, I], h_scale f32 [T*k]).

    The tiles follow perm/offsets (made with ``order``); a slot's h lands on
    its sorted row, or on ``dst_row[slot]`` when given (the slot_row of a
    moe_route in the other order). With ``return_h`` also the float32 h rows
    the codes were made from: (h_q, h_scale, h)."""
    import torch

    T, H = x_q.shape
    E, twoI, _ = w13_q.shape
    _check_order(offsets, E, topk, order)
    I = twoI // 2
    if dst_row is not None:
        _want(dst_row, torch.int32, 1, "dst_row")
        if dst_row.numel() != T * topk:
            raise ValueError("dst_row must have T * topk entries")
    nbytes = max(int(lib().moe_gate_up_swiglu_quant_workspace_bytes(T, I, topk)), 16)
    if workspace is None:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=x_q.device)
    h_q = torch.empty((T * topk, I), dtype=torch.uint8, device=x_q.device)
    h_s = torch.empty((T * topk,), dtype=torch.float32, device=x_q.device)
    h = torch.empty((T * topk, I), dtype=torch.float32, device=x_q.device) if return_h else None
    _check("moe_gate_up_swiglu_quant", lib().moe_gate_up_swiglu_quant(
        x_q.data_ptr(), x_scale.data_ptr(), perm.data_ptr(), offsets.data_ptr(),
        dst_row.data_ptr() if dst_row is not None else None, w13_q.data_ptr(), w13_scale.data_ptr(),
        h_q.data_ptr(), h_s.data_ptr(), h.data_ptr() if return_h else None, T, H, I, E, topk, order,
        workspace.data_ptr(), workspace.numel(), _stream(x_q)))
    return (h_q, h_s, h) if return_h else (h_q, h_s)


def moe_down_combine(h_q, h_scale, perm, offsets, topk_ids, topk_w, w2_q, w2_scale, order: int = 0, out=None,
                     y=None):
    """Down projection of the sorted rows and the router-weighted combine: BF16 [T, H].

    perm/offsets come from ``moe_route(..., order=order)``; ``y`` is float32
    scratch [T*k, H] for the per-slot weighted products, which the combine
    sums in float32 and rounds to BF16 once."""
    import torch

    T, k = topk_w.shape
    E, H, I = w2_q.shape
    _check_order(offsets, E, k, order)
    _want(topk_ids, torch.int32, 2, "topk_ids")
    if tuple(topk_ids.shape) != (T, k):
        raise ValueError("topk_ids and topk_w must both be [T, k]")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=h_q.device)
    if y is None:
        y = torch.empty((T * k, H), dtype=torch.float32, device=h_q.device)
    if y.numel() < T * k * H or y.dtype != torch.float32 or not y.is_contiguous():
        raise ValueError("y must be contiguous float32 with at least T * k * H elements")
    _check("moe_down_combine", lib().moe_down_combine(
        h_q.data_ptr(), h_scale.data_ptr(), perm.data_ptr(), offsets.data_ptr(), topk_ids.data_ptr(),
        topk_w.data_ptr(), w2_q.data_ptr(), w2_scale.data_ptr(), out.data_ptr(), y.data_ptr(), T, H, I, E, k,
        order, _stream(h_q)))
    return out


def w8a8_grouped_gemm(x_q, x_scale, topk_ids, w13_q, w13_scale):
    """Routing + BF16 gate/up grouped GEMM: (gu [T*k, 2I] sorted, perm [T*k], offsets [E+1])."""
    import torch

    for t, dt, nd, n in ((x_q, torch.uint8, 2, "x_q"), (x_scale, torch.float32, 1, "x_scale"),
                         (topk_ids, torch.int32, 2, "topk_ids"), (w13_q, torch.uint8, 3, "w13_q"),
                         (w13_scale, torch.float32, 2, "w13_scale")):
        _want(t, dt, nd, n)
    T, H, I, E, k = _moe_dims(x_q, topk_ids, w13_q)
    dev = x_q.device
    gu = torch.empty((T * k, 2 * I), dtype=torch.bfloat16, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    nbytes = max(int(lib().w8a8_grouped_gemm_workspace_bytes(T, k, E)), 16)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _check("w8a8_grouped_gemm", lib().w8a8_grouped_gemm(
        x_q.data_ptr(), x_scale.data_ptr(), topk_ids.data_ptr(), w13_q.data_ptr(), w13_scale.data_ptr(),
        gu.data_ptr(), perm.data_ptr(), offsets.data_ptr(), T, H, I, E, k, ws.data_ptr(), nbytes, _stream(x_q)))
    return gu, perm, offsets


def moe_workspace(T: int, H: int, I: int, E: int, topk: int, device="cuda"):
    """Scratch buffer sized for moe_w8a8_grouped."""
    import torch

    nbytes = int(lib().moe_w8a8_workspace_bytes(T, H, I, E, topk))
    if nbytes == 0 and T > 0:
        raise ValueError("unsupported routed-expert sizes")
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def moe_w8a8_grouped(x_q, x_scale, topk_ids, topk_w, w13_q, w13_scale, w2_q, w2_scale, out=None, workspace=None,
                     quantize_output=False):
    """One routed-expert pass on per-token FP8 tokens: BF16 [T, H].

    With ``quantize_output`` the pass also returns the per-token FP8 version
    of its output (codes [T, H], scales [T]), made in the combine: the input
    of the next pass. Returns ``out`` or ``(out, out_q, out_scale)``."""
    import torch

    for t, dt, nd, n in ((x_q, torch.uint8, 2, "x_q"), (x_scale, torch.float32, 1, "x_scale"),
                         (topk_ids, torch.int32, 2, "topk_ids"), (topk_w, torch.float32, 2, "topk_w"),
                         (w13_q, torch.uint8, 3, "w13_q"), (w13_scale, torch.float32, 2, "w13_scale"),
                         (w2_q, torch.uint8, 3, "w2_q"), (w2_scale, torch.float32, 2, "w2_scale")):
        _want(t, dt, nd, n)
    T, H, I, E, k = _moe_dims(x_q, topk_ids, w13_q)
    if tuple(w2_q.shape) != (E, H, I) or tuple(topk_w.shape) != (T, k):
        raise ValueError("w2_q must be [E, H, I] and topk_w [T, k]")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x_q.device)
    if workspace is None:
        workspace = moe_workspace(T, H, I, E, k, device=x_q.device)
    oq = os_ = None
    if quantize_output:
        oq = torch.empty((T, H), dtype=torch.uint8, device=x_q.device)
        os_ = torch.empty((T,), dtype=torch.float32, device=x_q.device)
    _check("moe_w8a8_grouped", lib().moe_w8a8_grouped(
        x_q.data_ptr(), x_scale.data_ptr(), topk_ids.data_ptr(), topk_w.data_ptr(), w13_q.data_ptr(),
        w13_scale.data_ptr(), w2_q.data_ptr(), w2_scale.data_ptr(), out.data_ptr(),
        oq.data_ptr() if quantize_output else None, os_.data_ptr() if quantize_output else None, T, H, I, E, k,
        workspace.data_ptr(), workspace.numel(), _stream(x_q)))
    return (out, oq, os_) if quantize_output else out


def moe_ffn(x, routes, w13_q, w13_scale, w2_q, w2_scale, workspace=None):
    """The routed-expert stage run once per entry of ``routes`` with the same
    weights, each pass fed the previous pass's output (every token goes
    through the block stack two times on one set of weights; sglang-metis
    0.1.0, "How the model maps onto SGLang"). ``routes`` is a list of
    (topk_ids, topk_w). The first pass's input is quantised per token here;
    each later pass takes the per-token FP8 output that the previous pass's
    combine wrote. Returns the list of per-pass BF16 outputs."""
    outs = []
    xq, xs = quantize_per_token(x)
    for i, (ids, w) in enumerate(routes):
        last = i + 1 == len(routes)
        r = moe_w8a8_grouped(xq, xs, ids, w, w13_q, w13_scale, w2_q, w2_scale, workspace=workspace,
                             quantize_output=not last)
        if last:
            outs.append(r)
        else:
            out, xq, xs = r
            outs.append(out)
    return outs


# ---- MXFP4 routed experts -------------------------------------------------------
#
# Codes are uint8 with two E2M1 values per byte (element 2i in the low
# nibble), scales uint8 E8M0 with one byte per 32 values along K:
# x_q [T, H/2] / x_scale [T, H/32], w13_q [E, 2I, H/2] / w13_scale
# [E, 2I, H/32], w2_q [E, H, I/2] / w2_scale [E, H, I/32].


def mxfp4_quantize(x, q=None, scale=None):
    """BF16 [M, K] -> (codes uint8 [M, K/2], E8M0 scales uint8 [M, K/32]), one
    power-of-two scale per 32 values: 2^(floor(log2 amax) - 2)."""
    import torch

    _want(x, torch.bfloat16, 2, "x")
    M, K = x.shape
    if q is None:
        q = torch.empty((M, K // 2), dtype=torch.uint8, device=x.device)
    if scale is None:
        scale = torch.empty((M, K // 32), dtype=torch.uint8, device=x.device)
    _want(q, torch.uint8, 2, "q")
    _want(scale, torch.uint8, 2, "scale")
    if tuple(q.shape) != (M, K // 2) or tuple(scale.shape) != (M, K // 32):
        raise ValueError("output shapes do not match x")
    _check("mxfp4_quantize", lib().mxfp4_quantize(x.data_ptr(), M, K, q.data_ptr(), scale.data_ptr(), _stream(x)))
    return q, scale


def _mx_dims(x_q, x_scale, topk_ids, w13_q, w13_scale):
    import torch

    for t, nd, n in ((x_q, 2, "x_q"), (x_scale, 2, "x_scale"), (w13_q, 3, "w13_q"), (w13_scale, 3, "w13_scale")):
        _want(t, torch.uint8, nd, n)
    T, Hh = x_q.shape
    H = 2 * Hh
    E, twoI, H2 = w13_q.shape
    if 2 * H2 != H or twoI % 2 or tuple(x_scale.shape) != (T, H // 32) or tuple(w13_scale.shape) != (E, twoI, H // 32):
        raise ValueError("x_q [T, H/2], x_scale [T, H/32], w13_q [E, 2I, H/2], w13_scale [E, 2I, H/32] expected")
    k = topk_ids.shape[1] if topk_ids is not None else None
    if topk_ids is not None and topk_ids.shape[0] != T:
        raise ValueError("topk_ids must be [T, k]")
    return T, H, twoI // 2, E, k


def moe_mxfp4_gate_up_bf16(x_q, x_scale, perm, offsets, w13_q, w13_scale, topk: int, order: int = 0):
    """Sorted-slot gate/up rows of the MXFP4 product in BF16: [T*k, 2I]."""
    import torch

    T, H, I, E, _ = _mx_dims(x_q, x_scale, None, w13_q, w13_scale)
    _check_order(offsets, E, topk, order)
    gu = torch.empty((T * topk, 2 * I), dtype=torch.bfloat16, device=x_q.device)
    _check("moe_mxfp4_gate_up_bf16", lib().moe_mxfp4_gate_up_bf16(
        x_q.data_ptr(), x_scale.data_ptr(), perm.data_ptr(), offsets.data_ptr(), w13_q.data_ptr(),
        w13_scale.data_ptr(), gu.data_ptr(), T, H, I, E, topk, order, _stream(x_q)))
    return gu


def moe_mxfp4_gate_up_swiglu_quant(x_q, x_scale, perm, offsets, w13_q, w13_scale, topk: int, order: int = 0,
                                   dst_row=None):
    """MXFP4 h = silu(g) * u of every routed slot: (h_q uint8 [T*k, I/2], h_scale uint8 [T*k, I/32]),
    on the sorted row of ``perm`` or on ``dst_row[slot]`` when given."""
    import torch

    T, H, I, E, _ = _mx_dims(x_q, x_scale, None, w13_q, w13_scale)
    _check_order(offsets, E, topk, order)
    if dst_row is not None:
        _want(dst_row, torch.int32, 1, "dst_row")
        if dst_row.numel() != T * topk:
            raise ValueError("dst_row must have T * topk entries")
    h_q = torch.empty((T * topk, I // 2), dtype=torch.uint8, device=x_q.device)
    h_s = torch.empty((T * topk, I // 32), dtype=torch.uint8, device=x_q.device)
    _check("moe_mxfp4_gate_up_swiglu_quant", lib().moe_mxfp4_gate_up_swiglu_quant(
        x_q.data_ptr(), x_scale.data_ptr(), perm.data_ptr(), offsets.data_ptr(),
        dst_row.data_ptr() if dst_row is not None else None, w13_q.data_ptr(), w13_scale.data_ptr(),
        h_q.data_ptr(), h_s.data_ptr(), T, H, I, E, topk, order, _stream(x_q)))
    return h_q, h_s


def moe_mxfp4_down_combine(h_q, h_scale, perm, offsets, topk_ids, topk_w, w2_q, w2_scale, order: int = 0,
                           out=None, y=None, quantize_output=False):
    """MXFP4 down projection and combine: BF16 [T, H], or (out, out_q, out_scale)
    with ``quantize_output`` (the MXFP4 version of out, made in the combine)."""
    import torch

    T, k = topk_w.shape
    E, H, Ih = w2_q.shape
    I = 2 * Ih
    _check_order(offsets, E, k, order)
    _want(topk_ids, torch.int32, 2, "topk_ids")
    if tuple(topk_ids.shape) != (T, k) or tuple(w2_scale.shape) != (E, H, I // 32):
        raise ValueError("topk_ids [T, k] and w2_scale [E, H, I/32] expected")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=h_q.device)
    if y is None:
        y = torch.empty((T * k, H), dtype=torch.float32, device=h_q.device)
    if y.numel() < T * k * H or y.dtype != torch.float32 or not y.is_contiguous():
        raise ValueError("y must be contiguous float32 with at least T * k * H elements")
    oq = os_ = None
    if quantize_output:
        oq = torch.empty((T, H // 2), dtype=torch.uint8, device=h_q.device)
        os_ = torch.empty((T, H // 32), dtype=torch.uint8, device=h_q.device)
    _check("moe_mxfp4_down_combine", lib().moe_mxfp4_down_combine(
        h_q.data_ptr(), h_scale.data_ptr(), perm.data_ptr(), offsets.data_ptr(), topk_ids.data_ptr(),
        topk_w.data_ptr(), w2_q.data_ptr(), w2_scale.data_ptr(), out.data_ptr(), y.data_ptr(),
        oq.data_ptr() if quantize_output else None, os_.data_ptr() if quantize_output else None, T, H, I, E, k,
        order, _stream(h_q)))
    return (out, oq, os_) if quantize_output else out


def moe_mxfp4_workspace(T: int, H: int, I: int, E: int, topk: int, device="cuda"):
    """Scratch buffer sized for moe_mxfp4_grouped."""
    import torch

    nbytes = int(lib().moe_mxfp4_workspace_bytes(T, H, I, E, topk))
    if nbytes == 0 and T > 0:
        raise ValueError("unsupported routed-expert sizes")
    return torch.empty(max(nbytes, 16), dtype=torch.uint8, device=device)


def moe_mxfp4_grouped(x_q, x_scale, topk_ids, topk_w, w13_q, w13_scale, w2_q, w2_scale, out=None, workspace=None,
                      quantize_output=False):
    """One MXFP4 routed-expert pass: BF16 [T, H], or (out, out_q, out_scale) with
    ``quantize_output`` (the MXFP4 input of the next pass)."""
    import torch

    _want(topk_ids, torch.int32, 2, "topk_ids")
    _want(topk_w, torch.float32, 2, "topk_w")
    _want(w2_q, torch.uint8, 3, "w2_q")
    _want(w2_scale, torch.uint8, 3, "w2_scale")
    T, H, I, E, k = _mx_dims(x_q, x_scale, topk_ids, w13_q, w13_scale)
    if tuple(w2_q.shape) != (E, H, I // 2) or tuple(w2_scale.shape) != (E, H, I // 32) or tuple(topk_w.shape) != (T, k):
        raise ValueError("w2_q [E, H, I/2], w2_scale [E, H, I/32] and topk_w [T, k] expected")
    if out is None:
        out = torch.empty((T, H), dtype=torch.bfloat16, device=x_q.device)
    if workspace is None:
        workspace = moe_mxfp4_workspace(T, H, I, E, k, device=x_q.device)
    oq = os_ = None
    if quantize_output:
        oq = torch.empty((T, H // 2), dtype=torch.uint8, device=x_q.device)
        os_ = torch.empty((T, H // 32), dtype=torch.uint8, device=x_q.device)
    _check("moe_mxfp4_grouped", lib().moe_mxfp4_grouped(
        x_q.data_ptr(), x_scale.data_ptr(), topk_ids.data_ptr(), topk_w.data_ptr(), w13_q.data_ptr(),
        w13_scale.data_ptr(), w2_q.data_ptr(), w2_scale.data_ptr(), out.data_ptr(),
        oq.data_ptr() if quantize_output else None, os_.data_ptr() if quantize_output else None, T, H, I, E, k,
        workspace.data_ptr(), workspace.numel(), _stream(x_q)))
    return (out, oq, os_) if quantize_output else out


def moe_mxfp4_ffn(x, routes, w13_q, w13_scale, w2_q, w2_scale, workspace=None):
    """The MXFP4 routed-expert stage run once per entry of ``routes`` on one set of
    weights, each pass fed the previous pass's output (quantised in its combine).
    Returns the list of per-pass BF16 outputs."""
    outs = []
    xq, xs = mxfp4_quantize(x)
    for i, (ids, w) in enumerate(routes):
        last = i + 1 == len(routes)
        r = moe_mxfp4_grouped(xq, xs, ids, w, w13_q, w13_scale, w2_q, w2_scale, workspace=workspace,
                              quantize_output=not last)
        if last:
            outs.append(r)
        else:
            out, xq, xs = r
            outs.append(out)
    return outs
