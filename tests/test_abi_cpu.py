"""The C ABI without a GPU: the library loads, exports every function that
include/w8a8.h declares, and rejects bad arguments on the host (before any
device work) with the documented status codes."""
import ctypes
import glob
import os
import re

import pytest

import w8a8_fp8_linear_amd as w8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DECL = re.compile(r"^\s*(?:const\s+)?(?:int64_t|int|size_t|char|void)\s*\*?\s*(\w+)\s*\(", re.M)

OK, NULL, SHAPE, MIS, UNSUP, WS, DEV, LAUNCH, SCRATCH = range(9)


def _declared():
    names = set()
    for h in glob.glob(os.path.join(ROOT, "include", "*.h")):
        names |= set(DECL.findall(open(h).read()))
    return names


def test_header_declares_entry_points():
    names = _declared()
    assert {"quantize_per_token", "w8a8_gemm", "w8a8_abi_version", "w8a8_status_string"} <= names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(w8.lib_path())
    for name in _declared():
        assert hasattr(lib, name), name


def test_binding_covers_every_declared_symbol():
    assert _declared() <= set(w8._SIGNATURES)


def test_abi_version_and_status_strings():
    assert w8.abi_version() == 2
    for s in range(9):
        assert w8.lib().w8a8_status_string(s)
    assert w8.lib().w8a8_status_string(99) == b"unknown status"


P = 1 << 20   # a fake, 16-byte aligned address; never dereferenced (checks fail first)


def test_quantize_argument_errors():
    f = w8.lib().quantize_per_token
    assert f(P, -1, 16, P, P, None) == SHAPE
    assert f(P, 4, -16, P, P, None) == SHAPE
    assert f(P, 1 << 62, 1 << 4, P, P, None) == SHAPE
    assert f(P, 4, 0, P, P, None) == UNSUP
    assert f(P, 4, 24, P, P, None) == UNSUP
    assert f(P, 0, 16, P, P, None) == OK          # empty: no-op, no device needed
    assert f(None, 4, 16, P, P, None) == NULL
    assert f(P, 4, 16, None, P, None) == NULL
    assert f(P, 4, 16, P, None, None) == NULL
    assert f(P + 8, 4, 16, P, P, None) == MIS
    assert f(P, 4, 16, P + 4, P, None) == MIS


def test_gemm_argument_errors():
    f = w8.lib().w8a8_gemm
    assert f(P, P, P, P, P, -1, 16, 16, None) == SHAPE
    assert f(P, P, P, P, P, 4, 16, 8, None) == UNSUP
    assert f(P, P, P, P, P, 4, 24, 16, None) == UNSUP
    assert f(P, P, P, P, P, 0, 16, 16, None) == OK
    assert f(P, P, P, P, P, 4, 0, 16, None) == OK
    assert f(None, P, P, P, P, 4, 16, 16, None) == NULL
    assert f(P, P, P, P, None, 4, 16, 16, None) == NULL
    assert f(P, P, P + 1, P, P, 4, 16, 16, None) == MIS


def test_gemm_timed_argument_errors():
    f = w8.lib().w8a8_gemm_timed
    E = ctypes.c_void_p(64)  # a non-null event handle; never used on these paths
    assert f(P, P, P, P, P, 4, 16, 16, None, None, E) == NULL
    assert f(P, P, P, P, P, 4, 16, 16, None, E, None) == NULL
    assert f(P, P, P, P, P, -1, 16, 16, None, E, E) == SHAPE
    assert f(P, P, P, P, P, 4, 16, 8, None, E, E) == UNSUP
    assert f(P, P, P, P, P, 0, 16, 16, None, E, E) == OK
    assert f(None, P, P, P, P, 4, 16, 16, None, E, E) == NULL
    assert f(P, P, P + 1, P, P, 4, 16, 16, None, E, E) == MIS


def test_valid_call_without_gpu_reports_device():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert w8.lib().quantize_per_token(P, 4, 16, P, P, None) == DEV
    assert w8.lib().w8a8_gemm(P, P, P, P, P, 4, 16, 16, None) == DEV


def test_w8a16_gemm_argument_errors():
    f = w8.lib().w8a16_gemm
    assert f(P, P, P, P, -1, 16, 16, None) == SHAPE
    assert f(P, P, P, P, 4, 16, 8, None) == UNSUP
    assert f(P, P, P, P, 4, 24, 16, None) == UNSUP
    assert f(P, P, P, P, 0, 16, 16, None) == OK
    assert f(None, P, P, P, 4, 16, 16, None) == NULL
    assert f(P, P, None, P, 4, 16, 16, None) == NULL
    assert f(P + 2, P, P, P, 4, 16, 16, None) == MIS


def test_fp8_linear_argument_errors():
    f = w8.lib().fp8_linear
    need = w8.lib().fp8_linear_workspace_bytes(64, 32)
    assert need == 64 * 32 + 256
    assert f(P, P, P, P, -1, 16, 16, 1, P, 1 << 20, None) == SHAPE
    assert f(P, P, P, P, 64, 16, 8, 1, P, 1 << 20, None) == UNSUP
    # the FP8 path (fast_math, M > 8) needs the workspace; the default path does not read it
    assert f(P, P, P, P, 64, 16, 32, 1, None, 0, None) == NULL
    assert f(P, P, P, P, 64, 16, 32, 1, P + 4, need, None) == MIS
    assert f(P, P, P, P, 64, 16, 32, 1, P, need - 1, None) == WS
    import torch
    if not torch.cuda.is_available():
        assert f(P, P, P, P, 8, 16, 32, 1, None, 0, None) == DEV   # M <= 8: default maths, no workspace
        assert f(P, P, P, P, 64, 16, 32, 0, None, 0, None) == DEV  # flag off: default maths
        assert f(P, P, P, P, 64, 16, 32, 1, P, need, None) == DEV
    g = w8.lib().fp8_linear_single_launch
    assert g(P, P, P, P, 33, 16, 32, None) == UNSUP          # M <= 32
    assert g(P, P, P, P, 16, 16, 2064, None) == UNSUP        # K <= 2048
    assert g(P, P, P, P, 16, 16, 24, None) == UNSUP          # K % 16
    assert g(P, P, P, P, 0, 16, 32, None) == OK
    assert g(None, P, P, P, 16, 16, 32, None) == NULL
    assert g(P, P, P, P + 2, 16, 16, 32, None) == MIS
    if not torch.cuda.is_available():
        assert g(P, P, P, P, 16, 16, 32, None) == DEV


def test_mxfp4_quantize_argument_errors():
    f = w8.lib().mxfp4_quantize
    assert f(P, -1, 32, P, P, None) == SHAPE
    assert f(P, 4, 16, P, P, None) == UNSUP      # K must be a multiple of 32
    assert f(P, 4, 0, P, P, None) == UNSUP
    assert f(P, 0, 32, P, P, None) == OK
    assert f(None, 4, 32, P, P, None) == NULL
    assert f(P, 4, 32, P, None, None) == NULL
    assert f(P, 4, 32, P, P + 8, None) == MIS
    import torch
    if not torch.cuda.is_available():
        assert f(P, 4, 32, P, P, None) == DEV


def test_mxfp4_expert_argument_errors():
    L = w8.lib()
    T, H, I, E, k = 64, 256, 128, 8, 2
    # H and I must be multiples of 128
    assert L.moe_mxfp4_gate_up_bf16(P, P, P, P, P, P, P, T, 192, I, E, k, 0, None) == UNSUP
    assert L.moe_mxfp4_gate_up_swiglu_quant(P, P, P, P, None, P, P, P, P, T, H, 64, E, k, 0, None) == UNSUP
    assert L.moe_mxfp4_gate_up_swiglu_quant(P, P, P, P, None, P, P, P, P, T, H, I, E, k, 2, None) == UNSUP
    assert L.moe_mxfp4_down_combine(*([P] * 12), -1, H, I, E, k, 0, None) == SHAPE
    assert L.moe_mxfp4_down_combine(*([P] * 12), 0, H, I, E, k, 0, None) == OK
    # out_q and out_scale come together
    assert L.moe_mxfp4_down_combine(*([P] * 10), P, None, T, H, I, E, k, 0, None) == NULL
    assert L.moe_mxfp4_gate_up_bf16(P, None, P, P, P, P, P, T, H, I, E, k, 0, None) == NULL
    assert L.moe_mxfp4_gate_up_swiglu_quant(P, P, P, P, P + 4, P, P, P, P, T, H, I, E, k, 0, None) == MIS
    need = L.moe_mxfp4_workspace_bytes(T, H, I, E, k)
    assert need > T * k * H * 2 and L.moe_mxfp4_workspace_bytes(T, H, 96, E, k) == 0
    g = L.moe_mxfp4_grouped
    assert g(*([P] * 9), None, None, T, H, I, E, k, P, need - 1, None) == WS
    assert g(*([P] * 9), P, None, T, H, I, E, k, P, need, None) == NULL
    assert g(*([P] * 9), None, None, T, H, I, 0, k, P, need, None) == UNSUP
    import torch
    if not torch.cuda.is_available():
        assert g(*([P] * 9), None, None, T, H, I, E, k, P, need, None) == DEV


def test_conversion_argument_errors():
    for name in ("e4m3_from_f32", "bf16_from_f32"):
        f = getattr(w8.lib(), name)
        assert f(P, -1, P, None) == SHAPE
        assert f(P, (1 << 40) + 1, P, None) == UNSUP
        assert f(P, 0, P, None) == OK              # empty: no-op, no device needed
        assert f(None, 4, P, None) == NULL
        assert f(P, 4, None, None) == NULL
        assert f(P + 4, 4, P, None) == MIS
        assert f(P, 4, P + 2, None) == MIS
        assert f(P, 4, P, None) == DEV             # valid arguments: no GPU here


def test_gate_up_swiglu_quant_h_output_alignment():
    f = w8.lib().moe_gate_up_swiglu_quant
    args = [P] * 9 + [P + 4]                       # h_f32 misaligned
    assert f(*args, 8, 256, 128, 2, 2, 0, P, 1 << 30, None) == MIS
    args[9] = None                                  # h_f32 is optional
    assert f(*args, 8, 256, 128, 2, 2, 0, P, 1 << 30, None) == DEV


def test_fp8_linear_noalloc_argument_errors():
    f = w8.lib().fp8_linear_noalloc
    limit = w8.lib().fp8_linear_noalloc_max_bytes()
    assert limit == 64 << 20
    assert f(P, P, P, P, -1, 16, 16, 1, None) == SHAPE
    assert f(P, P, P, P, 64, 16, 24, 1, None) == UNSUP
    # the FP8 path of 8192 x 8192 needs 64 MiB of codes plus the scales: refused before any launch
    assert f(P, P, P, P, 8192, 16, 8192, 1, None) == SCRATCH
    assert f(P, P, P, P, 8192, 16, 8192, 0, None) == DEV      # default maths: no scratch
    assert f(P, P, P, P, 16, 16, 2048, 1, None) == DEV        # single launch: no scratch
    assert f(P, P, P, P, 4096, 16, 2048, 1, None) == DEV      # fits
    assert f(P, P, P, P, 0, 16, 16, 1, None) == OK
    assert f(None, P, P, P, 64, 16, 16, 1, None) == NULL
    assert f(P, P, P, P + 8, 64, 16, 16, 1, None) == MIS


def test_clock_probe_argument_errors():
    f = w8.lib().clock_probe
    assert f(P, -1, None) == SHAPE
    assert f(P, 65537, None) == UNSUP
    assert f(P, 0, None) == OK
    assert f(None, 4, None) == NULL
    assert f(P + 8, 4, None) == MIS
    assert f(P, 4, None) == DEV


def test_read_probe_argument_errors():
    f = w8.lib().read_probe
    assert w8.lib().read_probe_sink_words(16809984) == 513
    assert w8.lib().read_probe_sink_words(32768) == 1
    assert f(P, -16, P, None) == SHAPE
    assert f(P, 24, P, None) == UNSUP
    assert f(P, 0, P, None) == OK
    assert f(None, 32, P, None) == NULL
    assert f(P, 32, None, None) == NULL
    assert f(P + 8, 32, P, None) == MIS
    assert f(P, 32, P, None) == DEV
