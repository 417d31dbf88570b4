"""The C-ABI library on a machine without a GPU: it loads, exports every declared symbol, and
rejects bad arguments on the host before touching HIP."""

import ctypes
import os
import re

import pytest

import gemv_layers_amd as g

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "gemm_bf16.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gemm_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    L = g.lib()
    names = _declared()
    assert len(names) >= 14
    for n in names:
        assert hasattr(L, n), n
    assert sorted(g.EXPORTS) == names


def test_status_strings():
    assert g.status_string(0) == "GEMM_OK"
    assert g.status_string(2) == "GEMM_ERR_UNSUPPORTED"
    assert g.status_string(99) == "GEMM_ERR_UNKNOWN"


P = ctypes.c_void_p(16)  # a non-null, 16-byte aligned stand-in; never dereferenced here


@pytest.mark.parametrize("args,status", [
    ((-1, 8, 8, P, 8, P, 8, P, 8), g.GEMM_ERR_INVALID_ARG),
    ((8, -1, 8, P, 8, P, 8, P, 8), g.GEMM_ERR_INVALID_ARG),
    ((8, 8, -1, P, 8, P, 8, P, 8), g.GEMM_ERR_INVALID_ARG),
    ((8, 8, 16, P, 8, P, 8, P, 8), g.GEMM_ERR_INVALID_ARG),      # lda < K
    ((8, 16, 8, P, 8, P, 8, P, 16), g.GEMM_ERR_INVALID_ARG),     # ldb < N
    ((8, 16, 8, P, 8, P, 16, P, 8), g.GEMM_ERR_INVALID_ARG),     # ldc < N
    ((8, 8, 8, None, 8, P, 8, P, 8), g.GEMM_ERR_INVALID_ARG),    # null A
    ((8, 8, 8, P, 8, None, 8, P, 8), g.GEMM_ERR_INVALID_ARG),    # null B
    ((8, 8, 8, P, 8, P, 8, None, 8), g.GEMM_ERR_INVALID_ARG),    # null C
    ((0, 8, 8, None, 8, P, 8, None, 8), g.GEMM_OK),              # empty output: no-op
    ((8, 0, 8, P, 8, None, 8, None, 8), g.GEMM_OK),
    ((0, 8, 8, None, 8, None, 8, None, 8), g.GEMM_ERR_INVALID_ARG),  # B (8 x 8) null
    ((8, 8, 8, P, 8, P, 8, P, 8), g.GEMM_ERR_NOT_INITIALIZED),   # no gemm_init yet
])
def test_validation_without_gpu(args, status):
    assert g.lib().gemm_bf16(*args, None) == status


def test_skinny_entry_rejects_large_m():
    L = g.lib()
    assert L.gemm_bf16_skinny(65, 8, 8, P, 8, P, 8, P, 8, None) == g.GEMM_ERR_UNSUPPORTED
    assert L.gemm_bf16_skinny(0, 8, 8, P, 8, P, 8, P, 8, None) == g.GEMM_ERR_UNSUPPORTED
    assert L.gemm_bf16_skinny(64, 8, 8, P, 8, P, 8, P, 8, None) == g.GEMM_ERR_NOT_INITIALIZED


def test_measurement_entry_validation():
    L = g.lib()
    assert L.gemm_peak_copy_launch(P, P, 17, None) == g.GEMM_ERR_INVALID_ARG
    assert L.gemm_peak_copy_launch(P, ctypes.c_void_p(8), 16, None) == g.GEMM_ERR_INVALID_ARG
    assert L.gemm_peak_copy_launch(P, P, 0, None) == g.GEMM_OK
    assert L.gemm_peak_read_launch(P, 16, None, None) == g.GEMM_ERR_INVALID_ARG
    assert L.gemm_fill_launch(P, 6, 0, None) == g.GEMM_ERR_INVALID_ARG
    assert L.gemm_peak_mfma_launch(10, 0, P, P, None) == g.GEMM_ERR_INVALID_ARG


def test_last_plan_buffer_handling():
    buf = ctypes.create_string_buffer(2)
    assert g.lib().gemm_last_plan(buf, 2) in (g.GEMM_OK, g.GEMM_ERR_INVALID_ARG)
    assert g.lib().gemm_last_plan(None, 0) == g.GEMM_ERR_INVALID_ARG


@pytest.mark.parametrize("args,status", [
    ((8, 8, 8, P, 8, P, 8, P, 8), g.GEMM_ERR_INVALID_ARG),       # ldb < 2N
    ((8, 8, 8, P, 8, P, 15, P, 8), g.GEMM_ERR_INVALID_ARG),      # ldb = 2N - 1
    ((8, 8, 8, P, 8, P, 16, P, 7), g.GEMM_ERR_INVALID_ARG),      # ldc < N
    ((8, 8, 16, P, 8, P, 16, P, 8), g.GEMM_ERR_INVALID_ARG),     # lda < K
    ((8, 8, 8, P, 8, None, 16, P, 8), g.GEMM_ERR_INVALID_ARG),   # null B
    ((-1, 8, 8, P, 8, P, 16, P, 8), g.GEMM_ERR_INVALID_ARG),
    ((8, 2**62, 8, P, 8, P, 2**63 - 1, P, 2**62), g.GEMM_ERR_INVALID_ARG),  # 2N overflows
    ((0, 8, 8, None, 8, P, 16, None, 8), g.GEMM_OK),             # empty output: no-op
    ((8, 8, 8, P, 8, P, 16, P, 8), g.GEMM_ERR_NOT_INITIALIZED),  # valid, no gemm_init yet
])
def test_swiglu_validation_without_gpu(args, status):
    assert g.lib().gemm_bf16_swiglu(*args, None) == status


def test_plan_describe_flags():
    buf = ctypes.create_string_buffer(4096)
    assert g.lib().gemm_plan_describe(4, 64, 64, 256, 16, buf, 4096) == g.GEMM_ERR_INVALID_ARG
    assert g.lib().gemm_plan_describe(4, 64, 64, 256, 12, buf, 4096) == g.GEMM_ERR_INVALID_ARG
    assert g.lib().gemm_plan_describe(4, 64, 64, 256, 8, buf, 4096) == g.GEMM_OK
    assert g.lib().gemm_plan_describe(4, 64, 48, 256, 8, buf, 4096) == g.GEMM_ERR_UNSUPPORTED
    assert g.lib().gemm_plan_describe(4, 64, 128, 256, 5, buf, 4096) == g.GEMM_ERR_INVALID_ARG
    assert g.lib().gemm_plan_describe(4, 64, 64, 256, 4, buf, 4096) == g.GEMM_ERR_UNSUPPORTED
    assert g.lib().gemm_plan_describe(65, 64, 64, 256, 3, buf, 4096) == g.GEMM_ERR_UNSUPPORTED
    assert g.gemm_plan_describe(4, 64, 64, swiglu=True)["op"] == "swiglu"
    assert g.gemm_plan_describe(4, 64, 64)["op"] == "gemm"


# ---- block-scaled (MX) entry points: validation on the host ---------------------------------

def test_mx_packed_sizes():
    w, s = ctypes.c_int64(), ctypes.c_int64()
    L = g.lib()
    assert L.gemm_mx_packed_sizes(11008, 4096, ctypes.byref(w), ctypes.byref(s)) == g.GEMM_OK
    assert (w.value, s.value) == (688 * 32 * 1024, 688 * 8 * 256)
    assert L.gemm_mx_packed_sizes(4096, 11008, ctypes.byref(w), ctypes.byref(s)) == g.GEMM_OK
    assert (w.value, s.value) == (256 * 86 * 1024, 256 * 22 * 256)
    assert L.gemm_mx_packed_sizes(17, 128, ctypes.byref(w), ctypes.byref(s)) == g.GEMM_ERR_INVALID_ARG
    assert L.gemm_mx_packed_sizes(16, 100, ctypes.byref(w), ctypes.byref(s)) == g.GEMM_ERR_INVALID_ARG


def test_mx_validation_without_gpu():
    L = g.lib()
    Q = ctypes.c_void_p(4096)
    # decode: M > 64, N % 16, K % 128 unsupported; misaligned or short leading dimensions invalid
    assert L.gemm_mx_decode(65, 16, 128, Q, 128, Q, 4, Q, Q, Q, 16, None) == g.GEMM_ERR_UNSUPPORTED
    assert L.gemm_mx_decode(1, 24, 128, Q, 128, Q, 4, Q, Q, Q, 24, None) == g.GEMM_ERR_UNSUPPORTED
    assert L.gemm_mx_decode(1, 16, 96, Q, 128, Q, 4, Q, Q, Q, 16, None) == g.GEMM_ERR_UNSUPPORTED
    assert L.gemm_mx_decode(1, 16, 128, Q, 120, Q, 4, Q, Q, Q, 16, None) == g.GEMM_ERR_INVALID_ARG
    assert L.gemm_mx_decode(1, 16, 128, Q, 136, Q, 4, Q, Q, Q, 16, None) == g.GEMM_ERR_INVALID_ARG
    assert L.gemm_mx_decode(1, 16, 128, Q, 128, Q, 3, Q, Q, Q, 16, None) == g.GEMM_ERR_INVALID_ARG
    assert L.gemm_mx_decode(1, 16, 128, Q, 128, Q, 4, Q, Q, ctypes.c_void_p(4098), 16, None) \
        == g.GEMM_ERR_INVALID_ARG
    assert L.gemm_mx_decode(1, 16, 128, Q, 128, Q, 4, None, Q, Q, 16, None) == g.GEMM_ERR_INVALID_ARG
    assert L.gemm_mx_decode(0, 16, 128, None, 128, None, 4, Q, Q, None, 16, None) == g.GEMM_OK
    assert L.gemm_mx_decode(1, 16, 128, Q, 128, Q, 4, Q, Q, Q, 16, None) == g.GEMM_ERR_NOT_INITIALIZED
    # conversions
    assert L.gemm_mx_quantize_act(1, 48, Q, 48, Q, 48, Q, 2, None) == g.GEMM_ERR_INVALID_ARG   # K % 32
    assert L.gemm_mx_quantize_act(1, 64, Q, 60, Q, 64, Q, 2, None) == g.GEMM_ERR_INVALID_ARG   # lda < K
    assert L.gemm_mx_quantize_act(1, 64, Q, 64, Q, 72, Q, 2, None) == g.GEMM_ERR_INVALID_ARG   # ldaq % 16
    assert L.gemm_mx_quantize_act(1, 64, Q, 64, Q, 64, Q, 2, None) == g.GEMM_ERR_NOT_INITIALIZED
    assert L.gemm_mx_pack_weight(24, 128, Q, 128, Q, Q, None) == g.GEMM_ERR_INVALID_ARG
    assert L.gemm_mx_pack_weight(16, 128, Q, 120, Q, Q, None) == g.GEMM_ERR_INVALID_ARG
    assert L.gemm_mx_pack_weight(16, 128, Q, 128, Q, Q, None) == g.GEMM_ERR_NOT_INITIALIZED
    assert L.gemm_mx_decode_bf16(65, 16, 128, Q, 128, Q, Q, Q, 16, None) == g.GEMM_ERR_UNSUPPORTED
    assert L.gemm_mx_decode_bf16(1, 16, 128, Q, 128, Q, Q, Q, 16, None) == g.GEMM_ERR_NOT_INITIALIZED


def test_packed_validation_without_gpu():
    L = g.lib()
    Q = ctypes.c_void_p(4096)
    assert L.gemm_pack_weight_bf16(48, 16, Q, 16, Q, None) == g.GEMM_ERR_INVALID_ARG   # K % 32
    assert L.gemm_pack_weight_bf16(64, 24, Q, 24, Q, None) == g.GEMM_ERR_INVALID_ARG   # N % 16
    assert L.gemm_pack_weight_bf16(64, 16, Q, 8, Q, None) == g.GEMM_ERR_INVALID_ARG    # ldb < N
    assert L.gemm_pack_weight_bf16(64, 16, Q, 16, Q, None) == g.GEMM_ERR_NOT_INITIALIZED
    assert L.gemm_bf16_packed(65, 16, 64, Q, 64, Q, Q, 16, None) == g.GEMM_ERR_UNSUPPORTED
    assert L.gemm_bf16_packed(1, 24, 64, Q, 64, Q, Q, 24, None) == g.GEMM_ERR_UNSUPPORTED
    assert L.gemm_bf16_packed(1, 16, 48, Q, 48, Q, Q, 16, None) == g.GEMM_ERR_UNSUPPORTED
    assert L.gemm_bf16_packed(1, 16, 64, Q, 60, Q, Q, 16, None) == g.GEMM_ERR_INVALID_ARG  # lda < K
    assert L.gemm_bf16_packed(1, 16, 64, Q, 68, Q, Q, 16, None) == g.GEMM_ERR_INVALID_ARG  # lda % 8
    assert L.gemm_bf16_packed(0, 16, 64, None, 64, Q, None, 16, None) == g.GEMM_OK
    assert L.gemm_bf16_packed(1, 16, 64, Q, 64, Q, Q, 16, None) == g.GEMM_ERR_NOT_INITIALIZED
