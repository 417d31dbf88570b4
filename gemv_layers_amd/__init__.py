"""Python binding of libgemm_bf16.so, the gfx950 bf16 GEMM library (include/gemm_bf16.h).

Argument marshalling only: every function forwards to the C ABI function of the same name, and
every step of the product runs in the library's HIP kernels. There is no CPU or PyTorch
fallback: if the library is not built, or a call fails, an exception is raised.

The ``matmul`` helper takes PyTorch bf16 tensors (PyTorch is used for device memory and streams
only) and passes their device pointers, leading dimensions and the current stream.
"""

from __future__ import annotations

import ctypes
import json
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgemm_bf16.so")

GEMM_OK = 0
GEMM_ERR_INVALID_ARG = 1
GEMM_ERR_UNSUPPORTED = 2
GEMM_ERR_NOT_INITIALIZED = 3
GEMM_ERR_HIP = 4

GEMM_PLAN_SKINNY = 1
GEMM_PLAN_SWIGLU = 2
GEMM_PLAN_MX = 4
GEMM_PLAN_PACKED = 8

# every symbol include/gemm_bf16.h declares
EXPORTS = (
    "gemm_init", "gemm_bf16", "gemm_bf16_noalloc", "gemm_bf16_skinny", "gemm_bf16_tiled", "gemm_bf16_swiglu",
    "gemm_plan_describe",
    "gemm_wave_efficiency", "gemm_last_plan", "gemm_status_string", "gemm_finalize",
    "gemm_peak_mfma_launch", "gemm_peak_mfma_data_launch", "gemm_peak_copy_launch", "gemm_peak_read_launch",
    "gemm_peak_clock_launch", "gemm_peak_xcc_launch",
    "gemm_peak_empty_launch", "gemm_fill_launch",
    "gemm_mx_packed_sizes", "gemm_mx_pack_weight", "gemm_mx_quantize_act", "gemm_mx_decode",
    "gemm_mx_decode_bf16", "gemm_pack_weight_bf16", "gemm_bf16_packed",
)


class GemmError(RuntimeError):
    def __init__(self, func: str, status: int):
        self.status = status
        super().__init__(f"{func} failed: {status_string(status)} ({status})")


_lib = None


def lib() -> ctypes.CDLL:
    """Load the in-tree library (built by gemv_layers_amd.build); raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m gemv_layers_amd.build` "
                           "(there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    i64, i32, p, u32 = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p, ctypes.c_uint32
    gemm_sig = [i64, i64, i64, p, i64, p, i64, p, i64, p]
    for name in ("gemm_bf16", "gemm_bf16_noalloc", "gemm_bf16_skinny", "gemm_bf16_tiled", "gemm_bf16_swiglu"):
        getattr(L, name).argtypes = gemm_sig
        getattr(L, name).restype = i32
    L.gemm_init.argtypes = [i32]
    L.gemm_init.restype = i32
    L.gemm_plan_describe.argtypes = [i64, i64, i64, i32, i32, ctypes.c_char_p, i32]
    L.gemm_plan_describe.restype = i32
    L.gemm_wave_efficiency.argtypes = [i64, i64, ctypes.POINTER(ctypes.c_double),
                                       ctypes.POINTER(ctypes.c_int64)]
    L.gemm_wave_efficiency.restype = i32
    L.gemm_last_plan.argtypes = [ctypes.c_char_p, i32]
    L.gemm_last_plan.restype = i32
    L.gemm_status_string.argtypes = [i32]
    L.gemm_status_string.restype = ctypes.c_char_p
    L.gemm_finalize.argtypes = []
    L.gemm_finalize.restype = i32
    L.gemm_peak_mfma_launch.argtypes = [i64, i32, p, p, p]
    L.gemm_peak_mfma_launch.restype = i32
    L.gemm_peak_mfma_data_launch.argtypes = [p, i64, i32, p, p, p]
    L.gemm_peak_mfma_data_launch.restype = i32
    L.gemm_peak_copy_launch.argtypes = [p, p, i64, p]
    L.gemm_peak_copy_launch.restype = i32
    L.gemm_peak_read_launch.argtypes = [p, i64, p, p]
    L.gemm_peak_read_launch.restype = i32
    L.gemm_peak_clock_launch.argtypes = [i64, i32, p, p]
    L.gemm_peak_clock_launch.restype = i32
    L.gemm_peak_xcc_launch.argtypes = [i32, p, p]
    L.gemm_peak_xcc_launch.restype = i32
    L.gemm_peak_empty_launch.argtypes = [p]
    L.gemm_peak_empty_launch.restype = i32
    L.gemm_fill_launch.argtypes = [p, i64, u32, p]
    L.gemm_fill_launch.restype = i32
    L.gemm_mx_packed_sizes.argtypes = [i64, i64, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int64)]
    L.gemm_mx_packed_sizes.restype = i32
    L.gemm_mx_pack_weight.argtypes = [i64, i64, p, i64, p, p, p]
    L.gemm_mx_pack_weight.restype = i32
    L.gemm_mx_quantize_act.argtypes = [i64, i64, p, i64, p, i64, p, i64, p]
    L.gemm_mx_quantize_act.restype = i32
    L.gemm_mx_decode.argtypes = [i64, i64, i64, p, i64, p, i64, p, p, p, i64, p]
    L.gemm_mx_decode.restype = i32
    L.gemm_mx_decode_bf16.argtypes = [i64, i64, i64, p, i64, p, p, p, i64, p]
    L.gemm_mx_decode_bf16.restype = i32
    L.gemm_pack_weight_bf16.argtypes = [i64, i64, p, i64, p, p]
    L.gemm_pack_weight_bf16.restype = i32
    L.gemm_bf16_packed.argtypes = [i64, i64, i64, p, i64, p, p, i64, p]
    L.gemm_bf16_packed.restype = i32
    _lib = L
    return L


def _check(func: str, status: int) -> None:
    if status != GEMM_OK:
        raise GemmError(func, status)


def status_string(status: int) -> str:
    return lib().gemm_status_string(int(status)).decode()


gemm_status_string = status_string


def gemm_init(device: int = 0) -> None:
    _check("gemm_init", lib().gemm_init(int(device)))


def gemm_finalize() -> None:
    _check("gemm_finalize", lib().gemm_finalize())


def _call(name, M, N, K, A, lda, B, ldb, C, ldc, stream):
    st = getattr(lib(), name)(int(M), int(N), int(K), A, int(lda), B, int(ldb), C, int(ldc), stream)
    _check(name, st)


def gemm_bf16(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    """C = A * B on raw device pointers (ints); see include/gemm_bf16.h."""
    _call("gemm_bf16", M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_bf16_noalloc(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    """gemm_bf16 with the library's fixed scratch array as workspace (never allocates)."""
    _call("gemm_bf16_noalloc", M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_bf16_skinny(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    _call("gemm_bf16_skinny", M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_bf16_tiled(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    _call("gemm_bf16_tiled", M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_bf16_swiglu(M, N, K, A, lda, B, ldb, C, ldc, stream=None) -> None:
    """C = silu(A * B[:, :N]) * (A * B[:, N:2N]) on raw device pointers; B is K x 2N."""
    _call("gemm_bf16_swiglu", M, N, K, A, lda, B, ldb, C, ldc, stream)


def gemm_plan_describe(M: int, N: int, K: int, cus: int = 256, skinny: bool = False,
                       swiglu: bool = False, mx: bool = False, packed: bool = False) -> dict:
    buf = ctypes.create_string_buffer(4096)
    flags = ((GEMM_PLAN_SKINNY if skinny else 0) | (GEMM_PLAN_SWIGLU if swiglu else 0)
             | (GEMM_PLAN_MX if mx else 0) | (GEMM_PLAN_PACKED if packed else 0))
    _check("gemm_plan_describe", lib().gemm_plan_describe(M, N, K, cus, flags, buf, 4096))
    return json.loads(buf.value.decode())


def gemm_mx_packed_sizes(N: int, K: int) -> tuple[int, int]:
    """(code bytes, scale bytes) of the packed MXFP4 form of an N x K weight."""
    w, s = ctypes.c_int64(), ctypes.c_int64()
    _check("gemm_mx_packed_sizes", lib().gemm_mx_packed_sizes(N, K, ctypes.byref(w), ctypes.byref(s)))
    return w.value, s.value


def gemm_mx_pack_weight(N, K, W, ldw, Wp, Sp, stream=None) -> None:
    _check("gemm_mx_pack_weight", lib().gemm_mx_pack_weight(N, K, W, ldw, Wp, Sp, stream))


def gemm_mx_quantize_act(M, K, A, lda, Aq, ldaq, As, ldas, stream=None) -> None:
    _check("gemm_mx_quantize_act", lib().gemm_mx_quantize_act(M, K, A, lda, Aq, ldaq, As, ldas, stream))


def gemm_mx_decode(M, N, K, Aq, ldaq, As, ldas, Wp, Sp, C, ldc, stream=None) -> None:
    _check("gemm_mx_decode", lib().gemm_mx_decode(M, N, K, Aq, ldaq, As, ldas, Wp, Sp, C, ldc, stream))


def gemm_mx_decode_bf16(M, N, K, A, lda, Wp, Sp, C, ldc, stream=None) -> None:
    _check("gemm_mx_decode_bf16", lib().gemm_mx_decode_bf16(M, N, K, A, lda, Wp, Sp, C, ldc, stream))


def gemm_pack_weight_bf16(K, N, B, ldb, Bp, stream=None) -> None:
    _check("gemm_pack_weight_bf16", lib().gemm_pack_weight_bf16(K, N, B, ldb, Bp, stream))


def gemm_bf16_packed(M, N, K, A, lda, Bp, C, ldc, stream=None) -> None:
    _check("gemm_bf16_packed", lib().gemm_bf16_packed(M, N, K, A, lda, Bp, C, ldc, stream))


def gemm_wave_efficiency(ctas: int, slots: int):
    eff, waves = ctypes.c_double(), ctypes.c_int64()
    _check("gemm_wave_efficiency", lib().gemm_wave_efficiency(ctas, slots, ctypes.byref(eff),
                                                              ctypes.byref(waves)))
    return eff.value, waves.value


def gemm_last_plan() -> dict:
    buf = ctypes.create_string_buffer(4096)
    _check("gemm_last_plan", lib().gemm_last_plan(buf, 4096))
    return json.loads(buf.value.decode())


def gemm_peak_mfma_launch(iters, blocks, sink, cycles, stream=None) -> None:
    _check("gemm_peak_mfma_launch", lib().gemm_peak_mfma_launch(iters, blocks, sink, cycles, stream))


def gemm_peak_copy_launch(src, dst, nbytes, stream=None) -> None:
    _check("gemm_peak_copy_launch", lib().gemm_peak_copy_launch(src, dst, nbytes, stream))


def gemm_peak_read_launch(src, nbytes, sink, stream=None) -> None:
    _check("gemm_peak_read_launch", lib().gemm_peak_read_launch(src, nbytes, sink, stream))


def gemm_peak_clock_launch(iters, blocks, out, stream=None) -> None:
    _check("gemm_peak_clock_launch", lib().gemm_peak_clock_launch(iters, blocks, out, stream))


def gemm_peak_mfma_data_launch(ops, iters, blocks, sink, cycles, stream=None) -> None:
    _check("gemm_peak_mfma_data_launch",
           lib().gemm_peak_mfma_data_launch(ops, iters, blocks, sink, cycles, stream))


def gemm_peak_xcc_launch(blocks, out, stream=None) -> None:
    _check("gemm_peak_xcc_launch", lib().gemm_peak_xcc_launch(blocks, out, stream))


def gemm_peak_empty_launch(stream=None) -> None:
    _check("gemm_peak_empty_launch", lib().gemm_peak_empty_launch(stream))


def gemm_fill_launch(dst, nbytes, value, stream=None) -> None:
    _check("gemm_fill_launch", lib().gemm_fill_launch(dst, nbytes, value & 0xFFFFFFFF, stream))


# ---- PyTorch marshalling helpers ----------------------------------------------------------

def current_stream_handle():
    import torch

    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


_ENTRY = {"auto": "gemm_bf16", "skinny": "gemm_bf16_skinny", "tiled": "gemm_bf16_tiled"}


def matmul(A, B, out=None, entry: str = "auto", stream=None):
    """C = A @ B for 2-D bf16 CUDA tensors with unit column stride; returns C (bf16)."""
    import torch

    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("A and B must be bfloat16")
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0]:
        raise ValueError("shapes do not form a matrix product")
    if not (A.is_cuda and B.is_cuda):
        raise ValueError("A and B must be device tensors")
    M, K = A.shape
    N = B.shape[1]
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    for t in (A, B, out):
        if t.numel() and t.stride(1) != 1:
            raise ValueError("unit column stride required")
    st = stream if stream is not None else current_stream_handle()
    _call(_ENTRY[entry], M, N, K, ctypes.c_void_p(A.data_ptr()), max(A.stride(0), K),
          ctypes.c_void_p(B.data_ptr()), max(B.stride(0), N), ctypes.c_void_p(out.data_ptr()),
          max(out.stride(0), N), st)
    return out


def swiglu_matmul(A, B, out=None, stream=None):
    """silu(A @ B[:, :N]) * (A @ B[:, N:]) for bf16 CUDA tensors, B of shape (K, 2N): the gate
    and up weights side by side. Returns the (M, N) bf16 result."""
    import torch

    if A.dtype != torch.bfloat16 or B.dtype != torch.bfloat16:
        raise TypeError("A and B must be bfloat16")
    if A.dim() != 2 or B.dim() != 2 or A.shape[1] != B.shape[0] or B.shape[1] % 2:
        raise ValueError("B must be K x 2N for A of shape M x K")
    if not (A.is_cuda and B.is_cuda):
        raise ValueError("A and B must be device tensors")
    M, K = A.shape
    N = B.shape[1] // 2
    if out is None:
        out = torch.empty((M, N), dtype=torch.bfloat16, device=A.device)
    for t in (A, B, out):
        if t.numel() and t.stride(1) != 1:
            raise ValueError("unit column stride required")
    st = stream if stream is not None else current_stream_handle()
    _call("gemm_bf16_swiglu", M, N, K, ctypes.c_void_p(A.data_ptr()), max(A.stride(0), K),
          ctypes.c_void_p(B.data_ptr()), max(B.stride(0), 2 * N), ctypes.c_void_p(out.data_ptr()),
          max(out.stride(0), N), st)
    return out
