"""Python access to the float64 CPU oracle (oracle.c).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check and by the
benchmark's CPU-baseline leg, never by the GPU library or its binding. See oracle.c for what
is computed and which passages it follows.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc into oracle/liboracle.so (plain C, no GPU code)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-Wall", "-Wextra",
               "-fno-fast-math", "-ffp-contract=off", "-o", tmp, _SRC, "-lm", "-lpthread"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


class CheckResult(ctypes.Structure):
    _fields_ = [
        ("checked", ctypes.c_int64),
        ("failures", ctypes.c_int64),
        ("nonfinite", ctypes.c_int64),
        ("worst_row", ctypes.c_int64),
        ("worst_col", ctypes.c_int64),
        ("worst_ratio", ctypes.c_double),
        ("err_sq", ctypes.c_double),
        ("ref_sq", ctypes.c_double),
    ]

    @property
    def rel_frob(self) -> float:
        if self.ref_sq == 0.0:
            return 0.0 if self.err_sq == 0.0 else float("inf")
        return float(np.sqrt(self.err_sq / self.ref_sq))

    @property
    def ok(self) -> bool:
        return self.failures == 0 and self.rel_frob <= REL_FROB_MAX

    def summary(self) -> dict:
        return {"checked": self.checked, "failures": self.failures,
                "nonfinite": self.nonfinite, "worst_ratio": self.worst_ratio,
                "worst_at": [self.worst_row, self.worst_col], "rel_frob": self.rel_frob}


REL_FROB_MAX = 4e-3


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        L = ctypes.CDLL(_LIB)
        i64, p = ctypes.c_int64, ctypes.c_void_p
        L.oracle_version.restype = ctypes.c_int
        L.oracle_bf16_rne.argtypes = [ctypes.c_double]
        L.oracle_bf16_rne.restype = ctypes.c_uint16
        L.oracle_bf16_to_f64.argtypes = [ctypes.c_uint16]
        L.oracle_bf16_to_f64.restype = ctypes.c_double
        L.oracle_gemm_rows.argtypes = [i64, i64, i64, i64, p, i64, p, i64, p, p, i64, ctypes.c_int]
        L.oracle_gemm_rows.restype = ctypes.c_int
        L.oracle_gemm.argtypes = [i64, i64, i64, p, i64, p, i64, p, p, i64, ctypes.c_int]
        L.oracle_gemm.restype = ctypes.c_int
        L.oracle_gemm_entries.argtypes = [i64, p, i64, p, i64, p, p, i64, p, p]
        L.oracle_gemm_entries.restype = ctypes.c_int
        L.oracle_check.argtypes = [i64, i64, p, i64, p, p, i64, ctypes.POINTER(CheckResult)]
        L.oracle_check.restype = ctypes.c_int
        L.oracle_bf16_rne_array.argtypes = [p, p, i64]
        L.oracle_bf16_rne_array.restype = None
        L.oracle_bf16_to_f64_array.argtypes = [p, p, i64]
        L.oracle_bf16_to_f64_array.restype = None
        _lib = L
    return _lib


def default_threads() -> int:
    """Host threads for the oracle: the cores this process may run on, at most 16."""
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _u16(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x)
    if x.dtype != np.uint16 or x.ndim != 2 or (x.size and x.strides[1] != 2):
        raise ValueError("expected a 2-D uint16 (bf16 bits) array with unit column stride")
    return x


def _ptr(x: np.ndarray):
    return ctypes.c_void_p(x.ctypes.data)


def gemm(A: np.ndarray, B: np.ndarray, M: int | None = None, N: int | None = None,
         K: int | None = None, with_abs: bool = True, threads: int | None = None):
    """float64 (ref, sabs) for C = A[:M, :K] @ B[:K, :N]; A and B are bf16 bit arrays."""
    A, B = _u16(A), _u16(B)
    M = A.shape[0] if M is None else M
    K = A.shape[1] if K is None else K
    N = B.shape[1] if N is None else N
    return gemm_rows(A, B, 0, M, N, K, with_abs, threads)


def gemm_rows(A: np.ndarray, B: np.ndarray, row0: int, nrows: int, N: int, K: int,
              with_abs: bool = True, threads: int | None = None):
    A, B = _u16(A), _u16(B)
    if row0 < 0 or row0 + nrows > A.shape[0] or K > A.shape[1] or K > B.shape[0] or N > B.shape[1]:
        raise ValueError("row range or K/N out of the operand bounds")
    ref = np.empty((nrows, N), dtype=np.float64)
    sabs = np.empty((nrows, N), dtype=np.float64) if with_abs else None
    rc = lib().oracle_gemm_rows(row0, nrows, N, K, _ptr(A), A.strides[0] // 2, _ptr(B),
                                B.strides[0] // 2, _ptr(ref),
                                _ptr(sabs) if sabs is not None else None, N,
                                threads or default_threads())
    if rc != 0:
        raise ValueError("oracle_gemm_rows rejected its arguments")
    return ref, sabs


def gemm_entries(A: np.ndarray, B: np.ndarray, rows, cols, K: int | None = None):
    """float64 (ref, sabs) of the single entries (rows[t], cols[t])."""
    A, B = _u16(A), _u16(B)
    K = A.shape[1] if K is None else K
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    cols = np.ascontiguousarray(cols, dtype=np.int64)
    if rows.shape != cols.shape or rows.ndim != 1:
        raise ValueError("rows and cols must be 1-D of equal length")
    if len(rows) and (rows.min() < 0 or rows.max() >= A.shape[0] or cols.min() < 0
                      or cols.max() >= B.shape[1]):
        raise ValueError("entry index out of bounds")
    ref = np.empty(len(rows), dtype=np.float64)
    sabs = np.empty(len(rows), dtype=np.float64)
    lib().oracle_gemm_entries(K, _ptr(A), A.strides[0] // 2, _ptr(B), B.strides[0] // 2,
                              _ptr(rows), _ptr(cols), len(rows), _ptr(ref), _ptr(sabs))
    return ref, sabs


def check(C: np.ndarray, ref: np.ndarray, sabs: np.ndarray) -> CheckResult:
    """Element-wise bound and relative Frobenius check of bf16 bits C against (ref, sabs)."""
    C = np.asarray(C)
    if C.ndim == 1:
        C = C.reshape(1, -1)
        ref = np.asarray(ref).reshape(1, -1)
        sabs = np.asarray(sabs).reshape(1, -1)
    C = _u16(C)
    ref = np.ascontiguousarray(ref, dtype=np.float64)
    sabs = np.ascontiguousarray(sabs, dtype=np.float64)
    M, N = ref.shape
    if C.shape[0] < M or C.shape[1] < N or sabs.shape != ref.shape:
        raise ValueError("shape mismatch")
    res = CheckResult()
    lib().oracle_check(M, N, _ptr(C), C.strides[0] // 2, _ptr(ref), _ptr(sabs), N,
                       ctypes.byref(res))
    return res


def bf16_rne(x) -> np.ndarray:
    """float64 -> bf16 bits (nearest, ties to even), element by element through the oracle."""
    a = np.ascontiguousarray(x, dtype=np.float64)
    out = np.empty(a.shape, dtype=np.uint16)
    lib().oracle_bf16_rne_array(_ptr(a), _ptr(out), a.size)
    return out


def bf16_to_f64(h) -> np.ndarray:
    """Exact widening of bf16 bits, through the oracle's own conversion."""
    a = np.ascontiguousarray(h, dtype=np.uint16)
    out = np.empty(a.shape, dtype=np.float64)
    lib().oracle_bf16_to_f64_array(_ptr(a), _ptr(out), a.size)
    return out


@dataclass
class Expected:
    """Oracle output for a (possibly row-sampled) problem."""
    rows: np.ndarray   # which matrix rows ref/sabs hold
    ref: np.ndarray
    sabs: np.ndarray
