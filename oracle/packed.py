"""Oracle for the packed bf16 weight layout of the decode product (CPU, exact byte work).

TEST INFRASTRUCTURE ONLY: imported by the tests, never by the GPU library or its binding.

A decode product streams a weight B (K x N, bf16, row-major) that does not change between calls,
so it can be stored once in the order the product consumes it (spark-kernels post, "the decode
kernel": the decode GEMM is a stream of weight bytes, read once). The packed layout: column tile
t holds columns n = 16 t .. 16 t + 15 and k-step s holds rows k = 32 s .. 32 s + 31. The 512
elements of (t, s) are one 1024-byte block at byte 1024 (t * KS + s), KS = K / 32, in which
lane l (0 .. 63) owns bytes 16 l .. 16 l + 15: the 8 elements B[32 s + 8 (l // 16) + j][16 t + l % 16],
j = 0 .. 7, in order. The product itself is the plain one (oracle.gemm on the unpacked B).
"""

from __future__ import annotations

import numpy as np


def packed_bytes(K: int, N: int) -> int:
    return K * N * 2


def pack(B: np.ndarray, K: int | None = None, N: int | None = None) -> np.ndarray:
    """The packed uint16 array (K * N elements) of the K x N bf16 bit matrix B[:K, :N]."""
    B = np.asarray(B, dtype=np.uint16)
    K = B.shape[0] if K is None else K
    N = B.shape[1] if N is None else N
    if K % 32 or N % 16:
        raise ValueError("K must be a multiple of 32 and N of 16")
    b = B[:K, :N].reshape(K // 32, 4, 8, N // 16, 16)        # [s, g, j, t, i]
    return np.ascontiguousarray(b.transpose(3, 0, 1, 4, 2)).reshape(-1)  # [t, s, g, i, j]


def unpack(P: np.ndarray, K: int, N: int) -> np.ndarray:
    """Inverse of pack."""
    p = np.asarray(P, dtype=np.uint16)[: K * N].reshape(N // 16, K // 32, 4, 16, 8)  # [t, s, g, i, j]
    return np.ascontiguousarray(p.transpose(1, 2, 4, 0, 3)).reshape(K, N)
