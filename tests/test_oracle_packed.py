"""Pins for the packed bf16 weight layout (oracle/packed.py): a term-by-term reading of the
definition on a small case, the round trip, and that every element appears exactly once."""

import numpy as np

from oracle import packed


def test_layout_term_by_term():
    K, N = 96, 48
    B = np.arange(K * N, dtype=np.uint32).astype(np.uint16).reshape(K, N)
    P = packed.pack(B)
    assert P.size == K * N and packed.packed_bytes(K, N) == 2 * K * N
    ks = K // 32
    for t in range(N // 16):
        for s in range(ks):
            for lane in range(64):
                for j in range(8):
                    e = 512 * (t * ks + s) + 8 * lane + j
                    assert P[e] == B[32 * s + 8 * (lane // 16) + j, 16 * t + lane % 16]


def test_round_trip_and_permutation():
    rng = np.random.default_rng(4)
    K, N = 4096, 64
    B = rng.integers(0, 65536, size=(K, N), dtype=np.uint16)
    P = packed.pack(B)
    assert np.array_equal(packed.unpack(P, K, N), B)
    # every position of B lands in exactly one place
    lab = (np.arange(K * N) % 65521).astype(np.uint16).reshape(K, N)
    assert np.array_equal(np.sort(packed.pack(lab)), np.sort(lab.reshape(-1)))
