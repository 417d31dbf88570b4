"""Pins for the SwiGLU oracle (oracle/swiglu.py), independent of the oracle's own code.

SiLU is pinned to closed forms (sigmoid(ln 3) = 3/4, sigmoid(ln 2) = 2/3), to the identity
silu(x) - silu(-x) = x, to torch's float64 silu as a library witness, and to its saturation.
The slope bound is pinned by finite differences. The fused value is pinned by brute force over
Python's exact integers and math.exp on tiny inputs, which catches swapped halves, a dropped
factor or a shifted column. The acceptance bound must pass a float32 model of the fused kernel
(float32 products, float32 silu, one bf16 rounding) and must reject: an unfused path that rounds
g and u to bf16 first, sigmoid for silu, a missing activation, silu of the wrong half, and an up
column off by one.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import swiglu as sw
from synth import bf16_bits_to_f32, f32_to_bf16_bits, matrix


def widen(h):
    return bf16_bits_to_f32(h).astype(np.float64)


# --- silu ------------------------------------------------------------------------------------

def test_silu_closed_forms():
    l3, l2 = math.log(3.0), math.log(2.0)
    got = sw.silu([0.0, l3, -l3, l2, -l2])
    want = [0.0, 0.75 * l3, -0.25 * l3, 2.0 / 3.0 * l2, -1.0 / 3.0 * l2]
    assert np.allclose(got, want, rtol=1e-15, atol=0)
    assert got[0] == 0.0


def test_silu_odd_part_identity():
    x = np.linspace(-30, 30, 6001)
    assert np.allclose(sw.silu(x) - sw.silu(-x), x, rtol=1e-14, atol=1e-14)


def test_silu_matches_torch_float64():
    torch = pytest.importorskip("torch")
    x = np.concatenate([np.linspace(-40, 40, 80001), np.random.default_rng(3).normal(0, 5, 10000)])
    want = torch.nn.functional.silu(torch.from_numpy(x)).numpy()
    assert np.allclose(sw.silu(x), want, rtol=1e-14, atol=1e-300)


def test_silu_saturates_without_nan():
    got = sw.silu([800.0, -800.0, 1e308, -1e308])
    assert got[0] == 800.0 and got[2] == 1e308
    assert got[1] == 0.0 and got[3] == 0.0
    assert np.isfinite(got).all()


def test_silu_slope_bound():
    x = np.linspace(-20, 20, 400001)
    h = 1e-6
    slope = (sw.silu(x + h) - sw.silu(x - h)) / (2 * h)
    assert slope.max() <= sw.SILU_SLOPE_MAX
    assert slope.max() > 1.099          # the bound is not loose: the peak is 1.09984
    assert slope.min() > -0.1 and slope.min() < -0.099
    assert abs(x[np.argmax(slope)] - 2.3994) < 1e-3


# --- the fused value --------------------------------------------------------------------------

def _brute(A, B, N, K):
    """h by exact integer sums and math.exp: silu(g) * u, g from columns 0..N-1, u from N..2N-1."""
    a, b = widen(A), widen(B)
    M = A.shape[0]
    out = np.empty((M, N))
    for i in range(M):
        for j in range(N):
            gi = sum(int(a[i, k]) * int(b[k, j]) for k in range(K))
            ui = sum(int(a[i, k]) * int(b[k, N + j]) for k in range(K))
            out[i, j] = gi / (1.0 + math.exp(-gi)) * ui if gi > -700 else 0.0 * ui
    return out


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (4, 9, 16)])
def test_fused_value_brute_force(oracle_lib, M, N, K):
    A = matrix("int", M, K, seed=11 + M, radius=3)
    B = matrix("int", K, 2 * N, seed=12 + N, radius=3)
    h, slack = sw.swiglu(A, B, M, N, K, threads=1)
    assert h.shape == (M, N) and slack.shape == (M, N)
    assert np.allclose(h, _brute(A, B, N, K), rtol=1e-14, atol=0)
    assert (slack >= 0).all()


def test_fused_value_with_leading_dimension(oracle_lib):
    M, N, K = 5, 6, 8
    A = matrix("int", M, K, seed=21, radius=2, ld=K + 3)
    B = matrix("int", K, 2 * N, seed=22, radius=2, ld=2 * N + 5)  # NaN padding past 2N
    h, _ = sw.swiglu(A, B, M, N, K, threads=1)
    assert np.allclose(h, _brute(A[:, :K], B[:, : 2 * N], N, K), rtol=1e-14, atol=0)


def test_rows_match_whole(oracle_lib):
    M, N, K = 9, 7, 24
    A = matrix("normal", M, K, seed=31)
    B = matrix("normal", K, 2 * N, seed=32, sigma=0.1)
    h, s = sw.swiglu(A, B, M, N, K)
    h2, s2 = sw.swiglu_rows(A, B, 4, 3, N, K)
    assert np.array_equal(h[4:7], h2) and np.array_equal(s[4:7], s2)


def test_k_zero_is_exact_zero(oracle_lib):
    A = np.zeros((2, 0), dtype=np.uint16)
    B = np.zeros((0, 6), dtype=np.uint16)
    h, slack = sw.swiglu(A, B, 2, 3, 0)
    assert (h == 0).all() and (slack == 0).all()
    assert sw.check(np.zeros((2, 3), dtype=np.uint16), h, slack).ok
    assert not sw.check(np.full((2, 3), 0x3F80, dtype=np.uint16), h, slack).ok


# --- the acceptance bound ---------------------------------------------------------------------

def _operands(M=64, N=512, K=4096, seed=41):
    A = matrix("normal", M, K, seed=seed)
    B = matrix("normal", K, 2 * N, seed=seed + 1, sigma=0.02)
    return A, B


def _f32_products(A, B, N):
    a = bf16_bits_to_f32(A)
    b = bf16_bits_to_f32(B)
    return a @ b[:, :N], a @ b[:, N:]  # float32 accumulation, library order


def _silu32(x):
    x = x.astype(np.float32)
    with np.errstate(over="ignore"):
        return (x / (np.float32(1) + np.exp(-x))).astype(np.float32)


@pytest.fixture(scope="module")
def problem(oracle_lib):
    A, B = _operands()
    M, N, K = A.shape[0], B.shape[1] // 2, A.shape[1]
    h, slack = sw.swiglu(A, B, M, N, K)
    g32, u32 = _f32_products(A, B, N)
    return A, B, h, slack, g32, u32


def test_fused_float32_model_passes(problem):
    _, _, h, slack, g32, u32 = problem
    c = f32_to_bf16_bits((_silu32(g32) * u32).astype(np.float32))
    res = sw.check(c, h, slack)
    assert res.ok, res.summary()


def test_unfused_bf16_intermediates_fail(problem):
    _, _, h, slack, g32, u32 = problem
    gb = bf16_bits_to_f32(f32_to_bf16_bits(g32))
    ub = bf16_bits_to_f32(f32_to_bf16_bits(u32))
    c = f32_to_bf16_bits((_silu32(gb) * ub).astype(np.float32))
    res = sw.check(c, h, slack)
    assert not res.ok and res.failures > 10, res.summary()


@pytest.mark.parametrize("mistake", ["sigmoid", "no_activation", "silu_of_up", "up_shifted"])
def test_planted_mistakes_fail(problem, mistake):
    _, _, h, slack, g32, u32 = problem
    if mistake == "sigmoid":
        v = g32 * 0 + (1 / (1 + np.exp(-g32))) * u32
    elif mistake == "no_activation":
        v = g32 * u32
    elif mistake == "silu_of_up":
        v = _silu32(u32) * g32
    else:
        v = _silu32(g32) * np.roll(u32, -1, axis=1)
    res = sw.check(f32_to_bf16_bits(v.astype(np.float32)), h, slack)
    assert not res.ok, (mistake, res.summary())


def test_nonfinite_fails(problem):
    _, _, h, slack, g32, u32 = problem
    c = f32_to_bf16_bits((_silu32(g32) * u32).astype(np.float32))
    c[3, 5] = 0x7FC0
    res = sw.check(c, h, slack)
    assert not res.ok and res.nonfinite == 1
