"""Pins for the float64 oracle, independent of the oracle's own code.

Each test pins the oracle to something other than itself: closed forms (all-ones gives C = K),
exact algebra (identity, permutation, rank-1), exhaustive integer brute force in Python's exact
integers, numpy's float64 matmul as an independent library witness, torch's float32 -> bfloat16
conversion as a witness for the rounding helper, printed tie cases, and negative cases for the
acceptance check. A plausible slip in the oracle (a dropped term, a transposed operand, a wrong
leading dimension, a missing |.|, a wrong rounding direction) fails at least one of them.
"""

import os

import numpy as np
import pytest

import oracle
from synth import matrix, integer_bf16, normal_bf16, bf16_bits_to_f32, f32_to_bf16_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def widen(h):
    """Independent exact widening used by the tests (numpy bit shift)."""
    return bf16_bits_to_f32(h).astype(np.float64)


# --- rounding helper -----------------------------------------------------------------------

def _rne_rows():
    rows = []
    with open(os.path.join(GOLDEN, "rne_ties.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            parts = line.split()
            rows.append((float(parts[0]), int(parts[1], 16)))
    return rows


def test_rne_golden_ties(oracle_lib):
    rows = _rne_rows()
    assert len(rows) >= 15
    got = oracle.bf16_rne([r[0] for r in rows])
    for (x, want), g in zip(rows, got):
        assert int(g) == want, f"bf16_rne({x!r}) = {int(g):#06x}, want {want:#06x}"


def test_rne_matches_torch_on_float32_values(oracle_lib):
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    # float32 values (so double -> bf16 and float -> bf16 agree), many exponents, plus exact
    # ties built by setting the low 16 bits to 0x8000.
    bits = rng.integers(0, 2**32, size=200000, dtype=np.uint64).astype(np.uint32)
    exp = (bits >> 23) & 0xFF
    bits = bits[(exp != 0xFF)]                     # no NaN/Inf
    ties = (bits & np.uint32(0xFFFF0000)) | np.uint32(0x8000)
    allbits = np.concatenate([bits, ties]).astype(np.uint32)
    x = allbits.view(np.float32)
    want = torch.from_numpy(x.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.bf16_rne(x.astype(np.float64))
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} mismatches, first x={x[bad[0]]!r}"


def test_widen_is_exact(oracle_lib):
    h = np.arange(0, 65536, dtype=np.uint32).astype(np.uint16)
    exp = (h >> 7) & 0xFF
    h = h[exp != 0xFF]
    np.testing.assert_array_equal(oracle.bf16_to_f64(h), widen(h))


# --- closed forms and exact algebra -----------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(3, 5, 7), (17, 33, 512), (2, 3, 11008), (1, 1, 16384)])
def test_all_ones_gives_K(oracle_lib, M, N, K):
    A = matrix("ones", M, K)
    B = matrix("ones", K, N)
    ref, sabs = oracle.gemm(A, B)
    assert np.all(ref == K) and np.all(sabs == K)


def test_identity_and_permutation_are_exact(oracle_lib):
    n = 48
    A = matrix("normal", 37, n, seed=11)
    I = f32_to_bf16_bits(np.eye(n, dtype=np.float32))
    ref, _ = oracle.gemm(A, I)
    np.testing.assert_array_equal(oracle.bf16_rne(ref), A)
    perm = np.random.default_rng(5).permutation(n)
    P = f32_to_bf16_bits(np.eye(n, dtype=np.float32)[:, perm])  # column j of P is e_perm[j]
    ref, _ = oracle.gemm(A, P)
    np.testing.assert_array_equal(oracle.bf16_rne(ref), A[:, perm])
    # left multiplication: P^T A permutes rows
    Bm = matrix("normal", n, 29, seed=12)
    ref, _ = oracle.gemm(f32_to_bf16_bits(np.eye(n, dtype=np.float32)[perm, :]), Bm)
    np.testing.assert_array_equal(oracle.bf16_rne(ref), Bm[perm, :])


def test_rank_one_outer_product(oracle_lib):
    # A = u x^T, B = y v^T  =>  C = (x . y) u v^T, exact with small powers of two / integers.
    rng = np.random.default_rng(3)
    M, N, K = 19, 23, 40
    u = rng.choice([-2.0, -1.0, 0.5, 1.0, 4.0], size=M)
    v = rng.choice([-1.0, 0.25, 1.0, 2.0], size=N)
    x = rng.integers(-3, 4, size=K).astype(np.float64)
    y = rng.integers(-3, 4, size=K).astype(np.float64)
    A = f32_to_bf16_bits(np.outer(u, x).astype(np.float32))
    B = f32_to_bf16_bits(np.outer(y, v).astype(np.float32))
    ref, sabs = oracle.gemm(A, B)
    np.testing.assert_array_equal(ref, float(x @ y) * np.outer(u, v))
    np.testing.assert_array_equal(sabs, float(np.abs(x) @ np.abs(y)) * np.abs(np.outer(u, v)))


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (2, 3, 5), (8, 16, 17), (5, 31, 33), (3, 64, 2)])
def test_integer_brute_force(oracle_lib, M, N, K):
    A = matrix("int", M, K, seed=100 + K)
    B = matrix("int", K, N, seed=200 + N)
    a = widen(A).astype(np.int64).tolist()
    b = widen(B).astype(np.int64).tolist()
    want = [[sum(a[i][k] * b[k][j] for k in range(K)) for j in range(N)] for i in range(M)]
    wabs = [[sum(abs(a[i][k] * b[k][j]) for k in range(K)) for j in range(N)] for i in range(M)]
    ref, sabs = oracle.gemm(A, B)
    assert ref.tolist() == [[float(v) for v in r] for r in want]
    assert sabs.tolist() == [[float(v) for v in r] for r in wabs]


@pytest.mark.parametrize("M,N,K", [(64, 80, 96), (33, 257, 300)])
def test_against_numpy_float64(oracle_lib, M, N, K):
    A = matrix("normal", M, K, seed=7)
    B = matrix("normal", K, N, seed=8, sigma=0.02)
    a, b = widen(A), widen(B)
    ref, sabs = oracle.gemm(A, B)
    want = a @ b
    wabs = np.abs(a) @ np.abs(b)
    tol = (K + 1) * 2.0 ** -52 * wabs
    assert np.all(np.abs(ref - want) <= tol)
    assert np.all(np.abs(sabs - wabs) <= tol)
    # a transposed operand or a dropped |.| would be far outside this tolerance
    assert np.max(np.abs(sabs - np.abs(want))) > 0  # sabs is not |ref|


def test_leading_dimensions_and_row_ranges(oracle_lib):
    M, N, K = 21, 30, 45
    A = matrix("normal", M, K, seed=21, ld=K + 7)
    B = matrix("normal", K, N, seed=22, ld=N + 3)
    ref, sabs = oracle.gemm(A, B, M=M, N=N, K=K)
    a, b = widen(A[:, :K]), widen(B[:, :N])
    assert np.all(np.isfinite(ref))          # padding holds NaN, so reading it would show
    np.testing.assert_allclose(ref, a @ b, rtol=0, atol=1e-9)
    r2, s2 = oracle.gemm_rows(A, B, 5, 9, N, K)
    np.testing.assert_array_equal(r2, ref[5:14])
    np.testing.assert_array_equal(s2, sabs[5:14])
    rows = np.array([0, 20, 7, 13])
    cols = np.array([29, 0, 15, 3])
    re, se = oracle.gemm_entries(A, B, rows, cols, K=K)
    np.testing.assert_array_equal(re, ref[rows, cols])
    np.testing.assert_array_equal(se, sabs[rows, cols])


def test_K_zero_gives_zero(oracle_lib):
    A = np.zeros((4, 0), dtype=np.uint16)
    B = np.zeros((0, 6), dtype=np.uint16)
    ref, sabs = oracle.gemm(A, B, M=4, N=6, K=0)
    assert np.all(ref == 0) and np.all(sabs == 0)


def test_statistical_scale(oracle_lib):
    K = 4096
    A = matrix("normal", 64, K, seed=31)
    B = matrix("normal", K, 64, seed=32)
    ref, _ = oracle.gemm(A, B)
    # entries of a product of independent N(0,1) vectors have variance K
    assert abs(ref.std() / np.sqrt(K) - 1.0) < 0.05


# --- the acceptance check, with negative cases first ------------------------------------------

def _exact_case():
    M, N, K = 64, 96, 1024
    A = matrix("normal", M, K, seed=41)
    B = matrix("normal", K, N, seed=42)
    ref, sabs = oracle.gemm(A, B)
    return ref, sabs


def test_check_rejects_truncation(oracle_lib):
    ref, sabs = _exact_case()
    # truncation toward zero of the float32-rounded value: drops the low 16 bits
    f32 = ref.astype(np.float32)
    trunc = (f32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    res = oracle.check(trunc, ref, sabs)
    assert res.failures > 0 and not res.ok


def test_check_rejects_single_perturbation_and_nan(oracle_lib):
    ref, sabs = _exact_case()
    good = oracle.bf16_rne(ref)
    assert oracle.check(good, ref, sabs).ok
    bad = good.copy()
    bad[10, 20] ^= np.uint16(0x0004)      # a few ulps off in one element
    r = oracle.check(bad, ref, sabs)
    assert r.failures == 1 and (r.worst_row, r.worst_col) == (10, 20)
    bad = good.copy()
    bad[3, 4] = 0x7FC0
    r = oracle.check(bad, ref, sabs)
    assert r.nonfinite == 1 and not r.ok
    bad = good.copy()
    bad[5, 6] = 0x7F80                    # +Inf
    assert not oracle.check(bad, ref, sabs).ok


def test_check_accepts_float32_accumulation_in_any_order(oracle_lib):
    ref, sabs = _exact_case()
    M, N, K = 64, 96, 1024
    A = matrix("normal", M, K, seed=41)
    B = matrix("normal", K, N, seed=42)
    a = widen(A).astype(np.float32)
    b = widen(B).astype(np.float32)
    # sequential float32 sum, and a reversed-order float32 sum, both rounded to bf16
    acc = np.zeros((M, N), dtype=np.float32)
    for k in range(K):
        acc += np.outer(a[:, k], b[k, :])
    assert oracle.check(f32_to_bf16_bits(acc), ref, sabs).ok
    acc = np.zeros((M, N), dtype=np.float32)
    for k in reversed(range(K)):
        acc += np.outer(a[:, k], b[k, :])
    assert oracle.check(f32_to_bf16_bits(acc), ref, sabs).ok


def test_check_rel_frobenius_bound(oracle_lib):
    ref, sabs = _exact_case()
    # scale every element by (1 + 5e-3): within nothing element-wise, and Frobenius > 4e-3
    scaled = oracle.bf16_rne(ref * (1 + 5e-3))
    assert oracle.check(scaled, ref, sabs).rel_frob > 4e-3


# --- the value-only branch (no sum of |a b|) ----------------------------------------------------
# The bit-exact GPU checks take their expected bits from oracle.gemm(..., with_abs=False), which
# runs a loop of its own in oracle.c. It is pinned here like the other branch: exact integer brute
# force with ragged shapes and leading dimensions, closed forms, numpy's float64 product, and bit
# equality with the pinned with_abs=True branch (both add the K products of an element in
# ascending k, so the bits must agree).

@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 7, 5), (9, 17, 33), (5, 31, 64), (2, 65, 3), (13, 8, 129)])
def test_value_only_integer_brute_force(oracle_lib, M, N, K):
    A = matrix("int", M, K, seed=300 + K, ld=K + 3)
    B = matrix("int", K, N, seed=400 + N, ld=N + 5)
    a = widen(A[:, :K]).astype(np.int64).tolist()
    b = widen(B[:, :N]).astype(np.int64).tolist()
    want = [[float(sum(a[i][k] * b[k][j] for k in range(K))) for j in range(N)] for i in range(M)]
    ref, sabs = oracle.gemm(A, B, M=M, N=N, K=K, with_abs=False)
    assert sabs is None
    assert ref.tolist() == want


def test_value_only_closed_forms(oracle_lib):
    for (M, N, K) in ((3, 5, 7), (2, 9, 11008), (1, 4, 16384)):
        ref, _ = oracle.gemm(matrix("ones", M, K), matrix("ones", K, N), with_abs=False)
        assert np.all(ref == K)
    n = 40
    A = matrix("normal", 23, n, seed=31)
    perm = np.random.default_rng(9).permutation(n)
    ref, _ = oracle.gemm(A, f32_to_bf16_bits(np.eye(n, dtype=np.float32)), with_abs=False)
    np.testing.assert_array_equal(oracle.bf16_rne(ref), A)
    ref, _ = oracle.gemm(A, f32_to_bf16_bits(np.eye(n, dtype=np.float32)[:, perm]), with_abs=False)
    np.testing.assert_array_equal(oracle.bf16_rne(ref), A[:, perm])
    Bm = matrix("normal", n, 19, seed=32)
    ref, _ = oracle.gemm(f32_to_bf16_bits(np.eye(n, dtype=np.float32)[perm, :]), Bm, with_abs=False)
    np.testing.assert_array_equal(oracle.bf16_rne(ref), Bm[perm, :])


@pytest.mark.parametrize("M,N,K", [(64, 80, 96), (33, 257, 300), (7, 1000, 1031)])
def test_value_only_matches_numpy_and_the_pinned_branch(oracle_lib, M, N, K):
    A = matrix("normal", M, K, seed=41, ld=K + 8)
    B = matrix("normal", K, N, seed=42, sigma=0.02, ld=N + 8)
    ref0, _ = oracle.gemm(A, B, M=M, N=N, K=K, with_abs=False)
    ref1, sabs = oracle.gemm(A, B, M=M, N=N, K=K, with_abs=True)
    np.testing.assert_array_equal(ref0, ref1)          # same bits as the pinned branch
    want = widen(A[:, :K]) @ widen(B[:, :N])
    assert np.all(np.abs(ref0 - want) <= (K + 1) * 2.0 ** -52 * sabs)
    # row ranges of the value-only branch land on the same rows
    r2, s2 = oracle.gemm_rows(A, B, 3, 4, N, K, with_abs=False)
    assert s2 is None
    np.testing.assert_array_equal(r2, ref0[3:7])
    # and integer inputs round to the exact bf16 of the exact integer sum
    Ai = matrix("int", M, K, seed=43)
    Bi = matrix("int", K, N, seed=44)
    ri, _ = oracle.gemm(Ai, Bi, with_abs=False)
    exact = widen(Ai).astype(np.int64) @ widen(Bi).astype(np.int64)
    np.testing.assert_array_equal(ri, exact.astype(np.float64))
    np.testing.assert_array_equal(oracle.bf16_rne(ri), f32_to_bf16_bits(exact.astype(np.float32)))
