"""Pins for the MX oracle (oracle/mx.py), independent of the oracle's own code.

The element formats are pinned to the OCP MX tables (the E2M1 magnitudes) and to torch's
float8_e4m3fn and float8_e8m0fnu decoders for every code. Element rounding is pinned to torch's
float32 -> float8_e4m3fn cast (nearest even) inside the range, to a brute-force nearest-even
search over the E2M1 table, and to saturation outside it. Block conversion is pinned by hand
cases (shared exponent, saturation, ties, all-zero blocks, signed zeros) and by the round trip
(requantising dequantised values returns the same bytes). The product is pinned to the bf16
product oracle on the dequantised operands (exact in bf16), and the packed layout to a
term-by-term reading of its definition. The acceptance check must pass a float32 model of the
kernel and reject a dropped block scale, a shifted scale index and swapped nibbles.
"""

import math

import numpy as np
import pytest

import oracle
from oracle import mx
from synth import bf16_bits_to_f32, f32_to_bf16_bits, matrix

torch = pytest.importorskip("torch")


def test_e2m1_table():
    assert mx.value_table("e2m1").tolist() == [0, 0.5, 1, 1.5, 2, 3, 4, 6,
                                               -0.0, -0.5, -1, -1.5, -2, -3, -4, -6]


def test_e4m3_table_matches_torch():
    want = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).float().double().numpy()
    got = mx.value_table("e4m3")
    assert np.array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert np.array_equal(got[ok], want[ok])
    assert got[0x7E] == 448 and got[0x08] == 2.0 ** -6 and got[0x01] == 2.0 ** -9 and got[0x38] == 1


def test_e8m0_matches_torch():
    want = torch.arange(256, dtype=torch.uint8).view(torch.float8_e8m0fnu).float().double().numpy()
    got = np.array([mx.scale_value(e) for e in range(256)])
    assert np.isnan(got[255]) and np.isnan(want[255])
    # torch decodes through float32, which has no 2^-127; compare the rest exactly
    assert np.array_equal(got[1:255], want[1:255])
    assert got[0] == 2.0 ** -127


def test_e4m3_rounding_matches_torch_in_range():
    rng = np.random.default_rng(5)
    x = np.concatenate([rng.normal(0, 50, 20000), rng.normal(0, 0.01, 20000),
                        rng.uniform(-447.9, 447.9, 20000)]).astype(np.float32)
    # exact ties of the E4M3 grid, normal and subnormal
    t = mx.value_table("e4m3")
    grid = np.unique(np.abs(t[~np.isnan(t)]))
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)
    x = np.concatenate([x, mids, -mids])
    want = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = mx.encode_array(x.astype(np.float64), "e4m3")
    assert np.array_equal(got, want)
    assert all(mx.encode_element(float(v), "e4m3") == w for v, w in zip(x[:500], want[:500]))


def test_saturation():
    assert mx.encode_element(500.0, "e4m3") == 0x7E and mx.encode_element(-1e9, "e4m3") == 0xFE
    assert mx.encode_element(464.0, "e4m3") == 0x7E
    assert mx.encode_element(7.0, "e2m1") == 0x7 and mx.encode_element(-100.0, "e2m1") == 0xF


def _nearest_even_e2m1(x):
    t = mx.value_table("e2m1")[:8]
    a = min(abs(x), 6.0)
    d = np.abs(t - a)
    best = np.flatnonzero(d == d.min())
    code = int(best[0]) if len(best) == 1 else int([c for c in best if c % 2 == 0][0])
    return code | (8 if math.copysign(1.0, x) < 0 else 0)


def test_e2m1_rounding_brute_force():
    xs = [k / 16 for k in range(-130, 131)] + [6.5, -7.99, 5.0, -5.0, 2.5, 0.25, -0.25, 0.75]
    for x in xs:
        want = _nearest_even_e2m1(x)
        assert mx.encode_element(x, "e2m1") == want, x
        assert mx.encode_array(np.array([x]), "e2m1")[0] == want, x


def _bf16(vals):
    return f32_to_bf16_bits(np.asarray(vals, dtype=np.float32))


def test_block_conversion_hand_cases():
    # 1 .. 32: amax 32 = 2^5, E4M3 emax 8: shared exponent -3, elements v * 8 rounded
    v = np.arange(1, 33, dtype=np.float32)
    q, s = mx.quantize(_bf16(v)[None, :], "e4m3")
    assert s.tolist() == [[124]]
    want = torch.from_numpy(v * 8).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(q[0], want)
    # E2M1: amax 7 -> exponent 2 - 2 = 0; 7 saturates to 6, 5 ties to 4 (even), 2.5 ties to 2,
    # -0.75 ties between -0.5 (odd mantissa) and -1 (even): -1
    v = np.zeros(32, dtype=np.float32)
    v[:5] = [7.0, 5.0, 2.5, -0.75, 0.2]
    q, s = mx.quantize(_bf16(v)[None, :], "e2m1")
    assert s.tolist() == [[127]]
    assert q[0, :5].tolist() == [0x7, 0x6, 0x4, 0xA, 0x0]
    # an all-zero block (with a negative zero) takes scale byte 0 and zero codes
    v = np.zeros(32, dtype=np.float32)
    v[3] = -0.0
    q, s = mx.quantize(_bf16(v)[None, :], "e4m3")
    assert s.tolist() == [[0]] and q[0, 3] == 0x80 and q[0].sum() == 0x80
    # scales clamp to the E8M0 range
    v = np.full(32, 2.0 ** -130, dtype=np.float32)
    q, s = mx.quantize(_bf16(v)[None, :], "e2m1")
    assert s[0, 0] == 0


@pytest.mark.parametrize("fmt", ["e4m3", "e2m1"])
def test_round_trip(fmt):
    X = matrix("normal", 8, 256, seed=17, sigma=0.3)
    q, s = mx.quantize(X, fmt)
    back = mx.dequantize(q, s, fmt)
    bits = f32_to_bf16_bits(back.astype(np.float32))
    assert np.array_equal(bf16_bits_to_f32(bits).astype(np.float64), back)  # exact in bf16
    q2, s2 = mx.quantize(bits, fmt)
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_product_matches_bf16_oracle(oracle_lib):
    M, N, K = 5, 48, 256
    A = matrix("normal", M, K, seed=21)
    W = matrix("normal", N, K, seed=22, sigma=0.02)
    aq, as_ = mx.quantize(A, "e4m3")
    wq, ws = mx.quantize(W, "e2m1")
    ref, sabs = mx.product(aq, as_, wq, ws)
    a16 = f32_to_bf16_bits(mx.dequantize(aq, as_, "e4m3").astype(np.float32))
    w16 = f32_to_bf16_bits(mx.dequantize(wq, ws, "e2m1").astype(np.float32))
    r2, s2 = oracle.gemm(a16, np.ascontiguousarray(w16.T))
    assert np.allclose(ref, r2, rtol=1e-12, atol=1e-300) and np.allclose(sabs, s2, rtol=1e-12)


def test_packed_layout_term_by_term():
    N, K = 32, 640  # KS = 5: a partial last group of four k-steps
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16, size=(N, K), dtype=np.uint8)
    scales = rng.integers(0, 255, size=(N, K // 32), dtype=np.uint8)
    wp, sp = mx.pack_weights(codes, scales)
    ks, kq = K // 128, 2
    assert (len(wp), len(sp)) == mx.packed_sizes(N, K) == (N // 16 * ks * 1024, N // 16 * kq * 256)
    for t in range(N // 16):
        for s in range(ks):
            for lane in range(64):
                n, k0 = 16 * t + lane % 16, 128 * s + 32 * (lane // 16)
                for j in range(32):
                    byte = wp[1024 * (t * ks + s) + 16 * lane + j // 2]
                    assert (byte >> (4 * (j % 2))) & 0xF == codes[n, k0 + j]
                assert sp[256 * (t * kq + s // 4) + 4 * lane + s % 4] == scales[n, k0 // 32]
    # the slots of the missing k-steps 5 .. 7 are zero
    for t in range(N // 16):
        for lane in range(64):
            for s in (5, 6, 7):
                assert sp[256 * (t * kq + 1) + 4 * lane + s % 4] == 0


@pytest.fixture(scope="module")
def mx_problem(oracle_lib):
    M, N, K = 16, 256, 4096
    A = matrix("normal", M, K, seed=31)
    W = matrix("normal", N, K, seed=32, sigma=0.02)
    aq, as_ = mx.quantize(A, "e4m3")
    wq, ws = mx.quantize(W, "e2m1")
    ref, sabs = mx.product(aq, as_, wq, ws)
    a = mx.dequantize(aq, as_, "e4m3").astype(np.float32)
    w = mx.dequantize(wq, ws, "e2m1").astype(np.float32)
    return aq, as_, wq, ws, ref, sabs, a, w


def test_float32_model_passes(mx_problem):
    *_, ref, sabs, a, w = mx_problem
    c = f32_to_bf16_bits((a @ w.T).astype(np.float32))
    res = oracle.check(c, ref, sabs)
    assert res.ok, res.summary()


@pytest.mark.parametrize("mistake", ["no_scale", "scale_shift", "nibbles_swapped"])
def test_planted_mistakes_fail(mx_problem, mistake):
    aq, as_, wq, ws, ref, sabs, a, w = mx_problem
    if mistake == "no_scale":
        w2 = mx.value_table("e2m1")[wq.astype(np.int64)].astype(np.float32)
    elif mistake == "scale_shift":
        w2 = mx.dequantize(wq, np.roll(ws, 1, axis=1), "e2m1").astype(np.float32)
    else:
        sw = wq.reshape(wq.shape[0], -1, 2)[:, :, ::-1].reshape(wq.shape)
        w2 = mx.dequantize(sw, ws, "e2m1").astype(np.float32)
    c = f32_to_bf16_bits((a @ w2.T).astype(np.float32))
    assert not oracle.check(c, ref, sabs).ok, mistake
