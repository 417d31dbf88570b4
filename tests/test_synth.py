"""The shared input generator: published SplitMix64 outputs, reproducibility, distributions."""

import numpy as np

from synth import (WORKLOADS, bf16_bits_to_f32, f32_to_bf16_bits, integer_bf16, matrix,
                   normal_bf16, splitmix64)


def _py_splitmix64(seed, c):
    m = (1 << 64) - 1
    x = (seed + (c + 1) * 0x9E3779B97F4A7C15) & m
    x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & m
    x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & m
    return x ^ (x >> 31)


def test_splitmix64_reference_outputs():
    # the first outputs of SplitMix64 started from state 0 (Vigna's reference splitmix64.c)
    got = splitmix64(0, np.arange(3, dtype=np.uint64))
    assert [int(v) for v in got] == [0xE220A8397B1DCDAF, 0x6E789E6AA1B965F4, 0x06C45D188009454F]
    idx = np.array([0, 1, 12345, 2**40], dtype=np.uint64)
    for seed in (0x5EED0000, 0xFFFFFFFFFFFFFFFF):
        assert [int(v) for v in splitmix64(seed, idx)] == [_py_splitmix64(seed, int(i)) for i in idx]


def test_reproducible_and_indexable():
    a = normal_bf16(7, 1000)
    b = normal_bf16(7, 1000)
    np.testing.assert_array_equal(a, b)
    np.testing.assert_array_equal(normal_bf16(7, 300, start=700), a[700:])
    assert not np.array_equal(normal_bf16(8, 1000), a)
    m = matrix("normal", 10, 12, seed=7, ld=16)
    np.testing.assert_array_equal(m[:, :12].reshape(-1), normal_bf16(7, 120))
    assert np.all(m[:, 12:] == 0x7FC0)


def test_normal_moments():
    x = bf16_bits_to_f32(normal_bf16(99, 1 << 20, sigma=0.02)).astype(np.float64)
    assert abs(x.mean()) < 1e-4
    assert abs(x.std() / 0.02 - 1) < 0.01
    assert abs(((x / 0.02) ** 4).mean() - 3.0) < 0.05       # Gaussian kurtosis


def test_integer_range_and_exactness():
    v = bf16_bits_to_f32(integer_bf16(5, 100000, radius=4))
    assert set(np.unique(v).tolist()) == set(float(i) for i in range(-4, 5))
    assert np.all(f32_to_bf16_bits(v) == integer_bf16(5, 100000, radius=4))


def test_f32_to_bf16_is_round_to_nearest_even():
    x = np.array([4112.0, 4144.0, 4120.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8], dtype=np.float32)
    got = bf16_bits_to_f32(f32_to_bf16_bits(x))
    assert got.tolist() == [4096.0, 4160.0, 4128.0, 1.0, 1.0 + 2 ** -6]


def test_workloads():
    w = WORKLOADS
    assert (w["sq4096"].M, w["sq4096"].N, w["sq4096"].K) == (4096, 4096, 4096)
    assert (w["mlp_up"].N, w["mlp_up"].K) == (11008, 4096)
    assert (w["mlp_down"].N, w["mlp_down"].K) == (4096, 11008)
    assert w["dec_down_M64"].K == 11008 and w["dec_up_M1"].N == 11008
    assert w["sq4096"].flops == 2 * 4096 ** 3
    assert w["dec_up_M1"].bytes == 2 * (4096 + 4096 * 11008 + 11008)
    assert len({(x.seed_a, x.seed_b) for x in w.values()}) == 10
    assert w["glu_prefill"].b_cols == 2 * 11008 and w["glu_prefill"].flops == 2 * 4096 * 22016 * 4096
    assert w["glu_dec_M1"].bytes == 2 * (4096 + 4096 * 22016 + 11008)
