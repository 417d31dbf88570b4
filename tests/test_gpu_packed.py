"""Parity of the packed-weight decode entry points with the oracle, through the C ABI.

gemm_pack_weight_bf16 is byte work and must match the oracle's packed layout (oracle/packed.py)
bit for bit, with the poison past its output intact. gemm_bf16_packed takes the oracle's own
packed bytes and is checked against the float64 product oracle on the unpacked weight: the
element-wise bound |c - ref| <= 2^-8 |ref| + 2^-16 sum|ab| and a relative Frobenius error <= 4e-3.
Shapes cover one to four 16-row tiles of M, partial groups of column tiles, K split over
workgroups or not, and the Llama-7B decode shapes at full size.
"""

import ctypes

import numpy as np
import pytest

import oracle
from oracle import packed
from synth import WORKLOADS, matrix

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gemv_layers_amd as g  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.set_device(0)
    g.gemm_init(0)
    yield


def P(t):
    return ctypes.c_void_p(t.data_ptr())


def dev16(h):
    return torch.from_numpy(np.ascontiguousarray(h).view(np.int16)).cuda()


@pytest.mark.parametrize("K,N,pad", [(32, 16, 0), (640, 48, 8), (4096, 1040, 0), (11008, 4096, 0)])
def test_pack_bit_exact(K, N, pad):
    B = matrix("normal", K, N, seed=1000 + N, sigma=0.02, ld=N + pad)
    dB = dev16(B)
    out = torch.full((K * N + 64,), 0x5A5A, dtype=torch.int16, device="cuda")
    g.gemm_pack_weight_bf16(K, N, P(dB), N + pad, P(out), g.current_stream_handle())
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)
    assert np.array_equal(got[: K * N], packed.pack(B, K, N))
    assert (got[K * N:] == 0x5A5A).all()


def run_packed(A, B, M, N, K, ldc=None):
    ldc = N if ldc is None else ldc
    dA = dev16(A)
    dP = dev16(packed.pack(B, K, N)) if K else torch.zeros(8, dtype=torch.int16, device="cuda")
    C = torch.empty(max(M * ldc, 8), dtype=torch.int16, device="cuda")
    g.gemm_fill_launch(P(C), C.numel() * 2 // 4 * 4, 0x7FC07FC0)
    g.gemm_bf16_packed(M, N, K, P(dA), A.shape[1] if A.size else max(K, 8), P(dP), P(C), ldc,
                       g.current_stream_handle())
    torch.cuda.synchronize()
    c = C.cpu().numpy().view(np.uint16)[: M * ldc].reshape(M, ldc)
    return c, g.gemm_last_plan()


SHAPES = [(1, 16, 32), (1, 64, 640), (3, 80, 512), (2, 256, 11008), (16, 4096, 4096),
          (17, 1040, 2048), (33, 2048, 1024), (48, 512, 4096), (64, 1040, 1152)]


@pytest.mark.parametrize("M,N,K", SHAPES)
def test_packed_parity(M, N, K):
    A = matrix("normal", M, K, seed=1100 + M)
    B = matrix("normal", K, N, seed=1200 + N, sigma=0.02)
    C, plan = run_packed(A, B, M, N, K)
    assert plan["kernel"] == "packed", plan
    ref, sabs = oracle.gemm(A, B)
    res = oracle.check(C, ref, sabs)
    assert res.ok, f"packed {M}x{N}x{K} splits={plan['splits']}: {res.summary()}"


@pytest.mark.parametrize("name", ["dec_up_M1", "dec_up_M16", "dec_up_M64", "dec_down_M1",
                                  "dec_down_M64"])
def test_packed_llama7b_full(name):
    w = WORKLOADS[name]
    A = matrix("normal", w.M, w.K, seed=w.seed_a, sigma=w.sigma_a)
    B = matrix("normal", w.K, w.N, seed=w.seed_b, sigma=w.sigma_b)
    C, plan = run_packed(A, B, w.M, w.N, w.K)
    ref, sabs = oracle.gemm(A, B)
    res = oracle.check(C, ref, sabs)
    assert res.ok, f"{name} splits={plan['splits']}: {res.summary()}"


def test_integer_inputs_bit_exact():
    M, N, K = 5, 256, 4096
    A = matrix("int", M, K, seed=1300, radius=3)
    B = matrix("int", K, N, seed=1301, radius=3)
    C, plan = run_packed(A, B, M, N, K)
    ref, _ = oracle.gemm(A, B, with_abs=False)
    assert plan["splits"] > 1
    assert np.array_equal(C, oracle.bf16_rne(ref))


def test_ldc_padding_k_zero_and_determinism():
    M, N, K = 3, 2048, 11008
    A = matrix("normal", M, K, seed=1400)
    B = matrix("normal", K, N, seed=1401, sigma=0.02)
    C1, plan = run_packed(A, B, M, N, K, ldc=N + 20)
    C2, _ = run_packed(A, B, M, N, K, ldc=N + 20)
    assert plan["splits"] > 1 and np.array_equal(C1, C2)
    assert (C1[:, N:] == 0x7FC0).all()
    ref, sabs = oracle.gemm(A, B)
    assert oracle.check(C1[:, :N], ref, sabs).ok
    C0, _ = run_packed(np.zeros((2, 0), np.uint16), np.zeros((0, 32), np.uint16), 2, 32, 0)
    assert (C0 == 0).all()


def test_largest_packed_weight_and_row_major_stream():
    # the largest weight gemm_bf16_packed takes (2 K N bytes just under 2^31: 32-bit offsets),
    # with a 0/1 weight whose pattern differs from column to column, (k + 3 n) % 7 == 0, and
    # integer activations: every partial sum is an integer below 2^24, so the result is exact and
    # C[m][n] is the bf16 rounding of the sum of A[m][k] over k = -3 n (mod 7). The same weight
    # also goes through the row-major entry (gemm_bf16, M <= 64: the skinny kernel).
    M, K, N = 2, 32768, 32752
    assert 2 * K * N <= 2**31 - 1
    A = matrix("int", M, K, seed=1500, radius=2)
    kk = torch.arange(K, device="cuda", dtype=torch.int32)[:, None]
    nn = torch.arange(N, device="cuda", dtype=torch.int32)[None, :]
    B = ((kk + 3 * nn) % 7 == 0).to(torch.bfloat16)
    del kk, nn
    s = g.current_stream_handle()
    Bp = torch.empty(K * N, dtype=torch.bfloat16, device="cuda")
    g.gemm_pack_weight_bf16(K, N, P(B), N, P(Bp), s)
    dA = dev16(A)
    Af = oracle.bf16_to_f64(A)
    residue = np.arange(K) % 7
    sums = np.stack([Af[:, residue == c].sum(axis=1) for c in range(7)], axis=1)  # M x 7, exact
    want = oracle.bf16_rne(sums[:, (-3 * np.arange(N)) % 7])
    for name in ("packed", "row-major"):
        C = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
        if name == "packed":
            g.gemm_bf16_packed(M, N, K, P(dA), K, P(Bp), P(C), N, s)
        else:
            g.gemm_bf16(M, N, K, P(dA), K, P(B), N, P(C), N, s)
        torch.cuda.synchronize()
        got = C.cpu().view(torch.int16).numpy().view(np.uint16)
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"{name}: {len(bad)} mismatches, first at {bad[0].tolist()}"
    del B, Bp
    torch.cuda.empty_cache()
