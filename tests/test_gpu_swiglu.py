"""Parity of the fused gate/up SwiGLU entry point (gemm_bf16_swiglu) with the float64 oracle.

Every output is compared element by element against oracle.swiglu: |c - h| <= 2^-8 |h| + the
bound the oracle derives from the product check's float32 allowance, plus the relative
Frobenius bound. Outputs are poisoned with NaN before each call. Shapes cover the skinny kernel
(M <= 64: aligned layouts, Stream-K ranges, 128- and 256-column strips), the large-tile kernel
(256 x 256 tiles, 128 x 128 tiles with K split), the general kernel (unaligned operands), ragged
edges in every dimension, K = 0, and the Llama-7B gate/up shapes at full size, on sampled rows
for the prefill shape.
"""

import ctypes

import numpy as np
import pytest

from oracle import swiglu as osw
from synth import WORKLOADS, matrix

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gemv_layers_amd as g  # noqa: E402

POISON = 0x7FC07FC0


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.set_device(0)
    g.gemm_init(0)
    yield


def dev(h: np.ndarray) -> "torch.Tensor":
    t = torch.from_numpy(np.ascontiguousarray(h).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda")


def host(t: "torch.Tensor") -> np.ndarray:
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def run(A, B, M, N, K, ldc=None, offset=0):
    """gemm_bf16_swiglu on host bf16-bit arrays A (M x lda) and B (K x ldb >= 2N); C bits.
    `offset` elements shift every operand off 16-byte alignment (the general kernel)."""
    ldc = N if ldc is None else ldc
    dA = dev(np.concatenate([np.zeros(offset, np.uint16), A.ravel()]))
    dB = dev(np.concatenate([np.zeros(offset, np.uint16), B.ravel()]))
    n = -(-(max(M * ldc, 8) + offset) // 8) * 8
    C = torch.empty(n, dtype=torch.bfloat16, device="cuda")
    g.gemm_fill_launch(ctypes.c_void_p(C.data_ptr()), C.numel() * 2, POISON)
    lda = A.shape[1] if A.size else max(K, 1)
    ldb = B.shape[1] if B.size else max(2 * N, 1)
    g.gemm_bf16_swiglu(M, N, K, ctypes.c_void_p(dA.data_ptr() + 2 * offset), lda,
                       ctypes.c_void_p(dB.data_ptr() + 2 * offset), ldb,
                       ctypes.c_void_p(C.data_ptr() + 2 * offset), ldc, g.current_stream_handle())
    torch.cuda.synchronize()
    plan = g.gemm_last_plan()
    return host(C)[offset: offset + M * ldc].reshape(M, ldc)[:, :N], plan


def check(C, A, B, M, N, K, what):
    h, slack = osw.swiglu(A, B, M, N, K)
    res = osw.check(C, h, slack)
    assert res.ok, f"{what} {res.summary()}"
    return res


SKINNY = [(1, 8, 64), (1, 520, 328), (2, 1000, 1000), (3, 128 * 141 + 8, 64 * 37 + 8),
          (16, 64, 2048), (17, 4104, 1032), (33, 2056, 520), (48, 1376, 4096), (64, 1000, 200)]


@pytest.mark.parametrize("M,N,K", SKINNY)
def test_skinny_swiglu(M, N, K):
    A = matrix("normal", M, K, seed=7100 + M)
    B = matrix("normal", K, 2 * N, seed=7200 + N, sigma=0.02)
    C, plan = run(A, B, M, N, K)
    assert plan["kernel"] == "skinny" and plan["op"] == "swiglu", plan
    check(C, A, B, M, N, K, f"skinny swiglu {M}x{N}x{K} plan={plan['strip']}/{plan['grid']}")


@pytest.mark.parametrize("name", ["glu_dec_M1", "glu_dec_M16", "glu_dec_M64"])
def test_llama7b_gate_up_decode_full(name):
    """The decode workloads at full size, every output element, dispatching entry point."""
    w = WORKLOADS[name]
    M, N, K = w.M, w.N, w.K
    A = matrix("normal", M, K, seed=w.seed_a, sigma=w.sigma_a)
    B = matrix("normal", K, 2 * N, seed=w.seed_b, sigma=w.sigma_b)
    C, plan = run(A, B, M, N, K)
    assert plan["kernel"] == "skinny" and plan["op"] == "swiglu", plan
    check(C, A, B, M, N, K, f"skinny swiglu {M}x{N}x{K} plan={plan['strip']}/{plan['grid']}")


TILED = [(65, 520, 328), (256, 256, 64), (300, 1000, 1000), (1000, 1000, 1000),
         (513, 1032, 2056), (1024, 2048, 1024)]


@pytest.mark.parametrize("M,N,K", TILED)
def test_tiled_swiglu(M, N, K):
    A = matrix("normal", M, K, seed=7300 + M)
    B = matrix("normal", K, 2 * N, seed=7400 + N, sigma=0.05)
    C, plan = run(A, B, M, N, K)
    assert plan["kernel"] == "tile" and plan["op"] == "swiglu", plan
    check(C, A, B, M, N, K, f"tile swiglu {M}x{N}x{K} bm={plan['bm']} splits={plan['splits']}")


def test_tiled_swiglu_split_k_is_used():
    # a grid of 128 x 128 tiles too small for the card: K is split and the fixup runs
    M, N, K = 128, 256, 4096
    A = matrix("normal", M, K, seed=7500)
    B = matrix("normal", K, 2 * N, seed=7501, sigma=0.02)
    C, plan = run(A, B, M, N, K)
    assert plan["schedule"] == "split-k" and plan["splits"] > 1, plan
    check(C, A, B, M, N, K, "tile swiglu split-k")


@pytest.mark.parametrize("M,N,K,ldpad", [(5, 13, 7, 0), (70, 100, 30, 0), (3, 24, 40, 3),
                                         (130, 200, 96, 5)])
def test_general_kernel_swiglu(M, N, K, ldpad):
    A = matrix("normal", M, K, seed=7600 + M, ld=K + ldpad)
    B = matrix("normal", K, 2 * N, seed=7700 + N, sigma=0.1, ld=2 * N + ldpad)
    C, plan = run(A, B, M, N, K, ldc=N + ldpad, offset=1 if ldpad == 0 else 0)
    assert plan["kernel"] == "generic", plan
    check(C, A[:, :K], B[:, : 2 * N], M, N, K, f"generic swiglu {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K", [(3, 520, 328), (300, 520, 328)])
def test_leading_dimensions_with_nan_padding(M, N, K):
    A = matrix("normal", M, K, seed=7800, ld=K + 8)
    B = matrix("normal", K, 2 * N, seed=7801, sigma=0.05, ld=2 * N + 16)  # NaN past 2N
    C, plan = run(A, B, M, N, K, ldc=N + 24)
    assert plan["kernel"] in ("skinny", "tile"), plan
    check(C, A[:, :K], B[:, : 2 * N], M, N, K, f"swiglu with ld padding {M}x{N}x{K}")


def test_k_zero_writes_zeros():
    for M in (4, 100):
        C, plan = run(np.zeros((M, 0), np.uint16), np.zeros((0, 32), np.uint16), M, 16, 0)
        assert (C == 0).all(), plan


def test_deterministic():
    M, N, K = 3, 128 * 141 + 8, 64 * 37 + 8
    A = matrix("normal", M, K, seed=7900)
    B = matrix("normal", K, 2 * N, seed=7901, sigma=0.02)
    C1, _ = run(A, B, M, N, K)
    C2, _ = run(A, B, M, N, K)
    assert np.array_equal(C1, C2)


def test_llama7b_gate_up_prefill_sampled_rows():
    """M = 4096 tokens against the 4096 x (2 x 11008) gate/up weight, in the launch configuration
    of the dispatching entry point; rows sampled across tiles, the last one included."""
    w = WORKLOADS["glu_prefill"]
    M, N, K = w.M, w.N, w.K
    A = matrix("normal", M, K, seed=w.seed_a, sigma=w.sigma_a)
    B = matrix("normal", K, 2 * N, seed=w.seed_b, sigma=w.sigma_b)
    C, plan = run(A, B, M, N, K)
    assert plan["kernel"] == "tile" and plan["bm"] == 256, plan
    for r in (0, 255, 256, 1999, 3071, 4095):
        h, slack = osw.swiglu_rows(A, B, r, 1, N, K)
        res = osw.check(C[r: r + 1], h, slack)
        assert res.ok, f"row {r}: {res.summary()}"


def test_sparse_last_wave_cut_across_rows():
    """4608 tokens against a 4096 x (2 x 2304) weight: 324 tiles of 256 x 256 leave a last wave of
    68, which is cut off as a row strip (the SwiGLU form cannot take a column cut) planned on its
    own; rows on both sides of the cut and at both ends are checked."""
    M, N, K = 4608, 2304, 1024
    A = matrix("normal", M, K, seed=7600)
    B = matrix("normal", K, 2 * N, seed=7601, sigma=0.05)
    C, plan = run(A, B, M, N, K)
    assert plan["op"] == "swiglu" and plan["cut"]["axis"] == "m" and plan["cut"]["at"] == 3584, plan
    assert plan["cut"]["rest"]["bm"] == 128
    for r in (0, 1000, 3583, 3584, 3585, 4000, 4607):
        h, slack = osw.swiglu_rows(A, B, r, 1, N, K)
        res = osw.check(C[r: r + 1], h, slack)
        assert res.ok, f"row {r}: {res.summary()}"


# ---- seeded random shapes across every dispatch regime ---------------------------------------

def _random_glu_cases(n, seed=20251203):
    """(M, N, K) from a fixed seed: M in the skinny, small-tile and large-tile ranges; N and K
    multiples of 8 (the fast kernels) or arbitrary (the general kernel); at most 1e9 multiply-adds
    over the gate and up halves together."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        regime = rng.choice(3, p=[0.4, 0.3, 0.3])
        M = int(rng.integers(1, 65) if regime == 0 else rng.integers(65, 400) if regime == 1
                else rng.integers(400, 1100))
        N, K = int(rng.integers(1, 2000)), int(rng.integers(1, 1600))
        if rng.random() < 0.75:
            N, K = max(8, N - N % 8), max(8, K - K % 8)
        if 2 * M * N * K <= 1e9:
            cases.append((M, N, K))
    return cases


RANDOM_GLU = _random_glu_cases(24)


@pytest.mark.parametrize("case", range(len(RANDOM_GLU)))
def test_random_shapes_swiglu(case):
    M, N, K = RANDOM_GLU[case]
    A = matrix("normal", M, K, seed=7700 + case)
    B = matrix("normal", K, 2 * N, seed=7800 + case, sigma=0.02)
    C, plan = run(A, B, M, N, K)
    check(C, A, B, M, N, K, f"swiglu {M}x{N}x{K} ({plan['kernel']})")
