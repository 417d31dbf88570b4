"""gemm_bf16_noalloc against gemm_bf16, through the C ABI, on an MI355X.

The allocation-free entry point runs gemm_bf16's own plan and kernels with the library's fixed
scratch array as workspace, so its output must equal gemm_bf16's bit for bit. Two calls in a row,
the second on a smaller input, for each layout that uses the workspace (skinny K split, skinny
Stream-K ranges, large-tile K split, one and two pieces per CU, a product cut into a rectangle
of whole waves and a K-split strip) and one that does not; every output is also checked against
the float64 oracle. The 1664 x 1664 x 4096 split plan (169 tiles
of 128 x 128 in 3 pieces, two per CU on most CUs) takes 8 306 688 of the array's 8 Mi floats
(the most a plan on 256 CUs can need is 8 Mi, 512 pieces); the skinny 17 x 264 x 11008 plan
takes 4 Mi.
"""

import ctypes

import numpy as np
import pytest

import oracle
from synth import matrix

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


def _call(fn, A, B, M, N, K):
    dA = torch.from_numpy(A.view(np.int16)).cuda()
    dB = torch.from_numpy(B.view(np.int16)).cuda()
    C = torch.empty(max(M * N, 8), dtype=torch.bfloat16, device="cuda")
    s = g.current_stream_handle()
    g.gemm_fill_launch(ctypes.c_void_p(C.data_ptr()), C.numel() * 2, POISON, s)
    fn(M, N, K, ctypes.c_void_p(dA.data_ptr()), K, ctypes.c_void_p(dB.data_ptr()), N,
       ctypes.c_void_p(C.data_ptr()), N, s)
    torch.cuda.synchronize()
    return C.cpu().view(torch.int16).numpy().view(np.uint16)[: M * N].reshape(M, N)


# (first call, second smaller call) per layout
PAIRS = [((17, 264, 11008), (16, 4096, 11008)),                        # every slot; skinny, K split
         ((3, 128 * 141 + 8, 64 * 37 + 8), (1, 128 * 131, 64 * 20)),   # skinny Stream-K ranges
         ((16, 4096, 11008), (3, 4096, 4096)),                          # skinny, K split
         ((1000, 1000, 1000), (512, 512, 512)),                        # 128 x 128 tiles, K split
         ((1664, 1664, 4096), (1536, 1536, 1024)),                      # K split, two pieces per CU
         ((4096, 4096, 4096), (300, 520, 328)),                        # 256 x 256 tiles, no split
         ((4096, 4352, 1024), (4352, 4096, 512))]                       # a sparse last wave cut off
                                                                        # (two launches, the strip K split)


@pytest.mark.parametrize("first,second", PAIRS)
def test_noalloc_matches_gemm_bf16_twice(first, second):
    for n, (M, N, K) in enumerate((first, second)):
        A = matrix("normal", M, K, seed=14000 + M + n)
        B = matrix("normal", K, N, seed=15000 + N + n, sigma=0.02)
        want = _call(g.gemm_bf16, A, B, M, N, K)
        plan = g.gemm_last_plan()
        if n == 0 and (M, N, K) == (17, 264, 11008):
            assert plan["ws_floats"] == 4 << 20
        if n == 0 and (M, N, K) == (1664, 1664, 4096):
            assert plan["splits"] == 3 and plan["ws_floats"] == 169 * 3 * 128 * 128 > 4 << 20
        if (M, N, K) in ((4096, 4352, 1024), (4352, 4096, 512)):
            assert "cut" in plan and plan["cut"]["rest"]["schedule"] == "split-k", plan
        got = _call(g.gemm_bf16_noalloc, A, B, M, N, K)
        assert g.gemm_last_plan() == plan
        bad = np.argwhere(got != want)
        assert bad.size == 0, f"call {n} {M}x{N}x{K}: {len(bad)} differ from gemm_bf16, first {bad[0].tolist()}"
        rows = np.arange(M) if M <= 64 else np.unique(np.linspace(0, M - 1, 40).astype(int))
        ref, sabs = oracle.gemm(np.ascontiguousarray(A[rows]), B, M=len(rows), N=N, K=K)
        res = oracle.check(np.ascontiguousarray(got[rows]), ref, sabs)
        assert res.ok, f"call {n} {M}x{N}x{K}: {res.summary()}"
