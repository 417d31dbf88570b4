"""Parity of the block-scaled (MX) entry points with the oracle (oracle/mx.py), through the C ABI.

* The conversions are integer work and must match bit for bit: gemm_mx_quantize_act against the
  oracle's E4M3 conversion, gemm_mx_pack_weight against the oracle's E2M1 conversion followed by
  its packed layout, on random data and on blocks built to hit every branch (all-zero blocks,
  signed zeros, subnormal bf16, saturation, ties, scales at the E8M0 limits). Bytes outside the
  outputs must keep their poison.
* The product gemm_mx_decode takes the oracle's own quantised bytes (nothing from the GPU
  conversions) and is checked like the bf16 product: |c - ref| <= 2^-8 |ref| + 2^-16 sum|ab| per
  element over the dequantised operands, and a relative Frobenius error <= 4e-3. Shapes cover
  one and several 16-row tiles of M, partial groups of column tiles, K split over workgroups or
  not, and the Llama-7B decode shapes at full size.
"""

import ctypes

import numpy as np
import pytest

import oracle
from oracle import mx
from synth import WORKLOADS, f32_to_bf16_bits, matrix

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import gemv_layers_amd as g  # noqa: E402

POISON8 = 0xA5


@pytest.fixture(scope="module", autouse=True)
def _device():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    torch.cuda.set_device(0)
    g.gemm_init(0)
    yield


def P(t):
    return ctypes.c_void_p(t.data_ptr())


def dev_bf16(h):
    return torch.from_numpy(np.ascontiguousarray(h).view(np.int16)).view(torch.bfloat16).cuda()


def dev_u8(h):
    return torch.from_numpy(np.ascontiguousarray(h, dtype=np.uint8)).cuda()


def poisoned(nbytes):
    return torch.full((max(nbytes, 16),), POISON8, dtype=torch.uint8, device="cuda")


def special_rows(K):
    """Rows (bf16 bits) whose blocks exercise every branch of the conversion."""
    rows = []
    z = np.zeros(K, dtype=np.uint16)
    rows.append(z.copy())                                 # all-zero blocks
    r = z.copy(); r[1::7] = 0x8000; rows.append(r)        # negative zeros only
    r = f32_to_bf16_bits(np.linspace(-9, 9, K).astype(np.float32)); rows.append(r)
    r = (np.arange(K) % 127 + 1).astype(np.uint16); rows.append(r)    # bf16 subnormals
    r = (np.arange(K) % 127 + 1).astype(np.uint16) | 0x8000; r[::5] = 0x0001; rows.append(r)
    big = f32_to_bf16_bits(np.full(K, 3.0e38, dtype=np.float32)); big[::3] ^= 0x8000; rows.append(big)
    r = f32_to_bf16_bits((2.0 ** ((np.arange(K) % 40) - 20)).astype(np.float32)); rows.append(r)
    # wide dynamic range inside a block: tiny values vanish, the largest saturate
    v = np.tile(np.array([1e-30, 7.0, -7.5, 5.0, 2.5, -0.75, 448.0, 500.0], dtype=np.float32), K // 8)
    rows.append(f32_to_bf16_bits(v))
    return np.stack(rows)


def run_quantize_act(A, M, K, lda, ldaq, ldas):
    dA = dev_bf16(A)
    q = poisoned(M * ldaq)
    s = poisoned(M * ldas)
    g.gemm_mx_quantize_act(M, K, P(dA), lda, P(q), ldaq, P(s), ldas, g.current_stream_handle())
    torch.cuda.synchronize()
    return q.cpu().numpy(), s.cpu().numpy()


@pytest.mark.parametrize("M,K,pad", [(1, 32, 0), (3, 4096, 8), (17, 11008, 0), (64, 4096, 24),
                                     (8, 256, 0)])
def test_quantize_act_bit_exact(M, K, pad):
    lda, ldaq, ldas = K + pad, K + (16 if pad else 0), K // 32 + (3 if pad else 0)
    A = matrix("normal", M, K, seed=500 + M, ld=lda)
    if M == 8:
        A = np.ascontiguousarray(special_rows(K))
    q, s = run_quantize_act(A, M, K, lda, ldaq, ldas)
    wq, ws = mx.quantize(A, "e4m3", cols=K)
    q2 = q[: M * ldaq].reshape(M, ldaq)
    s2 = s[: M * ldas].reshape(M, ldas)
    bad = np.argwhere(q2[:, :K] != wq)
    assert bad.size == 0, f"{len(bad)} code mismatches, first at {bad[0].tolist()}: " \
                          f"{q2[tuple(bad[0])]:#x} vs {wq[tuple(bad[0])]:#x}"
    assert np.array_equal(s2[:, : K // 32], ws)
    if pad:
        assert (q2[:, K:] == POISON8).all() and (s2[:, K // 32:] == POISON8).all()
    assert (q[M * ldaq:] == POISON8).all() and (s[M * ldas:] == POISON8).all()


def run_pack(W, N, K, ldw):
    wb, sb = g.gemm_mx_packed_sizes(N, K)
    wp = poisoned(wb + 64)
    sp = poisoned(sb + 64)
    dW = dev_bf16(W)
    g.gemm_mx_pack_weight(N, K, P(dW), ldw, P(wp), P(sp), g.current_stream_handle())
    torch.cuda.synchronize()
    return wp.cpu().numpy(), sp.cpu().numpy(), wb, sb


@pytest.mark.parametrize("N,K,pad", [(16, 128, 0), (32, 640, 8), (80, 512, 0), (48, 1152, 16)])
def test_pack_weight_bit_exact(N, K, pad):
    W = matrix("normal", N, K, seed=600 + N, sigma=0.02, ld=K + pad)
    if N == 80:
        W[:8] = special_rows(K)
    wp, sp, wb, sb = run_pack(W, N, K, K + pad)
    q, s = mx.quantize(W, "e2m1", cols=K)
    ep, es = mx.pack_weights(q, s)
    assert np.array_equal(wp[:wb], ep), f"{np.count_nonzero(wp[:wb] != ep)} packed code bytes differ"
    assert np.array_equal(sp[:sb], es), f"{np.count_nonzero(sp[:sb] != es)} packed scale bytes differ"
    assert (wp[wb:] == POISON8).all() and (sp[sb:] == POISON8).all()


def test_pack_weight_full_size_bit_exact():
    w = WORKLOADS["dec_down_M1"]  # the down projection weight in the nn.Linear layout: N x K
    N, K = w.N, w.K
    W = matrix("normal", N, K, seed=w.seed_b, sigma=w.sigma_b)
    wp, sp, wb, sb = run_pack(W, N, K, K)
    q, s = mx.quantize(W, "e2m1")
    ep, es = mx.pack_weights(q, s)
    assert np.array_equal(wp[:wb], ep) and np.array_equal(sp[:sb], es)


def oracle_operands(M, N, K, seed):
    A = matrix("normal", M, K, seed=seed)
    W = matrix("normal", N, K, seed=seed + 1, sigma=0.02)
    aq, as_ = mx.quantize(A, "e4m3")
    wq, ws = mx.quantize(W, "e2m1")
    wp, sp = mx.pack_weights(wq, ws)
    return A, aq, as_, wq, ws, wp, sp


def run_decode(aq, as_, wp, sp, M, N, K, ldc=None):
    ldc = N if ldc is None else ldc
    ldaq = -(-max(K, 16) // 16) * 16
    qa = np.zeros((M, ldaq), np.uint8)
    qa[:, :K] = aq
    dq, ds = dev_u8(qa), dev_u8(as_)
    dwp, dsp = dev_u8(wp), dev_u8(sp)
    C = torch.empty(max(M * ldc, 8), dtype=torch.bfloat16, device="cuda")
    g.gemm_fill_launch(P(C), C.numel() * 2 // 4 * 4, 0x7FC07FC0)
    g.gemm_mx_decode(M, N, K, P(dq), ldaq, P(ds), max(K // 32, 1), P(dwp), P(dsp), P(C), ldc,
                     g.current_stream_handle())
    torch.cuda.synchronize()
    c = C.cpu().view(torch.int16).numpy().view(np.uint16)[: M * ldc].reshape(M, ldc)
    return c, g.gemm_last_plan()


DECODE = [(1, 16, 128), (1, 64, 640), (3, 80, 512), (2, 256, 11008), (16, 4096, 4096),
          (17, 1024, 2048), (33, 2048, 1024), (48, 512, 4096), (64, 1040, 1152), (2, 2000, 4096)]


@pytest.mark.parametrize("M,N,K", DECODE)
def test_decode_parity(M, N, K):
    _, aq, as_, wq, ws, wp, sp = oracle_operands(M, N, K, 700 + M + N)
    C, plan = run_decode(aq, as_, wp, sp, M, N, K)
    assert plan["kernel"] == "mx", plan
    ref, sabs = mx.product(aq, as_, wq, ws)
    res = oracle.check(C, ref, sabs)
    assert res.ok, f"mx {M}x{N}x{K} splits={plan['splits']}: {res.summary()}"


@pytest.mark.parametrize("name", ["dec_up_M1", "dec_up_M16", "dec_up_M64", "dec_down_M1",
                                  "dec_down_M64"])
def test_decode_llama7b_full(name):
    """The decode workloads' shapes at full size, every output (weights N x K, nn.Linear layout)."""
    w = WORKLOADS[name]
    M, N, K = w.M, w.N, w.K
    _, aq, as_, wq, ws, wp, sp = oracle_operands(M, N, K, w.seed_a)
    C, plan = run_decode(aq, as_, wp, sp, M, N, K)
    ref, sabs = mx.product(aq, as_, wq, ws)
    res = oracle.check(C, ref, sabs)
    assert res.ok, f"{name} splits={plan['splits']}: {res.summary()}"


def test_split_and_unsplit_plans_are_both_covered():
    assert g.gemm_plan_describe(1, 4096, 11008, mx=True)["splits"] > 1
    assert g.gemm_plan_describe(64, 11008, 4096, mx=True)["splits"] == 1
    assert g.gemm_plan_describe(2, 256, 11008, mx=True)["splits"] > 1
    assert g.gemm_plan_describe(16, 4096, 4096, mx=True)["splits"] > 1
    # both group widths, each with a last group short of tiles, K whole and K in pieces
    seen = set()
    for M, N, K in DECODE:
        p = g.gemm_plan_describe(M, N, K, mx=True)
        tn = p["strip"] // 16
        seen.add((tn, (N // 16) % tn != 0, p["splits"] > 1))
    assert {(3, True, True), (3, True, False), (4, True, True), (4, True, False), (4, False, True)} <= seen


def test_decode_bf16_pipeline_and_ldc():
    M, N, K = 5, 4096, 4096
    A, aq, as_, wq, ws, wp, sp = oracle_operands(M, N, K, 900)
    dA, dwp, dsp = dev_bf16(A), dev_u8(wp), dev_u8(sp)
    ldc = N + 12
    C = torch.empty(M * ldc, dtype=torch.bfloat16, device="cuda")
    g.gemm_fill_launch(P(C), C.numel() * 2, 0x7FC07FC0)
    g.gemm_mx_decode_bf16(M, N, K, P(dA), K, P(dwp), P(dsp), P(C), ldc, g.current_stream_handle())
    torch.cuda.synchronize()
    c = C.cpu().view(torch.int16).numpy().view(np.uint16).reshape(M, ldc)
    ref, sabs = mx.product(aq, as_, wq, ws)
    res = oracle.check(c[:, :N], ref, sabs)
    assert res.ok, res.summary()
    assert (c[:, N:] == 0x7FC0).all()  # the padding columns are never written


def test_k_zero_and_determinism():
    C, _ = run_decode(np.zeros((2, 0), np.uint8), np.zeros((2, 1), np.uint8),
                      np.zeros(16, np.uint8), np.zeros(16, np.uint8), 2, 32, 0)
    assert (C == 0).all()
    M, N, K = 3, 2048, 11008
    _, aq, as_, wq, ws, wp, sp = oracle_operands(M, N, K, 950)
    C1, plan = run_decode(aq, as_, wp, sp, M, N, K)
    C2, _ = run_decode(aq, as_, wp, sp, M, N, K)
    assert plan["splits"] > 1 and np.array_equal(C1, C2)


def _graph_kernel_names(graph):
    paths = sorted({ln.split()[-1] for ln in open("/proc/self/maps") if "libamdhip64" in ln})
    hip = ctypes.CDLL(paths[0])
    hip.hipKernelNameRefByPtr.restype = ctypes.c_char_p
    hip.hipKernelNameRefByPtr.argtypes = [ctypes.c_void_p, ctypes.c_void_p]

    class KP(ctypes.Structure):  # hipKernelNodeParams
        _fields_ = [("blockDim", ctypes.c_uint * 3), ("extra", ctypes.c_void_p), ("func", ctypes.c_void_p),
                    ("gridDim", ctypes.c_uint * 3), ("kernelParams", ctypes.c_void_p),
                    ("sharedMemBytes", ctypes.c_uint)]
    handle = ctypes.c_void_p(graph.raw_cuda_graph())
    n = ctypes.c_size_t(0)
    assert hip.hipGraphGetNodes(handle, None, ctypes.byref(n)) == 0
    nodes = (ctypes.c_void_p * max(n.value, 1))()
    assert hip.hipGraphGetNodes(handle, nodes, ctypes.byref(n)) == 0
    names = []
    for i in range(n.value):
        kind = ctypes.c_int(-1)
        assert hip.hipGraphNodeGetType(ctypes.c_void_p(nodes[i]), ctypes.byref(kind)) == 0
        assert kind.value == 0, f"node {i} is not a kernel node (type {kind.value})"
        prm = KP()
        assert hip.hipGraphKernelNodeGetParams(ctypes.c_void_p(nodes[i]), ctypes.byref(prm)) == 0
        names.append((hip.hipKernelNameRefByPtr(prm.func, None) or b"").decode())
    return names


@pytest.mark.parametrize("entry", ["mx_decode", "mx_decode_bf16", "packed"])
def test_graph_capture_of_decode_entry_points(entry):
    """Captured on torch's capture stream, the calls record kernel nodes only (the conversion and
    the product for gemm_mx_decode_bf16), run nothing during capture, and every replay equals the
    eager result bit for bit, with other calls between replays."""
    from oracle import packed as opk
    M, N, K = 3, 2048, 4096
    A, aq, as_, wq, ws, wp, sp = oracle_operands(M, N, K, 990)
    dA = dev_bf16(A)
    daq, das, dwp, dsp = dev_u8(np.ascontiguousarray(aq)), dev_u8(as_), dev_u8(wp), dev_u8(sp)
    B = matrix("normal", K, N, seed=991, sigma=0.02)
    dP = torch.from_numpy(opk.pack(B).view(np.int16)).cuda()
    C = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def call():
        st = g.current_stream_handle()
        if entry == "mx_decode":
            g.gemm_mx_decode(M, N, K, P(daq), K, P(das), K // 32, P(dwp), P(dsp), P(C), N, st)
        elif entry == "mx_decode_bf16":
            g.gemm_mx_decode_bf16(M, N, K, P(dA), K, P(dwp), P(dsp), P(C), N, st)
        else:
            g.gemm_bf16_packed(M, N, K, P(dA), K, P(dP), P(C), N, st)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    eager = C.clone()
    g.gemm_fill_launch(P(C), C.numel() * 2, 0x7FC07FC0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph(keep_graph=True)
    with torch.cuda.graph(graph):
        call()
    torch.cuda.synchronize()
    names = _graph_kernel_names(graph)
    want = {"mx_decode": ["mx_decode_kernel"], "mx_decode_bf16": ["mx_quant_kernel", "mx_decode_kernel"],
            "packed": ["pk_decode_kernel"]}[entry]
    assert len(names) == len(want) and all(sum(w in n for n in names) == 1 for w in want), names
    assert (C.view(torch.int16) == 0x7FC0).all(), "capture ran the kernels"
    graph.instantiate()
    other = torch.empty((2, 1024), dtype=torch.bfloat16, device="cuda")
    for rep in range(3):
        g.gemm_fill_launch(P(C), C.numel() * 2, 0x7FC07FC0)
        g.gemm_bf16_packed(2, 1024, K, P(dA), K, P(dP), P(other), 1024, g.current_stream_handle())
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(C.view(torch.int16), eager.view(torch.int16)), f"replay {rep} of {entry}"


@pytest.mark.parametrize("M,N,K", [(1, 11008, 4096), (2, 4096, 11008), (1, 80, 640), (2, 1040, 1152)])
def test_fused_conversion_matches_two_launches(M, N, K):
    """For one or two rows gemm_mx_decode_bf16 converts the activations inside the product (one
    launch); its output must equal the conversion launch followed by gemm_mx_decode, bit for bit,
    and pass the oracle's check on the oracle's own conversion."""
    A, aq, as_, wq, ws, wp, sp = oracle_operands(M, N, K, 1500 + M)
    dA, dwp, dsp = dev_bf16(A), dev_u8(wp), dev_u8(sp)
    C1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    C2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    st = g.current_stream_handle()
    g.gemm_mx_decode_bf16(M, N, K, P(dA), K, P(dwp), P(dsp), P(C1), N, st)
    q = torch.empty(M * K, dtype=torch.uint8, device="cuda")
    sc = torch.empty(M * K // 32, dtype=torch.uint8, device="cuda")
    g.gemm_mx_quantize_act(M, K, P(dA), K, P(q), K, P(sc), K // 32, st)
    g.gemm_mx_decode(M, N, K, P(q), K, P(sc), K // 32, P(dwp), P(dsp), P(C2), N, st)
    torch.cuda.synchronize()
    assert torch.equal(C1.view(torch.int16), C2.view(torch.int16))
    c = C1.cpu().view(torch.int16).numpy().view(np.uint16)
    ref, sabs = mx.product(aq, as_, wq, ws)
    res = oracle.check(c, ref, sabs)
    assert res.ok, res.summary()


def test_largest_packed_mx_weight():
    # the largest weight the MX entries take: N K / 2 code bytes just under 2^31 (32-bit offsets).
    # W[n][k] = 1 where (k + 3 n) % 7 == 0, else 0 (nn.Linear layout, N x K), and integer
    # activations in [-2, 2]: both convert exactly (a weight block holding a 1 gets scale 2^-2 and
    # code 4.0; an activation block with maximum 2 gets scale 2^-7 and codes 0, +-128, +-256, with
    # maximum 1 scale 2^-8), every product and partial sum is an integer below 2^24, so C[m][n]
    # is the bf16 rounding of the sum of A[m][k] over k = -3 n (mod 7). Through
    # gemm_mx_decode_bf16 at M = 2 (the conversion inside the product).
    M, N, K = 2, 65520, 65536
    wb, sb = g.gemm_mx_packed_sizes(N, K)
    assert wb <= 2**31 - 1 and wb == N * K // 2
    A = matrix("int", M, K, seed=1600, radius=2)
    W = torch.empty((N, K), dtype=torch.bfloat16, device="cuda")
    kk = torch.arange(K, device="cuda", dtype=torch.int32)[None, :]
    for r0 in range(0, N, 2048):
        nn = torch.arange(r0, min(N, r0 + 2048), device="cuda", dtype=torch.int32)[:, None]
        W[r0:r0 + nn.shape[0]] = ((kk + 3 * nn) % 7 == 0).to(torch.bfloat16)
    del kk, nn
    s = g.current_stream_handle()
    wp = torch.empty(wb, dtype=torch.uint8, device="cuda")
    sp = torch.empty(sb, dtype=torch.uint8, device="cuda")
    g.gemm_mx_pack_weight(N, K, P(W), K, P(wp), P(sp), s)
    del W
    dA = dev_bf16(A)
    C = torch.full((M, N), 7.0, dtype=torch.bfloat16, device="cuda")
    g.gemm_mx_decode_bf16(M, N, K, P(dA), K, P(wp), P(sp), P(C), N, s)
    torch.cuda.synchronize()
    Af = oracle.bf16_to_f64(A)
    residue = np.arange(K) % 7
    sums = np.stack([Af[:, residue == c].sum(axis=1) for c in range(7)], axis=1)  # M x 7, exact
    want = oracle.bf16_rne(sums[:, (-3 * np.arange(N)) % 7])
    got = C.cpu().view(torch.int16).numpy().view(np.uint16)
    bad = np.argwhere(got != want)
    assert bad.size == 0, f"{len(bad)} mismatches, first at {bad[0].tolist()}"
    del wp, sp
    torch.cuda.empty_cache()
