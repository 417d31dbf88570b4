"""Oracle for the block-scaled (MX) decode product (CPU, float64 and exact integer work).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check and by the
benchmark's CPU-baseline leg, never by the GPU library or its binding. It shares no code with
the GPU path.

Formats, from the OCP Microscaling Formats (MX) specification v1.0. A block of 32 consecutive
elements along K shares one scale X = 2^(e - 127), stored as an E8M0 byte e (255 is NaN); each
element is a small float code P, and the block holds the values X * P.
  * E2M1 (FP4): sign, 2 exponent bits (bias 1), 1 mantissa bit; magnitudes 0, 0.5, 1, 1.5, 2, 3,
    4, 6; no Inf or NaN. Largest exponent emax = 2.
  * E4M3 (FP8): sign, 4 exponent bits (bias 7), 3 mantissa bits; subnormals below 2^-6; largest
    normal 448 (S.1111.110); S.1111.111 is NaN; no Inf. emax = 8.
The pages measure block-scaled low-precision GEMMs on pre-quantized operands (the "Benchmarks"
page of gemm3, "Implementations": packed NVFP4 operands with E4M3 scales, dense W4A4); the MX
formats are the ones gfx950's scaled matrix instructions take.

Conversion of a block V (the specification's quantisation): the shared exponent is
floor(log2(max |V_i|)) - emax of the element format, clamped to E8M0's range [-127, 127]; each
element is V_i / X rounded to the element format, nearest with ties to even, saturating at the
largest magnitude. An all-zero block takes the smallest scale (byte 0) and zero elements. The
bf16 inputs are exact in float64 and X is a power of two, so every decision here is exact.

The product (weight-only quantised decode, the weights W in the nn.Linear layout N x K):
    ref[m][n] = sum_k a[m][k] w[n][k],  sabs[m][n] = sum_k |a[m][k] w[n][k]|
over the dequantised values of the MXFP8 activations A (M x K) and the MXFP4 weights W, in
float64 (every product of an E4M3 and an E2M1 value times two powers of two is exact). The
acceptance check is the product oracle's: |c - ref| <= 2^-8 |ref| + 2^-16 sabs element-wise and a
relative Frobenius error <= 4e-3 (oracle.check).

The packed weight layout the library's decode kernel reads (weights quantised once, ahead of
the product) is defined by pack_weights below.
"""

from __future__ import annotations

import math

import numpy as np

BLOCK = 32  # elements per shared scale

FORMATS = {
    # name: (exponent bits, mantissa bits, bias, largest magnitude, emax, has NaN code)
    "e2m1": (2, 1, 1, 6.0, 2, False),
    "e4m3": (4, 3, 7, 448.0, 8, True),
}


def element_value(code: int, fmt: str) -> float:
    """Value of one element code (sign bit on top), from the bit fields."""
    eb, mb, bias, _, _, has_nan = FORMATS[fmt]
    nbits = 1 + eb + mb
    code &= (1 << nbits) - 1
    sign = -1.0 if code >> (nbits - 1) else 1.0
    e = (code >> mb) & ((1 << eb) - 1)
    m = code & ((1 << mb) - 1)
    if has_nan and e == (1 << eb) - 1 and m == (1 << mb) - 1:
        return float("nan")
    if e == 0:
        return sign * math.ldexp(m, 1 - bias - mb)
    return sign * math.ldexp((1 << mb) + m, e - bias - mb)


def value_table(fmt: str) -> np.ndarray:
    eb, mb = FORMATS[fmt][:2]
    return np.array([element_value(c, fmt) for c in range(1 << (1 + eb + mb))])


def scale_value(e: int) -> float:
    """E8M0: 2^(e - 127); 255 is NaN."""
    return float("nan") if e == 255 else math.ldexp(1.0, int(e) - 127)


def encode_element(x: float, fmt: str) -> int:
    """x (already divided by the block scale) to the element code: nearest, ties to even,
    saturating at the largest magnitude."""
    eb, mb, bias, vmax, _, _ = FORMATS[fmt]
    nbits = 1 + eb + mb
    sign = 1 if (x < 0 or (x == 0 and math.copysign(1.0, x) < 0)) else 0
    a = abs(x)
    if a >= vmax:
        mag = vmax
    else:
        # quantum: 2^(exponent - mb), with the exponent at least the smallest normal's
        e = max(math.frexp(a)[1] - 1 if a > 0 else 1 - bias, 1 - bias)
        q = math.ldexp(1.0, e - mb)
        r = a / q                      # exact: q is a power of two
        n = math.floor(r)
        frac = r - n
        if frac > 0.5 or (frac == 0.5 and n % 2 == 1):
            n += 1
        mag = min(n * q, vmax)
    # encode the (exactly representable) magnitude
    if mag == 0:
        return sign << (nbits - 1)
    e = math.frexp(mag)[1] - 1
    if e < 1 - bias:                   # subnormal
        field_e, field_m = 0, int(mag / math.ldexp(1.0, 1 - bias - mb))
    else:
        field_e = e + bias
        field_m = int(mag / math.ldexp(1.0, e - mb)) - (1 << mb)
    return (sign << (nbits - 1)) | (field_e << mb) | field_m


def _widen_bf16(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def encode_array(x: np.ndarray, fmt: str) -> np.ndarray:
    """encode_element over an array (the same steps, element by element, vectorised)."""
    eb, mb, bias, vmax, _, _ = FORMATS[fmt]
    nbits = 1 + eb + mb
    x = np.asarray(x, dtype=np.float64)
    sign = np.signbit(x).astype(np.uint8)
    a = np.abs(x)
    e = np.maximum(np.frexp(a)[1] - 1, 1 - bias)
    q = np.ldexp(1.0, e - mb)
    n = np.rint(a / q)                 # nearest, ties to even; a / q is exact
    mag = np.where(a >= vmax, vmax, np.minimum(n * q, vmax))
    e2 = np.frexp(mag)[1] - 1
    sub = (mag == 0) | (e2 < 1 - bias)
    field_e = np.where(sub, 0, e2 + bias)
    field_m = np.where(sub, mag / math.ldexp(1.0, 1 - bias - mb),
                       mag / np.ldexp(1.0, e2 - mb) - (1 << mb))
    code = (sign.astype(np.int64) << (nbits - 1)) | (field_e.astype(np.int64) << mb) | field_m.astype(np.int64)
    return code.astype(np.uint8)


def quantize(X: np.ndarray, fmt: str, cols: int | None = None):
    """MX conversion of the rows of a bf16 bit matrix, blocks of 32 along each row.

    Returns (codes uint8 [rows, cols], scales uint8 [rows, cols / 32]); cols % 32 == 0."""
    X = np.asarray(X)
    rows = X.shape[0]
    cols = X.shape[1] if cols is None else cols
    if cols % BLOCK:
        raise ValueError("cols must be a multiple of 32")
    v = _widen_bf16(X[:, :cols]).reshape(rows, cols // BLOCK, BLOCK)
    emax = FORMATS[fmt][4]
    amax = np.max(np.abs(v), axis=2)
    se = np.clip(np.frexp(amax)[1] - 1 - emax, -127, 127)
    se = np.where(amax == 0, -127, se)          # all-zero block: smallest scale
    scaled = np.ldexp(v, -se[:, :, None])       # exact: a power-of-two scale
    codes = encode_array(scaled, fmt).reshape(rows, cols)
    return codes, (se + 127).astype(np.uint8)


def dequantize(codes: np.ndarray, scales: np.ndarray, fmt: str) -> np.ndarray:
    """float64 values X * P of a code matrix and its per-32 scales."""
    table = value_table(fmt)
    vals = table[np.asarray(codes, dtype=np.int64)]
    sc = np.array([scale_value(e) for e in range(256)])[np.asarray(scales, dtype=np.int64)]
    return vals * np.repeat(sc, BLOCK, axis=1)[:, : vals.shape[1]]


def product(Aq, As, Wq, Ws):
    """(ref, sabs) of deq(A) deq(W)^T in float64: A MXFP8 (M x K), W MXFP4 (N x K)."""
    a = dequantize(Aq, As, "e4m3")
    w = dequantize(Wq, Ws, "e2m1")
    return a @ w.T, np.abs(a) @ np.abs(w).T


# ---- the packed weight layout ------------------------------------------------------------------
# Column tile t holds the 16 weight rows n = 16 t .. 16 t + 15; k-step s holds k = 128 s .. +127.
# The codes of (t, s) are one 1024-byte block at byte 1024 (t * KS + s), KS = K / 128. Inside it,
# lane l (0 .. 63) owns bytes 16 l .. 16 l + 15: row n = 16 t + l % 16, the 32 codes of
# k = 128 s + 32 (l // 16) + j, j = 0 .. 31, two per byte, the even j in the low nibble.
# The scales of (t, s) are 64 bytes, lane l's byte being the scale of that same 32-element
# block; four consecutive k-steps share 256 bytes, lane l owning 4 bytes (one per k-step):
# scale (t, s, l) is at byte 256 (t * KQ + s // 4) + 4 l + s % 4, KQ = ceil(KS / 4), and the bytes
# of k-steps past the last (when KS % 4 != 0) are zero.

def packed_sizes(N: int, K: int) -> tuple[int, int]:
    ks = K // 128
    return (N // 16) * ks * 1024, (N // 16) * (-(-ks // 4)) * 256


def pack_weights(codes: np.ndarray, scales: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """The packed (codes, scales) byte arrays of an N x K MXFP4 weight (N % 16 == K % 128 == 0),
    by the layout above: [t][s][lane = 16 g + i][16 bytes] with n = 16 t + i and the k-block g
    of step s; scales [t][s // 4][lane][s % 4]."""
    codes = np.asarray(codes, dtype=np.uint8)
    N, K = codes.shape
    if N % 16 or K % 128:
        raise ValueError("N must be a multiple of 16 and K of 128")
    T, ks = N // 16, K // 128
    kq = -(-ks // 4)
    c = (codes & 0xF).reshape(T, 16, ks, 4, 32).transpose(0, 2, 3, 1, 4)   # [t, s, g, i, j]
    wp = (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8).reshape(-1)
    sc = np.zeros((T, 16, kq * 4, 4), dtype=np.uint8)                      # [t, i, s, g]
    sc[:, :, :ks, :] = np.asarray(scales, dtype=np.uint8).reshape(T, 16, ks, 4)
    sp = sc.reshape(T, 16, kq, 4, 4).transpose(0, 2, 4, 1, 3).reshape(-1)  # [t, q, g, i, s % 4]
    return wp, sp
