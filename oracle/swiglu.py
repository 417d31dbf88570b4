"""Oracle for the SwiGLU-fused gate/up product (CPU, float64).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the package smoke check and by the
benchmark's CPU-baseline leg, never by the GPU library or its binding. It shares no code with
the GPU path.

What is computed. The up and gate projections of a Llama MLP are two products of the same
activations A (M x K): g = A Wg and u = A Wu, each N wide. SwiGLU multiplies the SiLU of the
gate by the up projection, element by element (spark-kernels post, "the memory-bound kernels":
the fused SwiGLU kernel replaces the two kernels of F.silu(g) * u; the post's opening paragraph
lists SwiGLU among the pieces of a Llama decoder block). SiLU is x * sigmoid(x) = x / (1 + e^-x).
The gate and up weights are the two halves of one K x 2N row-major matrix B: columns 0 .. N-1
are Wg and columns N .. 2N-1 are Wu (the gate and up projections concatenated along their
output dimension, the layout of a merged gate/up weight).

    h[i][j] = silu(g[i][j]) * u[i][j],   g = sum_k a[i][k] b[k][j],   u = sum_k a[i][k] b[k][N+j]

all in float64 (g and u come from the plain float64 product oracle in oracle.c).

Reading of the fusion: the product that makes g and u also applies the activation, so g and u
are the float32 accumulators and only h is rounded to bf16, once. (An unfused path rounds g and
u to bf16 first; the acceptance bound below is tight enough to reject that.)

Acceptance bound, derived from the product oracle's own allowance. The product check allows a
float32 result g' with |g' - g| <= dg = 2^-16 * sum_k |a b| (and du for u). With
L = sup |silu'| (SILU_SLOPE_MAX), first and second order:
    |silu(g') u' - silu(g) u| <= L dg (|u| + du) + |silu(g)| du.
Evaluating silu and the product in float32 adds a relative error far below 2^-20 of
(|silu(g)| + L dg)(|u| + du). Rounding the float32 value h' to bf16 adds at most 2^-8 |h'|, and
|h'| <= |h| + E, so
    |c - h| <= 2^-8 |h| + (1 + 2^-8) E,
    E = L dg (|u| + du) + |silu(g)| du + 2^-20 (|silu(g)| + L dg)(|u| + du),
for every element (NaN or Inf fails), and ||c - h||_F / ||h||_F <= 4e-3 over what is checked,
as for the plain product.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import REL_FROB_MAX, bf16_to_f64, gemm_rows

# sup over x of |d/dx x sigmoid(x)|: the slope sigmoid(x) (1 + x (1 - sigmoid(x))) peaks at
# 1.09984 near x = 2.3994 (and dips to -0.09984 near x = -2.3994); rounded up.
SILU_SLOPE_MAX = 1.1


def silu(x) -> np.ndarray:
    """x / (1 + e^-x) in float64; saturates to x for large x and to -0 for very negative x."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def combine(g, sg, u, su):
    """(h, slack) from the gate and up products and their sums of |a b| (all float64)."""
    g, sg, u, su = (np.asarray(v, dtype=np.float64) for v in (g, sg, u, su))
    dg = np.ldexp(sg, -16)
    du = np.ldexp(su, -16)
    s = silu(g)
    h = s * u
    au = np.abs(u) + du
    e = (SILU_SLOPE_MAX * dg * au + np.abs(s) * du
         + np.ldexp((np.abs(s) + SILU_SLOPE_MAX * dg) * au, -20))
    return h, (1.0 + 2.0 ** -8) * e


def swiglu_rows(A: np.ndarray, B: np.ndarray, row0: int, nrows: int, N: int, K: int,
                threads: int | None = None):
    """(h, slack) for rows row0 .. row0 + nrows - 1 of h = silu(A B[:, :N]) * (A B[:, N:2N])."""
    B = np.asarray(B)
    if B.ndim != 2 or B.shape[1] < 2 * N:
        raise ValueError("B must hold 2N columns: gate then up")
    g, sg = gemm_rows(A, B[:, :N], row0, nrows, N, K, True, threads)
    u, su = gemm_rows(A, B[:, N:2 * N], row0, nrows, N, K, True, threads)
    return combine(g, sg, u, su)


def swiglu(A: np.ndarray, B: np.ndarray, M: int | None = None, N: int | None = None,
           K: int | None = None, threads: int | None = None):
    """(h, slack) for the whole M x N output."""
    M = np.asarray(A).shape[0] if M is None else M
    K = np.asarray(A).shape[1] if K is None else K
    N = np.asarray(B).shape[1] // 2 if N is None else N
    return swiglu_rows(A, B, 0, M, N, K, threads)


@dataclass
class BoundCheck:
    checked: int
    failures: int
    nonfinite: int
    worst_at: tuple
    worst_ratio: float
    rel_frob: float

    @property
    def ok(self) -> bool:
        return self.failures == 0 and self.rel_frob <= REL_FROB_MAX

    def summary(self) -> dict:
        return {"checked": self.checked, "failures": self.failures, "nonfinite": self.nonfinite,
                "worst_ratio": self.worst_ratio, "worst_at": list(self.worst_at),
                "rel_frob": self.rel_frob}


def check(C: np.ndarray, h: np.ndarray, slack: np.ndarray) -> BoundCheck:
    """|c - h| <= 2^-8 |h| + slack element-wise (NaN/Inf fail) and the relative Frobenius bound,
    for bf16 bits C against the float64 (h, slack) of combine()."""
    h = np.asarray(h, dtype=np.float64)
    if h.ndim == 1:
        h = h.reshape(1, -1)
    slack = np.asarray(slack, dtype=np.float64).reshape(h.shape)
    C = np.asarray(C)
    if C.ndim == 1:
        C = C.reshape(1, -1)
    if C.shape[0] < h.shape[0] or C.shape[1] < h.shape[1]:
        raise ValueError("shape mismatch")
    c = bf16_to_f64(C[: h.shape[0], : h.shape[1]])
    finite = np.isfinite(c)
    err = np.abs(c - h)
    allow = np.ldexp(np.abs(h), -8) + slack
    bad = ~(err <= allow)  # NaN compares false, so it fails
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = np.where(finite, err / np.where(allow > 0, allow, np.inf), np.inf)
        ratio = np.where((allow == 0) & (err == 0), 0.0, ratio)
    if ratio.size:
        at = np.unravel_index(int(np.argmax(ratio)), ratio.shape)
        worst = float(ratio[at])
    else:
        at, worst = (0, 0), 0.0
    ref_sq = float(np.sum(h * h))
    err_sq = float(np.sum(np.where(finite, err, 0.0) ** 2))
    if ref_sq == 0.0:
        rel = 0.0 if err_sq == 0.0 else float("inf")
    else:
        rel = float(np.sqrt(err_sq / ref_sq))
    if not finite.all():
        rel = float("inf")
    return BoundCheck(int(h.size), int(bad.sum()), int((~finite).sum()), tuple(int(v) for v in at),
                      worst, rel)
