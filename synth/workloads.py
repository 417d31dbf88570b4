"""The synthetic workloads: shapes, value distributions and seeds.

The shapes are the ones the pages measure on: square products, the Llama-7B MLP projections at
4096 prefill tokens (hidden size 4096, MLP width 11008), and decode with M = 1, 2, 16 and 64 rows
against the same MLP weights (spark-kernels post, sections "the bf16 gemm" and "the decode
kernel"; "The kernels that were there", section "The GEMV"). Trained weights are replaced by
N(0, 0.02) samples of the same shape; activations are N(0, 1). A is M x K, B is K x N, both
row-major.

Seeds: operand A of workload family ``f`` uses ``0x5EED0000 + 2 f``, operand B
``0x5EED0000 + 2 f + 1``. The decode workloads of one weight shape share a family, so the
M-row activations are the first M rows of the same stream.

The SwiGLU workloads (``glu``) are the gate and up projections of the same MLP in one product:
B is the K x 2N concatenation of the two 4096 x 11008 weights (gate columns first), C is the
M x N result silu(A Wg) * (A Wu), at the prefill and decode row counts.
"""

from __future__ import annotations

from dataclasses import dataclass

SEED_BASE = 0x5EED0000


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    sigma_a: float
    sigma_b: float
    family: int
    bound: str  # "mfma", "hbm" or "latency"
    glu: bool = False  # SwiGLU form: B is K x 2N (gate, then up), C is M x N

    @property
    def seed_a(self) -> int:
        return SEED_BASE + 2 * self.family

    @property
    def seed_b(self) -> int:
        return SEED_BASE + 2 * self.family + 1

    @property
    def b_cols(self) -> int:
        """Columns of B: N, or 2N for the SwiGLU form."""
        return 2 * self.N if self.glu else self.N

    @property
    def flops(self) -> int:
        return 2 * self.M * self.b_cols * self.K

    @property
    def bytes(self) -> int:
        """Algorithmic bytes: A and B read once, C written once, all bf16."""
        return 2 * (self.M * self.K + self.K * self.b_cols + self.M * self.N)


def _mk():
    w = [
        Workload("sq512", 512, 512, 512, 1.0, 1.0, 0, "latency"),
        Workload("sq4096", 4096, 4096, 4096, 1.0, 1.0, 1, "mfma"),
        Workload("sq8192", 8192, 8192, 8192, 1.0, 1.0, 2, "mfma"),
        Workload("sq16384", 16384, 16384, 16384, 1.0, 1.0, 3, "mfma"),
        Workload("mlp_up", 4096, 11008, 4096, 1.0, 0.02, 4, "mfma"),
        Workload("mlp_down", 4096, 4096, 11008, 1.0, 0.02, 5, "mfma"),
    ]
    for m in (1, 2, 16, 64):
        w.append(Workload(f"dec_up_M{m}", m, 11008, 4096, 1.0, 0.02, 6, "hbm"))
    for m in (1, 2, 16, 64):
        w.append(Workload(f"dec_down_M{m}", m, 4096, 11008, 1.0, 0.02, 7, "hbm"))
    w.append(Workload("glu_prefill", 4096, 11008, 4096, 1.0, 0.02, 8, "mfma", glu=True))
    for m in (1, 16, 64):
        w.append(Workload(f"glu_dec_M{m}", m, 11008, 4096, 1.0, 0.02, 9, "hbm", glu=True))
    return {x.name: x for x in w}


WORKLOADS = _mk()


def workload(name: str) -> Workload:
    return WORKLOADS[name]
