"""The five synthetic GEMM workloads, named by what they are.

Each entry fixes shape, batch, operand and output formats, storage layouts,
value distribution and seed.  Leading dimensions are tight (lda = K for a
row-major A, ldb = N for a row-major B, ldb = K for a column-major B, ldc = N)
and batched problems are packed (strides M*K, K*N, M*N); tests also use padded
leading dimensions.

The first workload is the 64x128x128 f16 GEMM used as the running example on
"The PTSS Cliff" page (section "The Arithmetic of 'Fully Unrolled K'"); the
rest are synthetic shapes that exercise deep K, a square MFMA-bound product,
ragged edges in all three dimensions and a skinny, HBM-bound batch.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

from .inputs import BF16, F16, make_operands


@dataclass(frozen=True)
class Workload:
    name: str
    M: int
    N: int
    K: int
    batch: int
    in_fmt: str          # "f16" | "bf16"
    out_fmt: str         # "f32" | "f16"
    a_layout: str        # "row" | "col"
    b_layout: str        # "row" | "col"
    dist: tuple = field(default=("uniform", -1.0, 1.0))
    seed: int = 0

    @property
    def flops(self) -> int:
        return 2 * self.M * self.N * self.K * self.batch

    @property
    def bytes(self) -> int:
        """Algorithmic HBM bytes: A and B read once, C written once."""
        out_b = 4 if self.out_fmt == "f32" else 2
        return self.batch * (2 * self.M * self.K + 2 * self.K * self.N + out_b * self.M * self.N)

    def lds(self):
        """Tight leading dimensions (lda, ldb, ldc) in elements."""
        lda = self.K if self.a_layout == "row" else self.M
        ldb = self.N if self.b_layout == "row" else self.K
        return lda, ldb, self.N

    def strides(self):
        return self.M * self.K, self.K * self.N, self.M * self.N

    def operands(self):
        return make_operands(self.seed, self.batch, self.M, self.N, self.K, self.in_fmt, self.dist,
                             self.a_layout, self.b_layout)


WORKLOADS = {
    w.name: w
    for w in [
        Workload("single_f16_64x128x128", 64, 128, 128, 1, F16, "f32", "row", "row",
                 ("uniform", -1.0, 1.0), 0),
        Workload("largek_f16_256x256x8192", 256, 256, 8192, 1, F16, "f32", "row", "row",
                 ("uniform", -1.0, 1.0), 1),
        Workload("square_bf16_8192", 8192, 8192, 8192, 1, BF16, "f16", "row", "col",
                 ("normal", 1.0 / math.sqrt(8192)), 2),
        Workload("ragged_f16_1000x1500x777", 1000, 1500, 777, 1, F16, "f32", "row", "row",
                 ("uniform", -1.0, 1.0), 3),
        Workload("skinny_f16_16x16384x8192_b8", 16, 16384, 8192, 8, F16, "f32", "row", "row",
                 ("uniform", -0.5, 0.5), 4),
    ]
}

ORDER = list(WORKLOADS)
