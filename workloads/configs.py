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

import numpy as np

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


@dataclass(frozen=True)
class GroupedWorkload:
    """A grouped product: `groups` problems of capacity M rows, problem g using its first rows()[g] rows.

    Shaped like a mixture-of-experts layer (the A[expert, :tokens, :] slice of
    the Intel XPU Triton README): `tokens` routed rows are spread over the
    groups by a seeded multinomial draw whose probabilities come from a
    symmetric Dirichlet(2) draw, so the groups are unevenly loaded; each count
    is capped at the capacity M.
    """
    name: str
    groups: int
    M: int               # row capacity of every group
    N: int
    K: int
    tokens: int          # rows routed in total, before capping
    in_fmt: str
    out_fmt: str
    a_layout: str
    b_layout: str
    dist: tuple = field(default=("uniform", -1.0, 1.0))
    seed: int = 0

    @property
    def batch(self) -> int:
        return self.groups

    def rows(self) -> np.ndarray:
        rng = np.random.default_rng([self.seed, 7])
        p = rng.dirichlet([2.0] * self.groups)
        return np.minimum(rng.multinomial(self.tokens, p), self.M).astype(np.int32)

    @property
    def flops(self) -> int:
        return 2 * int(self.rows().sum()) * self.N * self.K

    @property
    def bytes(self) -> int:
        """Algorithmic HBM bytes: the valid rows of A, every B, the valid rows of C."""
        out_b = 4 if self.out_fmt == "f32" else 2
        m = int(self.rows().sum())
        return 2 * m * self.K + self.groups * 2 * self.K * self.N + out_b * m * self.N

    def lds(self):
        lda = self.K if self.a_layout == "row" else self.M
        ldb = self.N if self.b_layout == "row" else self.K
        return lda, ldb, self.N

    def strides(self):
        return self.M * self.K, self.K * self.N, self.M * self.N

    def operands(self):
        return make_operands(self.seed, self.groups, self.M, self.N, self.K, self.in_fmt, self.dist,
                             self.a_layout, self.b_layout)


# Measured beside the five workloads above; not one of them.
GROUPED = {
    w.name: w
    for w in [
        GroupedWorkload("moe_bf16_e8_t16384_n2048_k4096", 8, 4096, 2048, 4096, 16384, BF16, "f16", "row", "col",
                        ("normal", 1.0 / 64.0), 5),
    ]
}


@dataclass(frozen=True)
class RowsumWorkload:
    """Row sums of an R x C matrix (contiguous rows), values uniform[-1, 1]."""
    name: str
    R: int
    C: int
    fmt: str             # "f32" | "f16" | "bf16"
    seed: int = 0

    @property
    def flops(self) -> int:
        return self.R * self.C  # one add per element

    @property
    def bytes(self) -> int:
        """Algorithmic HBM bytes: X read once, the R float32 sums written once."""
        return self.R * self.C * (4 if self.fmt == "f32" else 2) + 4 * self.R

    def operand(self):
        """Flat storage: float32 values, or 16-bit patterns (the shared generator, rows of C)."""
        from .inputs import draw_matrix_bits

        if self.fmt == "f32":
            rng = np.random.default_rng([self.seed, 9])
            return rng.uniform(-1.0, 1.0, self.R * self.C).astype(np.float32)
        return draw_matrix_bits(self.seed, 0, 0, ("uniform", -1.0, 1.0), self.R, self.C, self.fmt).reshape(-1)


# Measured beside the five workloads above; not one of them: one problem a
# little over one round of 256 x 256 tiles (272 = 256 + 16), the case the
# hybrid split covers.
PARTIAL = {
    w.name: w
    for w in [
        Workload("partial_bf16_4352x4096x8192", 4352, 4096, 8192, 1, BF16, "f16", "row", "col",
                 ("normal", 1.0 / math.sqrt(8192)), 8),
    ]
}


ROWSUM = {
    w.name: w
    for w in [
        # 1 GiB of float32: many rows, one wave each
        RowsumWorkload("rowsum_f32_16384x16384", 16384, 16384, "f32", 6),
        # the page's 8 x 1000 float32 rows (launch-bound)
        RowsumWorkload("rowsum_f32_8x1000", 8, 1000, "f32", 7),
    ]
}


def lookup(name: str):
    """A workload of any kind by name."""
    for table in (WORKLOADS, GROUPED, PARTIAL, ROWSUM):
        if name in table:
            return table[name]
    raise KeyError(name)
