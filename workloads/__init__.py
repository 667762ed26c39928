"""Seeded synthetic inputs and workload definitions shared by tests and bench.

Holds no GEMM arithmetic; see ``inputs`` for the generator contract.
"""

from .configs import (GROUPED, ORDER, PARTIAL, ROWSUM, WORKLOADS, GroupedWorkload, RowsumWorkload, Workload,  # noqa: F401
                      lookup)
from .inputs import (BF16, F16, bits_to_f64, integer_operands, make_operands,  # noqa: F401
                     round_f64_to_bits)
