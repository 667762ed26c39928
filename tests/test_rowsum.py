"""Row sums on the GPU against the oracle, through the C ABI.

Acceptance per row (float64): |out - ref| <= C * 2^-24 * sum_c |x|, the bound
of any float32 summation order.  The printed examples of "A Dumb Triton Runtime
Error" ("What I ran": the 2x3 matrix of ones gives [3.0, 3.0], also with the
output pre-filled with 100.0) are checked exactly.
"""

import numpy as np
import pytest

from gpu_util import say
from workloads.inputs import BF16, F16, round_f64_to_bits

import tiled_shared_memory_amd as tsm

pytestmark = pytest.mark.gpu

CODE = {"f32": tsm.TSM_ROWSUM_F32, F16: tsm.TSM_ROWSUM_F16, BF16: tsm.TSM_ROWSUM_BF16}


def storage(vals, fmt):
    """Flat storage of float64 values: float32, or rounded 16-bit patterns."""
    if fmt == "f32":
        return np.ascontiguousarray(vals, dtype=np.float32).reshape(-1)
    return round_f64_to_bits(np.asarray(vals, dtype=np.float64), fmt).reshape(-1)


def run_rowsum(X, R, C, rs, cs, fmt, fill=np.nan, kernel=None):
    import torch

    if fmt == "f32":
        x = torch.from_numpy(X.view(np.float32).copy()).cuda()
    else:
        x = torch.from_numpy(X.view(np.int16).copy()).cuda()
    out = torch.full((max(R, 1) + 4,), float(fill), dtype=torch.float32, device="cuda")
    if kernel is not None:
        name = tsm.tsm_rowsum_kernel_name(R, C, x, rs, cs, CODE[fmt], out)
        assert name == kernel, f"routed to {name}, expected {kernel}"
    tsm.rowsum(R, C, x, rs, cs, CODE[fmt], out, 0)
    torch.cuda.synchronize()
    host = out.cpu().numpy().astype(np.float64)
    assert np.all(np.isnan(host[R:])) if np.isnan(fill) else np.all(host[R:] == fill)  # nothing past R written
    return host[:R]


def check_rows(got, ref, S, C, what):
    assert np.all(np.isfinite(got)), what
    bnd = C * 2.0 ** -24 * S
    bad = np.flatnonzero(np.abs(got - ref) > bnd)
    assert bad.size == 0, f"{what}: row {bad[0]} got {got[bad[0]]!r} ref {ref[bad[0]]!r} bound {bnd[bad[0]]!r}"
    return float(np.max(np.abs(got - ref))) if got.size else 0.0


@pytest.mark.parametrize("fmt", ["f32", F16, BF16])
@pytest.mark.parametrize("fill", [0.0, 100.0])
def test_printed_example_ones(orc, fmt, fill):
    """2x3 ones -> [3.0, 3.0] exactly; the output's previous contents (100.0) do not leak in."""
    say(f"[gpu] rowsum ones 2x3 {fmt} fill {fill}")
    got = run_rowsum(storage(np.ones((2, 3)), fmt), 2, 3, 3, 1, fmt, fill=fill)
    assert np.array_equal(got, [3.0, 3.0])


def test_page_shape_8x1000_random(orc):
    """The page's 8 x 1000 random float32 rows: within the bound (the page saw errors of about 4e-6)."""
    x = np.random.default_rng(21).standard_normal((8, 1000))
    X = storage(x, "f32")
    say("[gpu] rowsum 8x1000")
    got = run_rowsum(X, 8, 1000, 1000, 1, "f32", kernel="rowsum_wave_vec16")
    ref, S = orc.rowsum(X, 8, 1000, 1000, 1, "f32")
    err = check_rows(got, ref, S, 1000, "8x1000")
    say(f"[gpu] rowsum 8x1000 max abs error {err:.3g}")


CASES = [
    # R, C, row_stride, col_stride, fmt, expected kernel
    (4096, 4096, 4096, 1, "f32", "rowsum_wave_vec16"),
    (3000, 2051, 2056, 1, F16, "rowsum_wave_vec16"),      # padded rows, ragged tail
    (3000, 999, 999, 1, BF16, "rowsum_wave_elem"),        # row starts not 16-byte aligned
    (2500, 700, 1, 2500, "f32", "rowsum_wave_elem"),      # the transposed view
    (2100, 300, 1000, 3, F16, "rowsum_wave_elem"),        # every third column
    (6, (1 << 20) + 3, (1 << 20) + 8, 1, "f32", "rowsum_block_vec16"),
    (5, 300001, 300001, 1, BF16, "rowsum_block_elem"),
    (1000, 1, 1, 1, "f32", "rowsum_wave_elem"),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[0]}x{c[1]}_{c[4]}_{c[5]}")
def test_rowsum_against_oracle(orc, case):
    R, C, rs, cs, fmt, kernel = case
    span = (R - 1) * rs + (C - 1) * cs + 1
    rng = np.random.default_rng(R + C)
    X = storage(rng.uniform(-1.0, 1.0, span), fmt)
    say(f"[gpu] rowsum {case}")
    got = run_rowsum(X, R, C, rs, cs, fmt, kernel=kernel)
    ref, S = orc.rowsum(X, R, C, rs, cs, fmt)
    check_rows(got, ref, S, C, str(case))
    # the reduction order is fixed: bitwise reproducible
    assert np.array_equal(run_rowsum(X, R, C, rs, cs, fmt), got)


@pytest.mark.parametrize("fmt", ["f32", F16, BF16])
def test_rowsum_integer_exact(orc, fmt):
    """Integer entries: every float32 partial sum is exact, so the GPU equals the oracle bit for bit."""
    R, C = 2048, 5000
    vals = np.random.default_rng(22).integers(-8, 9, (R, C)).astype(np.float64)
    X = storage(vals, fmt)
    say(f"[gpu] rowsum integer {fmt}")
    got = run_rowsum(X, R, C, C, 1, fmt)
    assert np.array_equal(got, vals.sum(axis=1))


def test_rowsum_zero_columns_writes_zeros(orc):
    say("[gpu] rowsum C=0")
    got = run_rowsum(np.zeros(4, np.float32), 3, 0, 4, 1, "f32", fill=100.0)
    assert np.array_equal(got, [0.0, 0.0, 0.0])


def test_rowsum_more_rows_than_one_launch_covers(orc):
    """2^26 + 5 single-element rows: more work-items than one launch may have (64 per row), so the rows are
    split over two launches.  A one-element row sums to that element exactly."""
    import torch

    R = (1 << 26) + 5
    x = torch.arange(R, dtype=torch.float32, device="cuda")
    x = (x % 1021) - 510.0  # exact small integers
    out = torch.full((R,), float("nan"), dtype=torch.float32, device="cuda")
    assert tsm.tsm_rowsum_kernel_name(R, 1, x.data_ptr(), 1, 1, tsm.TSM_ROWSUM_F32, out.data_ptr()).startswith("rowsum_wave")
    say(f"[gpu] rowsum {R} rows of one element")
    tsm.rowsum(R, 1, x.data_ptr(), 1, 1, tsm.TSM_ROWSUM_F32, out.data_ptr(), 0)
    torch.cuda.synchronize()
    assert bool(torch.equal(out, x))
