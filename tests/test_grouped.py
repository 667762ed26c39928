"""Grouped products (per-problem row counts in device memory) against the oracle, through the C ABI.

Problem g computes C_g[0:m_g] = A_g[0:m_g] . B_g with m_g = rows[g] clamped to
[0, M]; rows m_g .. M-1 of C_g and the ld padding must stay untouched (C is
pre-filled with NaN).  Also: plain products whose M is not a multiple of 256 on
the large-tile kernels, which mask rows past M the same way.
"""

import numpy as np
import pytest

from gpu_util import DTYPE, LAYOUT, c_view, check, say, to_device, alloc_c
from workloads.inputs import BF16, F16, integer_operands, make_operands

import tiled_shared_memory_amd as tsm

pytestmark = pytest.mark.gpu


def run_grouped(A, B, M, N, K, in_fmt, out_fmt, rows, *, a_layout="row", b_layout="row", lda=None, ldb=None,
                ldc=None, kernel=None):
    import torch

    groups = len(rows)
    lda = lda if lda is not None else (K if a_layout == "row" else M)
    ldb = ldb if ldb is not None else (N if b_layout == "row" else K)
    ldc = ldc if ldc is not None else N
    sA, sB, sC = A.size // groups, B.size // groups, M * ldc
    a_buf, a_ptr = to_device(A)
    b_buf, b_ptr = to_device(B)
    r = torch.tensor(np.asarray(rows, dtype=np.int32), device="cuda")
    c = alloc_c(groups, M, N, ldc, sC, out_fmt, fill=float("nan"))
    args = (M, N, K, a_ptr, lda, LAYOUT[a_layout], sA, b_ptr, ldb, LAYOUT[b_layout], sB, c, ldc, sC, r, groups,
            DTYPE[(in_fmt, out_fmt)])
    if kernel is not None:
        name = tsm.tsm_gemm_grouped_kernel_name(*args)
        assert name is not None and name.startswith(kernel), f"routed to {name}, expected {kernel}"
    tsm.gemm_grouped(*args, 0)
    torch.cuda.synchronize()
    host = c.cpu().numpy().astype(np.float64)
    # the ld padding of every row and the tail after the last row stay NaN
    for g in range(groups):
        for i in range(M):
            o = g * sC + i * ldc
            assert np.all(np.isnan(host[o + N:o + ldc])), f"ld padding written, group {g} row {i}"
    return c_view(c, groups, M, N, ldc, sC, out_fmt)


def check_grouped(orc, C, A, B, M, N, K, fmt, out_fmt, rows, *, a_layout="row", b_layout="row", lda=None,
                  ldb=None, what=""):
    ref = orc.gemm_grouped(A, B, M, N, K, fmt, rows, lda=lda, ldb=ldb, a_layout=a_layout, b_layout=b_layout)
    for g, (Cr, S) in enumerate(ref):
        m = Cr.shape[0]
        check(C[g, :m], Cr, S, K, out_fmt, f"{what} group {g} (m={m})")
        assert np.all(np.isnan(C[g, m:])), f"{what}: group {g} rows past m={m} were written"


EDGE_ROWS = [600, 0, 257, 1, -7, 700, 256, 255]


@pytest.mark.parametrize("variant,b_layout", [("tile_256x256x64_mi16_st", "col"), ("tile_256x256x64_mi16", "col"),
                                              ("tile_256x256x32_mi16", "col"),
                                              ("tile_256x256x32_mi16_nn", "row"), ("tile_256x256x64_mi16_nn", "row"),
                                              ("tile_256x256x32_mi32", "col")])
@pytest.mark.parametrize("in_fmt,out_fmt", [(BF16, "f16"), (F16, "f32")])
def test_grouped_tile_variants(orc, monkeypatch, variant, b_layout, in_fmt, out_fmt):
    """Every large-tile variant with counts below 0, 0, 1, 255..257, M and above M."""
    monkeypatch.setenv("TSM_GEMM_KERNEL", variant)
    M, N, K = 600, 512, 256
    rows = EDGE_ROWS
    A, B = make_operands(41, len(rows), M, N, K, in_fmt, ("uniform", -1.0, 1.0), "row", b_layout)
    say(f"[gpu] grouped {variant} {in_fmt}->{out_fmt} rows={rows}")
    C = run_grouped(A, B, M, N, K, in_fmt, out_fmt, rows, b_layout=b_layout, kernel=variant)
    check_grouped(orc, C, A, B, M, N, K, in_fmt, out_fmt, rows, b_layout=b_layout, what=variant)


@pytest.mark.parametrize("a_layout,b_layout", [("row", "row"), ("col", "row"), ("row", "col"), ("col", "col")])
@pytest.mark.parametrize("shape", [(100, 72, 48), (130, 70, 51)], ids=["vec8", "odd"])
def test_grouped_masked(orc, a_layout, b_layout, shape):
    """The general kernel: any layout, ragged sizes, 16-byte and element loads."""
    M, N, K = shape
    rows = [-1, 0, 33, M, M + 50, 1]
    A, B = make_operands(M + N + K, len(rows), M, N, K, F16, ("uniform", -1.0, 1.0), a_layout, b_layout)
    say(f"[gpu] grouped masked {shape} {a_layout}/{b_layout}")
    C = run_grouped(A, B, M, N, K, F16, "f32", rows, a_layout=a_layout, b_layout=b_layout, kernel="masked_")
    check_grouped(orc, C, A, B, M, N, K, F16, "f32", rows, a_layout=a_layout, b_layout=b_layout, what="masked")


@pytest.mark.parametrize("M,variant", [(16, "skinny_m16_n64_k64"), (64, "skinny_m64_n64_k64"),
                                       (128, "skinny_m128_n64_k64"), (32, "skinny_m32_n256_k64"),
                                       (32, "skinny_m32_n128_k64"), (128, "skinny_m128_n128_k64")])
def test_grouped_skinny(orc, monkeypatch, M, variant):
    """Grouped rows on the streaming kernel: counts past M, zero and negative, ragged inside a 16-row block."""
    monkeypatch.setenv("TSM_GEMM_KERNEL", variant)
    N, K = 512, 512
    rows = [0, 1, 7, M, M + 20, -3, M - 1, 17]
    A, B = make_operands(43 + M, len(rows), M, N, K, F16, ("uniform", -0.5, 0.5))
    say(f"[gpu] grouped {variant} rows={rows}")
    C = run_grouped(A, B, M, N, K, F16, "f32", rows, kernel=variant)
    check_grouped(orc, C, A, B, M, N, K, F16, "f32", rows, what=variant)


def test_grouped_deep_k_avoids_split_k(orc):
    M, N, K = 160, 64, 4096
    rows = [160, 17, 0]
    A, B = make_operands(44, len(rows), M, N, K, F16, ("uniform", -1.0, 1.0))
    say("[gpu] grouped deep K")
    C = run_grouped(A, B, M, N, K, F16, "f32", rows, kernel="masked_")
    check_grouped(orc, C, A, B, M, N, K, F16, "f32", rows, what="deep K")


def test_grouped_moe_shape_sampled(orc):
    """8 experts x up to 2048 tokens, 1024 x 512 weights stored K-contiguous (bf16 -> f16) on the 256 x 256
    kernel: sampled cells of every group against the oracle, every row past the counts untouched."""
    E, M, N, K = 8, 2048, 1024, 512
    rng = np.random.default_rng(45)
    rows = [int(x) for x in rng.integers(0, M + 1, E)]
    rows[0], rows[1] = 0, M
    A, B = make_operands(45, E, M, N, K, BF16, ("normal", 1.0 / 16), "row", "col")
    say(f"[gpu] grouped moe rows={rows}")
    C = run_grouped(A, B, M, N, K, BF16, "f16", rows, b_layout="col", kernel="tile_256x256x64_mi16")
    for g, m in enumerate(rows):
        assert np.all(np.isnan(C[g, m:]))
        if m == 0:
            continue
        i = np.concatenate([rng.integers(0, m, 300), [0, m - 1]])
        j = np.concatenate([rng.integers(0, N, 300), [N - 1, 0]])
        z = np.full(i.size, g)
        Cp, Sp = orc.gemm_points(A, B, M, N, K, BF16, z, i, j, strideA=A[0].size, strideB=B[0].size,
                                 b_layout="col")
        check(C[g, i, j], Cp, Sp, K, "f16", f"moe group {g}")


def test_grouped_integer_bit_exact(orc):
    """Integer entries: every float32 partial sum is exact, so each group matches the oracle bit for bit."""
    M, N, K = 300, 256, 128
    rows = [300, 1, 299, 0]
    A, B = integer_operands(46, len(rows), M, N, K, F16, -2, 2, "row", "col")
    say("[gpu] grouped integer")
    C = run_grouped(A, B, M, N, K, F16, "f32", rows, b_layout="col")
    for g, (Cr, _) in enumerate(orc.gemm_grouped(A, B, M, N, K, F16, rows, b_layout="col")):
        assert np.array_equal(C[g, :Cr.shape[0]], Cr)


@pytest.mark.parametrize("variant,b_layout", [("tile_256x256x64_mi16", "col"), ("tile_256x256x32_mi16_nn", "row")])
def test_plain_ragged_m_on_tile_kernel(orc, monkeypatch, variant, b_layout):
    """A plain product with M = 1000 (not a multiple of 256) on the large-tile kernels."""
    from gpu_util import run

    monkeypatch.setenv("TSM_GEMM_KERNEL", variant)
    M, N, K = 1000, 512, 384
    A, B = make_operands(47, 1, M, N, K, BF16, ("uniform", -1.0, 1.0), "row", b_layout)
    say(f"[gpu] ragged M {variant}")
    C = run(A, B, M, N, K, BF16, "f32", b_layout=b_layout, ldc=N + 4, fill=float("nan"), kernel=variant)
    Cr, S = orc.gemm_rows(A, B, M, N, K, BF16, b_layout=b_layout)
    check(C, Cr, S, K, "f32", f"ragged M {variant}")


def test_moe_workload_full_size(orc):
    """The grouped workload the benchmark times (8 groups of up to 4096 rows, 2048 x 4096 weights stored
    K-contiguous, bf16 -> f16, the seeded routing counts), every valid element against the oracle, every row past
    the counts untouched."""
    from workloads import GROUPED

    w = GROUPED["moe_bf16_e8_t16384_n2048_k4096"]
    rows = [int(x) for x in w.rows()]
    A, B = w.operands()
    say(f"[gpu] {w.name} rows={rows}")
    C = run_grouped(A, B, w.M, w.N, w.K, w.in_fmt, w.out_fmt, rows, a_layout=w.a_layout, b_layout=w.b_layout,
                    kernel="tile_256x256x64_mi16_st")
    check_grouped(orc, C, A, B, w.M, w.N, w.K, w.in_fmt, w.out_fmt, rows, a_layout=w.a_layout, b_layout=w.b_layout,
                  what=w.name)
