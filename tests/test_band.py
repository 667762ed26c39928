"""Row bands on the plain entry points against the oracle (needs an MI355X).

One problem a little over whole rounds of 256 x 256 tiles (one tile per CU) and no workspace: the rows that fill the
whole rounds run on the large-tile kernel, the rows past them as a problem of their own on the kernel the planner
picks for it (the streaming kernel, 64 x 64 masked tiles, or one round of 128 x 128 masked tiles).  The acceptance
bound is the same K * 2^-24 * sum|a*b| as for every kernel; C starts as NaN, so a row that neither band wrote fails.
Each band must also be the same bits as its kernel gives when it alone computes those rows.
"""

import numpy as np
import pytest

import tiled_shared_memory_amd as tsm
from gpu_util import DTYPE, check, run, say, workload_reference
from test_ksplit import run_ws
from workloads.inputs import BF16, F16, integer_operands, make_operands

pytestmark = pytest.mark.gpu

# (M, N, K, A layout, B layout, output, what the rows past the whole rounds run on)
SHAPES = [
    (4352, 4096, 1024, "row", "col", (BF16, "f16"), "masked_64x64x64"),     # 256 rows left, 16 tiles
    (4160, 4096, 1024, "row", "col", (F16, "f32"), "skinny_m64"),           # 64 rows left
    (4224, 4096, 1024, "row", "row", (BF16, "bf16"), "skinny_m128"),        # 128 rows, row-major B
    (5120, 4096, 1024, "col", "row", (F16, "f16"), "masked_128x128x32"),    # one round of 128 x 128 tiles
    (4600, 4104, 1024, "row", "col", (BF16, "f32"), "masked_128x128x32"),   # ragged; 15 rows of 17 tiles fill the round, 198 tiles of 128 x 128 left
    (4608, 4096, 1024, "col", "col", (BF16, "f16"), "masked_64x64x64"),
    (8448, 4096, 1024, "row", "col", (F16, "bf16"), "masked_64x64x64"),     # two whole rounds
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s[:5])))
def test_band_parity(orc, shape):
    """Every element against the oracle."""
    M, N, K, la, lb, (in_fmt, out_fmt), low = shape
    A, B = make_operands(M + 5 * N + K, 1, M, N, K, in_fmt, ("uniform", -1.0, 1.0), la, lb)
    say(f"[gpu] bands {shape}")
    C = run(A, B, M, N, K, in_fmt, out_fmt, a_layout=la, b_layout=lb, fill=float("nan"), kernel="band_")
    name = tsm.tsm_gemm_kernel_name(M, N, K, 1 << 40, M if la == "col" else K, int(la == "col"), 0, 2 << 40,
                                    K if lb == "col" else N, int(lb == "col"), 0, 3 << 40, N, 0, 1,
                                    DTYPE[(in_fmt, out_fmt)])
    assert name.split("+")[1].startswith(low), name
    Cr, S = orc.gemm_rows(A, B, M, N, K, in_fmt, a_layout=la, b_layout=lb)
    ratio = check(C, Cr, S, K, out_fmt, f"bands {shape}")
    say(f"[gpu] bands {shape}: max err/bound = {ratio:.3e}")


@pytest.mark.parametrize("M,la,low", [(4352, "row", "masked_64x64x64_vec8"), (4160, "row", "skinny_m64_n64_k64_t"),
                                      (4352, "col", "masked_64x64x64_vec8")])
def test_band_bits_are_each_kernels(monkeypatch, M, la, low):
    """Rows of the whole rounds: the bits of the large-tile kernel over the whole problem; rows past them: the bits
    of the plain call on those rows alone; a workspace too small to split: the same bits as no workspace."""
    N, K = 4096, 1024
    top = 4096
    A, B = make_operands(M + 11, 1, M, N, K, BF16, ("uniform", -1.0, 1.0), la, "col")
    big = {"row": "tile_256x256x64_mi16_st", "col": "tile_256x256x32_mi16_tt"}[la]
    say(f"[gpu] bands bits M={M} A {la}")
    C = run(A, B, M, N, K, BF16, "f16", a_layout=la, b_layout="col", fill=float("nan"), kernel=f"band_{big}+{low}")
    monkeypatch.setenv("TSM_GEMM_KERNEL", big)
    whole = run(A, B, M, N, K, BF16, "f16", a_layout=la, b_layout="col", kernel=big)
    monkeypatch.delenv("TSM_GEMM_KERNEL")
    assert np.array_equal(C[:, :top], whole[:, :top])
    A_low = np.ascontiguousarray(A[:, top:, :] if la == "row" else A[:, :, top:])
    C_low = run(A_low, B, M - top, N, K, BF16, "f16", a_layout=la, b_layout="col", kernel=low)
    assert np.array_equal(C[:, top:], C_low)
    C_ws = run_ws(A, B, M, N, K, BF16, "f16", ws_bytes=0, expect="band_", a_layout=la, b_layout="col")
    assert np.array_equal(C, C_ws)


def test_band_integers_exact(orc):
    """Integer entries: both bands give the exact sums."""
    M, N, K = 4608, 4096, 1024
    A, B = integer_operands(701, 1, M, N, K, BF16, -2, 2, "row", "col")
    say("[gpu] bands integers")
    C = run(A, B, M, N, K, BF16, "f32", b_layout="col", kernel="band_")
    Cr, _ = orc.gemm_rows(A, B, M, N, K, BF16, b_layout="col")
    assert np.array_equal(C, Cr)


@pytest.mark.parametrize("act,slope", [(tsm.TSM_ACT_RELU, 0.0), (tsm.TSM_ACT_LEAKY_RELU, 0.25)], ids=["relu", "leaky"])
def test_band_activation_padded_and_sentinel(orc, act, slope):
    """Padded strides; the activation applied on both bands; C's padding keeps its bits."""
    M, N, K = 4352, 4096, 1024
    lda, ldb, ldc = K + 16, K + 8, N + 8
    A, B = make_operands(702, 1, M, N, K, F16, ("uniform", -1.0, 1.0), "row", "col")
    Ap = np.zeros((1, M, lda), np.uint16)
    Ap[:, :, :K] = A
    Bp = np.zeros((1, N, ldb), np.uint16)
    Bp[:, :, :K] = B
    say(f"[gpu] bands act={act} padded")
    C, raw = run(Ap, Bp, M, N, K, F16, "f16", b_layout="col", lda=lda, ldb=ldb, ldc=ldc, act=act, slope=slope,
                 fill=100.0, keep=True, kernel="band_")
    Cr, S = orc.gemm_rows(A, B, M, N, K, F16, b_layout="col")
    check(C, Cr, S, K, "f16", "bands padded", act=act, slope=slope)
    host = raw.float().cpu().numpy().reshape(-1)
    for i in range(0, M, 61):
        assert np.all(host[i * ldc + N:(i + 1) * ldc] == 100.0)


def test_partial_round_workload_plain_call_full_size(orc):
    """The 4352 x 4096 x 8192 workload through the plain entry point (no workspace), every element."""
    from workloads import PARTIAL

    w = PARTIAL["partial_bf16_4352x4096x8192"]
    A, B, Cr, S = workload_reference(orc, w)
    say(f"[gpu] {w.name} in row bands")
    C = run(A, B, w.M, w.N, w.K, w.in_fmt, w.out_fmt, a_layout=w.a_layout, b_layout=w.b_layout, fill=float("nan"),
            kernel="band_tile_256x256x64_mi16_st+masked_64x64x64_vec8")
    ratio = check(C, Cr, S, w.K, w.out_fmt, w.name)
    say(f"[gpu] {w.name} in row bands: max err/bound = {ratio:.3e}")
