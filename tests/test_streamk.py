"""Stream-K through a caller's workspace (gemm_strided_batched_ws) against the oracle (needs an MI355X).

Products of 32 to 224 tiles of 256 x 256 leave CUs idle in a one-tile-per-workgroup launch.  Stream-K deals the
tiles' 128-deep K slices to one run per CU in equal contiguous runs; each run stores a float32 partial tile for every
tile it meets and a second kernel adds each tile's partials in K order.  It runs on request (TSM_GEMM_SPLIT=streamk,
set for every test here).  The acceptance bound is the same K * 2^-24 * sum|a*b| as for every kernel (one more
summation order), the result must not depend on what the workspace held, and it must be the same bits on every call.
"""

import numpy as np
import pytest

import tiled_shared_memory_amd as tsm
from gpu_util import check, say
from test_ksplit import run_ws
from workloads.inputs import BF16, F16, integer_operands, make_operands

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _request_streamk(monkeypatch):
    monkeypatch.setenv("TSM_GEMM_SPLIT", "streamk")

SK = "streamk_tile_256x256x32_mi16"
SUFFIX = {("row", "col"): "+reduce", ("row", "row"): "_nn+reduce", ("col", "row"): "_tn+reduce",
          ("col", "col"): "_tt+reduce"}

# (M, N, K, batch, A layout, B layout): ragged M and N, every layout pair, 32 tiles (the smallest stream-K
# takes), 224 (the largest), runs of 2 to 36 slices, tiles cut into 2 to 8 segments, a strided batch.
SHAPES = [(1600, 1304, 2048, 1, "row", "col"), (2000, 2056, 4096, 1, "row", "row"),
          (1544, 1800, 2560, 1, "col", "row"), (1800, 1544, 2176, 1, "col", "col"),
          (2048, 1024, 2048, 1, "row", "col"), (3584, 4096, 2048, 1, "row", "col"),
          (600, 520, 2048, 8, "row", "col"), (520, 600, 3072, 6, "row", "row")]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("in_fmt,out_fmt", [(BF16, "f16"), (F16, "f32"), (BF16, "bf16")])
def test_streamk_parity(orc, shape, in_fmt, out_fmt):
    """Every element against the oracle; the workspace starts as NaN and none of it leaks."""
    M, N, K, batch, la, lb = shape
    A, B = make_operands(M + 7 * N + K + batch, batch, M, N, K, in_fmt, ("uniform", -1.0, 1.0), la, lb)
    say(f"[gpu] stream-K {shape} {in_fmt}->{out_fmt}")
    C = run_ws(A, B, M, N, K, in_fmt, out_fmt, batch=batch, fill=float("nan"), expect=SK + SUFFIX[(la, lb)],
               a_layout=la, b_layout=lb)
    Cr, S = orc.gemm_rows(A, B, M, N, K, in_fmt, batch=batch, a_layout=la, b_layout=lb)
    ratio = check(C, Cr, S, K, out_fmt, f"stream-K {shape}")
    say(f"[gpu] stream-K {shape}: max err/bound = {ratio:.3e}")


def test_streamk_3072_square_full_size(orc):
    """3072 x 3072 x 8192 bf16 -> f16 (144 tiles, runs of 36 slices of 64 per tile), every element."""
    M = N = 3072
    K = 8192
    A, B = make_operands(3072, 1, M, N, K, BF16, ("normal", 1.0 / 64.0), "row", "col")
    say("[gpu] stream-K 3072x3072x8192 full size")
    C = run_ws(A, B, M, N, K, BF16, "f16", fill=float("nan"), expect=SK + "+reduce", b_layout="col")
    Cr, S = orc.gemm_rows(A, B, M, N, K, BF16, b_layout="col")
    ratio = check(C, Cr, S, K, "f16", "stream-K 3072^2 x 8192")
    say(f"[gpu] stream-K 3072^2 x 8192: max err/bound = {ratio:.3e}")


def test_streamk_bitwise_run_to_run():
    """The same bits on every call, whatever the workspace held before (NaN, then 7.0, then the previous call's
    partials)."""
    M, N, K = 2304, 1792, 4096
    A, B = make_operands(77, 1, M, N, K, BF16, ("uniform", -1.0, 1.0), "row", "col")
    say("[gpu] stream-K run to run")
    outs = [run_ws(A, B, M, N, K, BF16, "f32", ws_fill=f, expect=SK, b_layout="col") for f in
            (float("nan"), 7.0, 0.0)]
    for C in outs[1:]:
        assert np.array_equal(outs[0], C)


def test_streamk_integer_inputs_bit_exact(orc):
    """Integer entries: every partial and every sum of partials is an exact float32 integer, so the result
    equals the oracle exactly."""
    M, N, K = 1800, 1304, 2048
    A, B = integer_operands(503, 1, M, N, K, F16, -2, 2, "row", "row")
    say("[gpu] stream-K integers")
    C = run_ws(A, B, M, N, K, F16, "f32", expect=SK + "_nn")
    Cr, _ = orc.gemm_rows(A, B, M, N, K, F16)
    assert np.array_equal(C, Cr)


@pytest.mark.parametrize("act,slope", [(tsm.TSM_ACT_RELU, 0.0), (tsm.TSM_ACT_LEAKY_RELU, 0.2)], ids=["relu", "leaky"])
def test_streamk_activation_padded_and_sentinel(orc, act, slope):
    """Padded lda/ldb/ldc: the activation is applied once, after the last partial, and C's padding keeps its
    bits."""
    M, N, K = 1300, 1320, 2048
    lda, ldb, ldc = K + 8, K + 64, N + 4
    A, B = make_operands(504, 1, M, N, K, F16, ("uniform", -1.0, 1.0), "row", "col")
    Ap = np.zeros((1, M, lda), np.uint16)
    Ap[:, :, :K] = A
    Bp = np.zeros((1, N, ldb), np.uint16)
    Bp[:, :, :K] = B
    say(f"[gpu] stream-K act={act} padded")
    C, raw, _ = run_ws(Ap, Bp, M, N, K, F16, "f32", lda=lda, ldb=ldb, ldc=ldc, act=act, slope=slope, fill=100.0,
                       keep=True, expect=SK, b_layout="col")
    Cr, S = orc.gemm_rows(A, B, M, N, K, F16, b_layout="col")
    check(C, Cr, S, K, "f32", "stream-K padded", act=act, slope=slope)
    host = raw.cpu().numpy().reshape(-1)
    for i in range(M):
        assert np.all(host[i * ldc + N:(i + 1) * ldc] == 100.0)


def test_streamk_off_gives_the_tile_split_or_no_split(orc, monkeypatch):
    """Without the request the same shape takes the tile split, and with TSM_GEMM_SPLIT=none the kernel that
    needs no workspace; all three pass."""
    M, N, K = 2048, 1024, 8192
    A, B = make_operands(505, 1, M, N, K, BF16, ("uniform", -1.0, 1.0), "row", "col")
    Cr, S = orc.gemm_rows(A, B, M, N, K, BF16, b_layout="col")
    for mode, expect in ((None, "ksplit_tile_"), ("none", "masked_")):
        if mode is None:
            monkeypatch.delenv("TSM_GEMM_SPLIT")
        else:
            monkeypatch.setenv("TSM_GEMM_SPLIT", mode)
        say(f"[gpu] TSM_GEMM_SPLIT={mode}")
        C = run_ws(A, B, M, N, K, BF16, "f16", expect=expect, b_layout="col")
        check(C, Cr, S, K, "f16", f"TSM_GEMM_SPLIT={mode}")
