"""The hybrid through a caller's workspace (gemm_strided_batched_ws) against the oracle (needs an MI355X).

One problem a little over whole rounds of 256 x 256 tiles (one per CU): the whole rounds run on the data-parallel
kernel, and the last round's tiles are cut into equal chunks of K, one stream-K run each, whose float32 partials a
second kernel adds in K order.  The acceptance bound is the same K * 2^-24 * sum|a*b| as for every kernel; C starts as
NaN, so a tile that neither part wrote fails.
"""

import numpy as np
import pytest

import tiled_shared_memory_amd as tsm
from gpu_util import check, say, workload_reference
from test_ksplit import run_ws
from workloads.inputs import BF16, F16, integer_operands, make_operands

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _request_hybrid(monkeypatch):
    # up to K = 4096 the same calls take row bands unless the hybrid is asked for
    monkeypatch.setenv("TSM_GEMM_SPLIT", "hybrid")

DP = {("row", "col"): "tile_256x256x64_mi16_st", ("row", "row"): "tile_256x256x32_mi16_nn",
      ("col", "row"): "tile_256x256x32_mi16_tn", ("col", "col"): "tile_256x256x32_mi16_tt"}

# (M, N, K, A layout, B layout): 272, 288, 320 and 384 tiles (a last round of 16, 32, 64 and 128 tiles, cut into
# 8, 8, 4 and 2 chunks), ragged M and N (289 tiles: 33 left over, 4 chunks since K / 128 = 16 is not a multiple
# of 7), every layout pair
SHAPES = [(4352, 4096, 2048, "row", "col"), (4600, 4104, 2048, "row", "col"), (4608, 4096, 2048, "row", "row"),
          (5120, 4096, 2048, "col", "row"), (6144, 4096, 2048, "col", "col"), (4352, 4104, 2048, "row", "col")]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("in_fmt,out_fmt", [(BF16, "f16"), (F16, "f32")])
def test_hybrid_parity(orc, shape, in_fmt, out_fmt):
    """Every element against the oracle; the workspace starts as NaN and none of it leaks."""
    M, N, K, la, lb = shape
    A, B = make_operands(M + 3 * N + K, 1, M, N, K, in_fmt, ("uniform", -1.0, 1.0), la, lb)
    say(f"[gpu] hybrid {shape} {in_fmt}->{out_fmt}")
    C = run_ws(A, B, M, N, K, in_fmt, out_fmt, fill=float("nan"), expect="hybrid_" + DP[(la, lb)] + "+reduce",
               a_layout=la, b_layout=lb)
    Cr, S = orc.gemm_rows(A, B, M, N, K, in_fmt, a_layout=la, b_layout=lb)
    ratio = check(C, Cr, S, K, out_fmt, f"hybrid {shape}")
    say(f"[gpu] hybrid {shape}: max err/bound = {ratio:.3e}")


def test_hybrid_bitwise_run_to_run_and_integers(orc):
    """The same bits on every call whatever the workspace held; integer entries exact."""
    M, N, K = 4608, 4096, 2048
    A, B = integer_operands(601, 1, M, N, K, BF16, -2, 2, "row", "col")
    say("[gpu] hybrid run to run, integers")
    outs = [run_ws(A, B, M, N, K, BF16, "f32", ws_fill=f, expect="hybrid_", b_layout="col") for f in
            (float("nan"), 3.0)]
    assert np.array_equal(outs[0], outs[1])
    Cr, _ = orc.gemm_rows(A, B, M, N, K, BF16, b_layout="col")
    assert np.array_equal(outs[0], Cr)


@pytest.mark.parametrize("act,slope", [(tsm.TSM_ACT_RELU, 0.0), (tsm.TSM_ACT_LEAKY_RELU, 0.25)], ids=["relu", "leaky"])
def test_hybrid_activation_padded_and_sentinel(orc, act, slope):
    """Padded strides; the activation applied once on both parts; C's padding keeps its bits."""
    M, N, K = 4352, 4096, 2048
    lda, ldb, ldc = K + 16, K + 8, N + 8
    A, B = make_operands(602, 1, M, N, K, F16, ("uniform", -1.0, 1.0), "row", "col")
    Ap = np.zeros((1, M, lda), np.uint16)
    Ap[:, :, :K] = A
    Bp = np.zeros((1, N, ldb), np.uint16)
    Bp[:, :, :K] = B
    say(f"[gpu] hybrid act={act} padded")
    C, raw, _ = run_ws(Ap, Bp, M, N, K, F16, "f16", lda=lda, ldb=ldb, ldc=ldc, act=act, slope=slope, fill=100.0,
                       keep=True, expect="hybrid_", b_layout="col")
    Cr, S = orc.gemm_rows(A, B, M, N, K, F16, b_layout="col")
    check(C, Cr, S, K, "f16", "hybrid padded", act=act, slope=slope)
    host = raw.float().cpu().numpy().reshape(-1)
    for i in range(0, M, 97):
        assert np.all(host[i * ldc + N:(i + 1) * ldc] == 100.0)


def test_partial_round_workload_full_size(orc):
    """The 4352 x 4096 x 8192 workload (272 tiles) the benchmark times through the workspace, every element."""
    from workloads import PARTIAL

    w = PARTIAL["partial_bf16_4352x4096x8192"]
    A, B, Cr, S = workload_reference(orc, w)
    say(f"[gpu] {w.name} through the workspace")
    C = run_ws(A, B, w.M, w.N, w.K, w.in_fmt, w.out_fmt, fill=float("nan"),
               expect="hybrid_tile_256x256x64_mi16_st+reduce", a_layout=w.a_layout, b_layout=w.b_layout)
    ratio = check(C, Cr, S, w.K, w.out_fmt, w.name)
    say(f"[gpu] {w.name}: max err/bound = {ratio:.3e}")
