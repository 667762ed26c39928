"""K split through a caller's workspace (gemm_strided_batched_ws) against the oracle (needs an MI355X).

Pass 1 stores float32 partial sums of each K chunk into the workspace, pass 2 adds them in chunk order and applies
the epilogue.  The acceptance bound is the same K * 2^-24 * sum|a*b| as for every kernel: the chunked order is one
more summation order.
"""

import numpy as np
import pytest

import tiled_shared_memory_amd as tsm
from gpu_util import DTYPE, alloc_c, c_view, check, say, to_device
from workloads.inputs import BF16, F16, make_operands

pytestmark = pytest.mark.gpu


def run_ws(A, B, M, N, K, in_fmt, out_fmt, *, batch=1, lda=None, ldb=None, ldc=None, sA=None, sB=None, sC=None,
           act=tsm.TSM_ACT_NONE, slope=0.0, ws_bytes=None, ws_fill=float("nan"), fill=None, keep=False,
           expect=None, a_layout="row", b_layout="row"):
    """C = act(A.B) through gemm_strided_batched_ws with a workspace of ws_bytes (default: what the shape needs)."""
    import torch

    la = 1 if a_layout == "col" else 0
    lb = 1 if b_layout == "col" else 0
    lda = lda if lda is not None else (M if la else K)
    ldb = ldb if ldb is not None else (K if lb else N)
    ldc = ldc if ldc is not None else N
    sA = sA if sA is not None else A.size // batch
    sB = sB if sB is not None else B.size // batch
    sC = sC if sC is not None else M * ldc
    need = tsm.gemm_workspace_bytes(M, N, K, batch)
    ws_bytes = need if ws_bytes is None else ws_bytes
    ws = torch.full((max(ws_bytes, 16) // 4 + 4,), ws_fill, dtype=torch.float32, device="cuda")
    a_buf, a_ptr = to_device(A)
    b_buf, b_ptr = to_device(B)
    c = alloc_c(batch, M, N, ldc, sC, out_fmt, fill)
    code = DTYPE[(in_fmt, out_fmt)]
    name = tsm.tsm_gemm_ws_kernel_name(M, N, K, a_ptr, lda, la, sA, b_ptr, ldb, lb, sB, c, ldc, sC, batch, code, ws,
                                       ws_bytes)
    if expect is not None:
        assert name is not None and name.startswith(expect), f"routed to {name}, expected {expect}"
    tsm.gemm_strided_batched_ws(M, N, K, a_ptr, lda, la, sA, b_ptr, ldb, lb, sB, c, ldc, sC, batch, code, act, slope,
                                ws, ws_bytes, 0)
    torch.cuda.synchronize()
    res = c_view(c, batch, M, N, ldc, sC, out_fmt)
    return (res, c, name) if keep else res


SPLIT = "ksplit_"
SHAPES = [(256, 256, 8192, 1), (16, 4096, 4096, 1), (100, 192, 1344, 1), (48, 128, 2048, 3), (1, 64, 512, 2),
          (200, 320, 2112, 1),
          # 256-column panels
          (16, 8192, 1024, 1), (40, 8192, 2048, 1), (8, 4096, 1088, 2)]


@pytest.mark.parametrize("shape", [(384, 384, 2048, 1), (16, 4096, 1024, 1), (100, 192, 1344, 2)],
                         ids=lambda s: "x".join(map(str, s)))
def test_ksplit_col_b(orc, shape):
    """The skinny kernel's split with a K-contiguous B."""
    M, N, K, batch = shape
    A, B = make_operands(M + 5 * N + K, batch, M, N, K, BF16, ("uniform", -1.0, 1.0), "row", "col")
    say(f"[gpu] ksplit col-B {shape}")
    C = run_ws(A, B, M, N, K, BF16, "f32", batch=batch, expect="ksplit_skinny_", b_layout="col")
    Cr, S = orc.gemm_rows(A, B, M, N, K, BF16, batch=batch, b_layout="col")
    check(C, Cr, S, K, "f32", f"ksplit col-B {shape}")


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("in_fmt,out_fmt", [(F16, "f32"), (BF16, "f16"), (BF16, "bf16")])
def test_ksplit_parity(orc, shape, in_fmt, out_fmt):
    """Chunks of 256 or more (the last one ragged where K allows), row blocks ragged in M, batches, 64- and
    256-column panels; the workspace starts as NaN and none of it leaks."""
    M, N, K, batch = shape
    assert tsm.gemm_workspace_bytes(M, N, K, batch) > 0
    A, B = make_operands(M + 3 * N + K + batch, batch, M, N, K, in_fmt, ("uniform", -1.0, 1.0))
    say(f"[gpu] ksplit {shape} {in_fmt}->{out_fmt}")
    C = run_ws(A, B, M, N, K, in_fmt, out_fmt, batch=batch, expect=SPLIT)
    Cr, S = orc.gemm_rows(A, B, M, N, K, in_fmt, batch=batch)
    ratio = check(C, Cr, S, K, out_fmt, f"ksplit {shape}")
    say(f"[gpu] ksplit {shape}: max err/bound = {ratio:.3e}")


def test_largek_workload_through_the_workspace(orc):
    """The 256 x 256 x 8192 workload with its own seeded operands, through the workspace route that the
    benchmark times (pass 1 of the skinny kernel's split, then the reduction), against the oracle everywhere."""
    from workloads import WORKLOADS

    w = WORKLOADS["largek_f16_256x256x8192"]
    A, B = w.operands()
    say(f"[gpu] {w.name} through the workspace")
    C = run_ws(A, B, w.M, w.N, w.K, w.in_fmt, w.out_fmt, batch=w.batch, fill=float("nan"),
               expect="ksplit_skinny_m32_n64_k64+reduce")
    Cr, S = orc.gemm_rows(A, B, w.M, w.N, w.K, w.in_fmt, batch=w.batch)
    ratio = check(C, Cr, S, w.K, w.out_fmt, w.name)
    say(f"[gpu] {w.name} workspace: max err/bound = {ratio:.3e}")


TILE_SPLIT = [(640, 768, 8192, "row", "col"), (600, 520, 8192, "row", "row"), (1000, 512, 8192, "row", "row"),
              (600, 2304, 8192, "row", "col"), (520, 1024, 8192, "col", "row"), (1792, 1280, 8192, "col", "col")]


@pytest.mark.parametrize("shape", TILE_SPLIT, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("in_fmt,out_fmt", [(BF16, "f16"), (F16, "f32")])
def test_tile_split_parity(orc, shape, in_fmt, out_fmt):
    """The 256 x 256 kernels' split (products of 8-128 such tiles, more than 128 rows, K >= 8192, or K >= 4096
    from 64 tiles): the K chunks run as a strided batch into the workspace, ragged M and N, both B layouts."""
    M, N, K, a_layout, b_layout = shape
    A, B = make_operands(M + N + K, 1, M, N, K, in_fmt, ("uniform", -1.0, 1.0), a_layout, b_layout)
    say(f"[gpu] tile split {shape} {in_fmt}->{out_fmt}")
    C = run_ws(A, B, M, N, K, in_fmt, out_fmt, expect="ksplit_tile_", a_layout=a_layout, b_layout=b_layout)
    Cr, S = orc.gemm_rows(A, B, M, N, K, in_fmt, a_layout=a_layout, b_layout=b_layout)
    ratio = check(C, Cr, S, K, out_fmt, f"tile split {shape}")
    say(f"[gpu] tile split {shape}: max err/bound = {ratio:.3e}")


@pytest.mark.parametrize("act,slope", [(tsm.TSM_ACT_RELU, 0.0), (tsm.TSM_ACT_LEAKY_RELU, 0.2)], ids=["relu", "leaky"])
def test_ksplit_activation_padded_and_sentinel(orc, act, slope):
    """Padded lda/ldb/ldc and batch strides, C prefilled: the activation is applied once, after the last chunk,
    and C's padding keeps its bits."""
    M, N, K, batch = 40, 192, 1536, 2
    lda, ldb, ldc = K + 8, N + 64, N + 4
    A, B = make_operands(501, batch, M, N, K, F16, ("uniform", -1.0, 1.0))
    Ap = np.zeros((batch, M, lda), np.uint16)
    Ap[:, :, :K] = A
    Bp = np.zeros((batch, K, ldb), np.uint16)
    Bp[:, :, :N] = B
    sC = M * ldc + 8
    say(f"[gpu] ksplit act={act} padded")
    C, raw, _ = run_ws(Ap, Bp, M, N, K, F16, "f32", batch=batch, lda=lda, ldb=ldb, ldc=ldc, sC=sC, act=act,
                       slope=slope, fill=100.0, keep=True, expect=SPLIT)
    Cr, S = orc.gemm_rows(A, B, M, N, K, F16, batch=batch)
    check(C, Cr, S, K, "f32", "ksplit padded", act=act, slope=slope)
    host = raw.cpu().numpy()
    for z in range(batch):
        for i in range(M):
            o = z * sC + i * ldc
            assert np.all(host[o + N:o + ldc] == 100.0)


def test_ksplit_deterministic_and_small_workspace(orc):
    """Bitwise the same twice; with one byte too few of workspace the call runs the kernel that needs none, and the
    result still passes."""
    M, N, K = 256, 256, 8192
    A, B = make_operands(502, 1, M, N, K, F16, ("uniform", -1.0, 1.0))
    say("[gpu] ksplit determinism")
    C1 = run_ws(A, B, M, N, K, F16, "f32", expect=SPLIT)
    C2 = run_ws(A, B, M, N, K, F16, "f32", ws_fill=7.0, expect=SPLIT)
    assert np.array_equal(C1, C2)
    need = tsm.gemm_workspace_bytes(M, N, K, 1)
    C3 = run_ws(A, B, M, N, K, F16, "f32", ws_bytes=need - 1, expect="splitk_")
    Cr, S = orc.gemm_rows(A, B, M, N, K, F16)
    check(C3, Cr, S, K, "f32", "no split")


def test_ksplit_integer_inputs_bit_exact(orc):
    """Integer entries: every partial and every chunk sum is an exact float32 integer, so the result equals the
    oracle exactly."""
    from workloads.inputs import integer_operands

    M, N, K = 64, 128, 4096
    A, B = integer_operands(503, 1, M, N, K, F16, -2, 2, "row", "row")
    say("[gpu] ksplit integers")
    C = run_ws(A, B, M, N, K, F16, "f32", expect=SPLIT)
    Cr, _ = orc.gemm_rows(A, B, M, N, K, F16)
    assert np.array_equal(C, Cr)
