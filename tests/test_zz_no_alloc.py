"""The allocation-free entry point (static scratch) against the workspace entry point, through the C ABI.

Both run the same K split with the same kernels, so the outputs must agree bit for bit; every call after the first
is a smaller problem, so it reuses the scratch the one before left behind.  Each result is also checked
against the oracle within the stated bound.
"""

import numpy as np
import pytest

import oracle  # noqa: F401  (the orc fixture)
import tiled_shared_memory_amd as tsm
from gpu_util import DTYPE, LAYOUT, alloc_c, c_view, check, say, to_device
from workloads.inputs import BF16, F16, make_operands

pytestmark = pytest.mark.gpu

# (M, N, K, batch), operand format, output format, A layout, B layout; each smaller than the one before: the
# hybrid (272 tiles, its 16 leftover tiles in 8 chunks: 32 MiB of the scratch; asked for, since at this depth the
# plain call's row bands are the default), the streaming kernel's split, the same split on a batch
CASES = [((4352, 4096, 2048, 1), BF16, "f16", "row", "col"), ((256, 256, 8192, 1), F16, "f32", "row", "row"),
         ((64, 512, 2048, 2), BF16, "f16", "row", "col")]


def test_noalloc_matches_workspace_entry_twice(orc, monkeypatch):
    import torch

    monkeypatch.setenv("TSM_GEMM_SPLIT", "hybrid")

    for (M, N, K, batch), fin, fout, la, lb in CASES:
        A, B = make_operands(M + N + K + batch, batch, M, N, K, fin, ("uniform", -1.0, 1.0), la, lb)
        lda = K if la == "row" else M
        ldb = N if lb == "row" else K
        ldc = N
        sA, sB, sC = A[0].size, B[0].size, M * N
        need = tsm.gemm_workspace_bytes(M, N, K, batch)
        assert 0 < need <= tsm.gemm_noalloc_scratch_bytes()
        a_buf, a_ptr = to_device(A)
        b_buf, b_ptr = to_device(B)
        c_ws = alloc_c(batch, M, N, ldc, sC, fout, fill=float("nan"))
        c_na = alloc_c(batch, M, N, ldc, sC, fout, fill=float("nan"))
        ws = torch.empty((need + 3) // 4, dtype=torch.float32, device="cuda")
        args = (M, N, K, a_ptr, lda, LAYOUT[la], sA, b_ptr, ldb, LAYOUT[lb], sB)
        code = DTYPE[(fin, fout)]
        name = tsm.tsm_gemm_ws_kernel_name(*args, c_ws, ldc, sC, batch, code, ws, need)
        assert name.endswith("+reduce"), name  # the K split runs
        say(f"[gpu] noalloc vs workspace {M}x{N}x{K} batch {batch} {fin}->{fout}: {name}")
        tsm.gemm_strided_batched_ws(*args, c_ws, ldc, sC, batch, code, tsm.TSM_ACT_NONE, 0.0, ws, need, 0)
        tsm.gemm_strided_batched_noalloc(*args, c_na, ldc, sC, batch, code, tsm.TSM_ACT_NONE, 0.0, 0)
        torch.cuda.synchronize()
        got_ws = c_view(c_ws, batch, M, N, ldc, sC, fout)
        got_na = c_view(c_na, batch, M, N, ldc, sC, fout)
        assert np.array_equal(got_na, got_ws), "static-scratch result differs from the workspace result"
        Cr, S = orc.gemm_rows(A, B, M, N, K, fin, batch=batch, a_layout=la, b_layout=lb)
        check(got_na, Cr, S, K, fout, f"noalloc {M}x{N}x{K}")
