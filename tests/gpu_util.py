"""Helpers for the GPU tests: upload 16-bit operands, call the C ABI, compare with the oracle.

Inputs come from ``workloads`` (seeded, host-side); expected values come only
from the oracle.  Every GEMM here goes through the library's C entry points.
"""

from __future__ import annotations

import sys

import numpy as np

import oracle
import tiled_shared_memory_amd as tsm

DTYPE = {("f16", "f32"): tsm.TSM_F16_F32, ("f16", "f16"): tsm.TSM_F16_F16,
         ("bf16", "f32"): tsm.TSM_BF16_F32, ("bf16", "f16"): tsm.TSM_BF16_F16,
         ("f16", "bf16"): tsm.TSM_F16_BF16, ("bf16", "bf16"): tsm.TSM_BF16_BF16}
LAYOUT = {"row": tsm.TSM_ROW, "col": tsm.TSM_COL}


def say(msg: str):
    """Progress line on the real stdout (not captured), flushed before a GPU step."""
    sys.__stdout__.write(msg + "\n")
    sys.__stdout__.flush()


def to_device(bits: np.ndarray, offset_elems: int = 0):
    """Upload uint16 patterns; with an offset the data starts that many elements into the buffer."""
    import torch

    flat = np.ascontiguousarray(bits, dtype=np.uint16).reshape(-1)
    buf = torch.zeros(flat.size + offset_elems + 8, dtype=torch.int16, device="cuda")
    buf[offset_elems:offset_elems + flat.size].copy_(torch.from_numpy(flat.view(np.int16)))
    return buf, buf.data_ptr() + 2 * offset_elems


def alloc_c(batch, M, N, ldc, strideC, out_fmt, fill=None):
    import torch

    n = (batch - 1) * strideC + (M - 1) * ldc + N if batch and M and N else 1
    dt = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}[out_fmt]
    c = torch.empty(n + 4, dtype=dt, device="cuda")
    if fill is not None:
        c.fill_(fill)
    return c


def c_view(c_dev, batch, M, N, ldc, strideC, out_fmt) -> np.ndarray:
    """(batch, M, N) float64 copy of the logical C region."""
    host = c_dev.float().cpu().numpy().astype(np.float64)  # exact for every output format
    out = np.empty((batch, M, N))
    for z in range(batch):
        for i in range(M):
            o = z * strideC + i * ldc
            out[z, i] = host[o:o + N]
    return out


def run(A, B, M, N, K, in_fmt, out_fmt, *, batch=1, a_layout="row", b_layout="row", lda=None, ldb=None,
        ldc=None, sA=None, sB=None, sC=None, a_off=0, b_off=0, fill=None, stream=0, keep=False, kernel=None,
        act=None, slope=0.0):
    """C = A.B through gemm_strided_batched_ex (or, with ``act``, act(A.B) through gemm_strided_batched_act)
    on the given stored operands.

    Returns the float64 (batch, M, N) result (and the raw C buffer if ``keep``).
    If ``kernel`` is given, the call must be routed to the kernel of that name.
    """
    lda = lda if lda is not None else (K if a_layout == "row" else M)
    ldb = ldb if ldb is not None else (N if b_layout == "row" else K)
    ldc = ldc if ldc is not None else N
    sA = sA if sA is not None else (A.size // batch if batch else 0)
    sB = sB if sB is not None else (B.size // batch if batch else 0)
    sC = sC if sC is not None else M * ldc
    a_buf, a_ptr = to_device(A, a_off)
    b_buf, b_ptr = to_device(B, b_off)
    c = alloc_c(batch, M, N, ldc, sC, out_fmt, fill)
    if kernel is not None:
        name = tsm.tsm_gemm_kernel_name(M, N, K, a_ptr, lda, LAYOUT[a_layout], sA, b_ptr, ldb, LAYOUT[b_layout], sB,
                                        c, ldc, sC, batch, DTYPE[(in_fmt, out_fmt)])
        assert name is not None and name.startswith(kernel), f"routed to {name}, expected {kernel}"
    if act is None:
        tsm.gemm_strided_batched_ex(M, N, K, a_ptr, lda, LAYOUT[a_layout], sA, b_ptr, ldb, LAYOUT[b_layout], sB, c,
                                    ldc, sC, batch, DTYPE[(in_fmt, out_fmt)], stream)
    else:
        tsm.gemm_strided_batched_act(M, N, K, a_ptr, lda, LAYOUT[a_layout], sA, b_ptr, ldb, LAYOUT[b_layout], sB, c,
                                     ldc, sC, batch, DTYPE[(in_fmt, out_fmt)], act, slope, stream)
    import torch

    torch.cuda.synchronize()
    res = c_view(c, batch, M, N, ldc, sC, out_fmt)
    return (res, c) if keep else res


_WORKLOAD_REF = {}


def workload_reference(orc, w):
    """(A, B, C_ref, S) of a named workload, the oracle's result computed once per test session."""
    if w.name not in _WORKLOAD_REF:
        A, B = w.operands()
        Cr, S = orc.gemm_rows(A, B, w.M, w.N, w.K, w.in_fmt, batch=w.batch, a_layout=w.a_layout,
                              b_layout=w.b_layout)
        _WORKLOAD_REF[w.name] = (A, B, Cr, S)
    return _WORKLOAD_REF[w.name]


def check(C_gpu, C_ref, S, K, out_fmt, what="", act=0, slope=0.0):
    """Element-wise acceptance: |C_gpu - act(C_ref)| <= oracle.bound(...) (K*2^-24*S scaled for the
    activation, plus half an ulp of a 16-bit output); returns max err/bound."""
    assert np.all(np.isfinite(C_gpu)), f"{what}: non-finite output"
    C_ref = oracle.activate(C_ref, act, slope)
    err = np.abs(C_gpu - C_ref)
    bnd = oracle.bound(K, S, out_fmt, C_gpu, act, slope)
    ok = err <= bnd
    if not np.all(ok):
        idx = np.argwhere(~ok)[:5]
        raise AssertionError(f"{what}: {np.count_nonzero(~ok)} cells out of bound, first {idx.tolist()}: "
                             f"gpu={C_gpu[tuple(idx[0])]!r} ref={C_ref[tuple(idx[0])]!r} "
                             f"bound={bnd[tuple(idx[0])]!r}")
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(bnd > 0, err / bnd, 0.0)
    return float(r.max()) if r.size else 0.0
