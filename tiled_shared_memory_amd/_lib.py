"""ctypes binding of ``libtsm_gemm.so`` (the C ABI in ``include/tsm_gemm.h``).

Argument marshalling only: pointers, sizes and the stream handle go straight
to the C entry points of the same names, and a non-zero status becomes a
``TsmError``.  All arithmetic runs in the library's HIP kernels; there is no
fallback.  ``torch`` is imported first so the library binds to the HIP runtime
torch already loaded (both carry the soname ``libamdhip64.so.7``), which makes
torch's stream handles and device pointers valid inside the library.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(PKG, "libtsm_gemm.so")

TSM_SUCCESS = 0
TSM_ERROR_INVALID_VALUE = 1
TSM_ERROR_NOT_SUPPORTED = 2
TSM_ERROR_LAUNCH = 3

TSM_F16_F32 = 0
TSM_F16_F16 = 1
TSM_BF16_F32 = 2
TSM_BF16_F16 = 3
TSM_F16_BF16 = 4
TSM_BF16_BF16 = 5

TSM_ACT_NONE = 0
TSM_ACT_RELU = 1
TSM_ACT_LEAKY_RELU = 2

TSM_ROW = 0
TSM_COL = 1

TSM_ROWSUM_F32 = 0
TSM_ROWSUM_F16 = 1
TSM_ROWSUM_BF16 = 2

# Every function the header declares, with its ctypes signature.
_I64, _PTR, _INT = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
SIGNATURES = {
    "gemm": ([_I64, _I64, _I64, _PTR, _I64, _PTR, _I64, _PTR, _I64, _INT, _PTR], _INT),
    "gemm_ex": ([_I64, _I64, _I64, _PTR, _I64, _INT, _PTR, _I64, _INT, _PTR, _I64, _INT, _PTR], _INT),
    "gemm_strided_batched": ([_I64, _I64, _I64, _PTR, _I64, _I64, _PTR, _I64, _I64, _PTR, _I64, _I64, _I64, _INT,
                              _PTR], _INT),
    "gemm_strided_batched_ex": ([_I64, _I64, _I64, _PTR, _I64, _INT, _I64, _PTR, _I64, _INT, _I64, _PTR, _I64, _I64,
                                 _I64, _INT, _PTR], _INT),
    "tsm_status_string": ([_INT], ctypes.c_char_p),
    "tsm_last_error_detail": ([], ctypes.c_char_p),
    "tsm_gemm_kernel_name": ([_I64, _I64, _I64, _PTR, _I64, _INT, _I64, _PTR, _I64, _INT, _I64, _PTR, _I64, _I64,
                              _I64, _INT], ctypes.c_char_p),
    "gemm_grouped": ([_I64, _I64, _I64, _PTR, _I64, _INT, _I64, _PTR, _I64, _INT, _I64, _PTR, _I64, _I64, _PTR, _I64,
                      _INT, _PTR], _INT),
    "tsm_gemm_grouped_kernel_name": ([_I64, _I64, _I64, _PTR, _I64, _INT, _I64, _PTR, _I64, _INT, _I64, _PTR, _I64,
                                      _I64, _PTR, _I64, _INT], ctypes.c_char_p),
    "rowsum": ([_I64, _I64, _PTR, _I64, _I64, _INT, _PTR, _PTR], _INT),
    "gemm_strided_batched_act": ([_I64, _I64, _I64, _PTR, _I64, _INT, _I64, _PTR, _I64, _INT, _I64, _PTR, _I64, _I64,
                                  _I64, _INT, _INT, ctypes.c_float, _PTR], _INT),
    "tsm_rowsum_kernel_name": ([_I64, _I64, _PTR, _I64, _I64, _INT, _PTR], ctypes.c_char_p),
    "gemm_workspace_bytes": ([_I64, _I64, _I64, _I64], _I64),
    "gemm_strided_batched_ws": ([_I64, _I64, _I64, _PTR, _I64, _INT, _I64, _PTR, _I64, _INT, _I64, _PTR, _I64, _I64,
                                 _I64, _INT, _INT, ctypes.c_float, _PTR, _I64, _PTR], _INT),
    "gemm_strided_batched_noalloc": ([_I64, _I64, _I64, _PTR, _I64, _INT, _I64, _PTR, _I64, _INT, _I64, _PTR, _I64,
                                      _I64, _I64, _INT, _INT, ctypes.c_float, _PTR], _INT),
    "gemm_noalloc_scratch_bytes": ([], _I64),
    "tsm_gemm_ws_kernel_name": ([_I64, _I64, _I64, _PTR, _I64, _INT, _I64, _PTR, _I64, _INT, _I64, _PTR, _I64, _I64,
                                 _I64, _INT, _PTR, _I64], ctypes.c_char_p),
}


class TsmError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_status_text(status)} ({status}): {detail}")
        self.status = status
        self.detail = detail


_LIB = None


def load(path: str = LIBRARY):
    """Load the HIP library (after torch's HIP runtime); raise if it is not built."""
    global _LIB
    if _LIB is not None and path == LIBRARY:
        return _LIB
    import torch  # noqa: F401  -- binds the library to torch's HIP runtime

    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built: run `python -c 'import __graft_entry__ as g; g.build()'` "
                           "(there is no CPU fallback)")
    lib = ctypes.CDLL(path)
    for name, (args, res) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    if path == LIBRARY:
        _LIB = lib
    return lib


def _status_text(status: int) -> str:
    return {0: "success", 1: "invalid value", 2: "not supported", 3: "launch failure"}.get(status, "unknown status")


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(lib, status: int):
    if status != TSM_SUCCESS:
        detail = lib.tsm_last_error_detail()
        raise TsmError(status, detail.decode() if detail else "")
    return status


def gemm(M, N, K, A, lda, B, ldb, C, ldc, dtype, stream=None):
    lib = load()
    return _check(lib, lib.gemm(M, N, K, _ptr(A), lda, _ptr(B), ldb, _ptr(C), ldc, dtype, _stream(stream)))


def gemm_ex(M, N, K, A, lda, layout_a, B, ldb, layout_b, C, ldc, dtype, stream=None):
    lib = load()
    return _check(lib, lib.gemm_ex(M, N, K, _ptr(A), lda, layout_a, _ptr(B), ldb, layout_b, _ptr(C), ldc, dtype,
                                   _stream(stream)))


def gemm_strided_batched(M, N, K, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, dtype, stream=None):
    lib = load()
    return _check(lib, lib.gemm_strided_batched(M, N, K, _ptr(A), lda, strideA, _ptr(B), ldb, strideB, _ptr(C), ldc,
                                                strideC, batch, dtype, _stream(stream)))


def gemm_strided_batched_ex(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC, batch,
                            dtype, stream=None):
    lib = load()
    return _check(lib, lib.gemm_strided_batched_ex(M, N, K, _ptr(A), lda, layout_a, strideA, _ptr(B), ldb, layout_b,
                                                   strideB, _ptr(C), ldc, strideC, batch, dtype, _stream(stream)))


def gemm_strided_batched_act(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC, batch,
                             dtype, activation, slope, stream=None):
    lib = load()
    return _check(lib, lib.gemm_strided_batched_act(M, N, K, _ptr(A), lda, layout_a, strideA, _ptr(B), ldb, layout_b,
                                                    strideB, _ptr(C), ldc, strideC, batch, dtype, activation, slope,
                                                    _stream(stream)))


def gemm_workspace_bytes(M, N, K, batch):
    return int(load().gemm_workspace_bytes(M, N, K, batch))


def gemm_strided_batched_ws(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC, batch,
                            dtype, activation, slope, workspace, workspace_bytes, stream=None):
    lib = load()
    return _check(lib, lib.gemm_strided_batched_ws(M, N, K, _ptr(A), lda, layout_a, strideA, _ptr(B), ldb, layout_b,
                                                   strideB, _ptr(C), ldc, strideC, batch, dtype, activation, slope,
                                                   _ptr(workspace), workspace_bytes, _stream(stream)))


def gemm_strided_batched_noalloc(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC,
                                 batch, dtype, activation, slope, stream=None):
    lib = load()
    return _check(lib, lib.gemm_strided_batched_noalloc(M, N, K, _ptr(A), lda, layout_a, strideA, _ptr(B), ldb,
                                                        layout_b, strideB, _ptr(C), ldc, strideC, batch, dtype,
                                                        activation, slope, _stream(stream)))


def gemm_noalloc_scratch_bytes():
    return int(load().gemm_noalloc_scratch_bytes())


def tsm_gemm_ws_kernel_name(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC, batch,
                            dtype, workspace, workspace_bytes):
    r = load().tsm_gemm_ws_kernel_name(M, N, K, _ptr(A), lda, layout_a, strideA, _ptr(B), ldb, layout_b, strideB,
                                       _ptr(C), ldc, strideC, batch, dtype, _ptr(workspace), workspace_bytes)
    return r.decode() if r else None


def gemm_grouped(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC, rows, groups, dtype,
                 stream=None):
    lib = load()
    return _check(lib, lib.gemm_grouped(M, N, K, _ptr(A), lda, layout_a, strideA, _ptr(B), ldb, layout_b, strideB,
                                        _ptr(C), ldc, strideC, _ptr(rows), groups, dtype, _stream(stream)))


def tsm_status_string(status: int) -> str:
    return load().tsm_status_string(status).decode()


def tsm_last_error_detail() -> str:
    return load().tsm_last_error_detail().decode()


def tsm_gemm_kernel_name(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC, batch,
                         dtype):
    r = load().tsm_gemm_kernel_name(M, N, K, _ptr(A), lda, layout_a, strideA, _ptr(B), ldb, layout_b, strideB,
                                    _ptr(C), ldc, strideC, batch, dtype)
    return r.decode() if r else None


def tsm_gemm_grouped_kernel_name(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC, rows,
                                 groups, dtype):
    r = load().tsm_gemm_grouped_kernel_name(M, N, K, _ptr(A), lda, layout_a, strideA, _ptr(B), ldb, layout_b, strideB,
                                            _ptr(C), ldc, strideC, _ptr(rows), groups, dtype)
    return r.decode() if r else None


def rowsum(R, C, X, row_stride, col_stride, xdtype, out, stream=None):
    lib = load()
    return _check(lib, lib.rowsum(R, C, _ptr(X), row_stride, col_stride, xdtype, _ptr(out), _stream(stream)))


def tsm_rowsum_kernel_name(R, C, X, row_stride, col_stride, xdtype, out):
    r = load().tsm_rowsum_kernel_name(R, C, _ptr(X), row_stride, col_stride, xdtype, _ptr(out))
    return r.decode() if r else None
