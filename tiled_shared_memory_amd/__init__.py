"""Blocked GEMM for AMD MI355X (gfx950): C = A.B, f16/bf16 in, float32 accumulate.

The C entry points (``include/tsm_gemm.h``) are exposed under the same names
by ``_lib``; ``matmul`` is a convenience wrapper that reads sizes, strides and
layouts off torch tensors and allocates the output with torch.  torch serves
only as device memory and streams: every multiply-add runs in the library's
HIP kernels.
"""

from __future__ import annotations

from ._lib import (TSM_ACT_LEAKY_RELU, TSM_ACT_NONE, TSM_ACT_RELU, TSM_BF16_BF16, TSM_BF16_F16,  # noqa: F401
                   TSM_BF16_F32, TSM_COL, TSM_ERROR_INVALID_VALUE, TSM_ERROR_LAUNCH, TSM_ERROR_NOT_SUPPORTED,
                   TSM_F16_BF16, TSM_F16_F16, TSM_F16_F32, TSM_ROW, TSM_ROWSUM_BF16, TSM_ROWSUM_F16, TSM_ROWSUM_F32,
                   TSM_SUCCESS, TsmError, gemm, gemm_ex, gemm_grouped, gemm_strided_batched,
                   gemm_noalloc_scratch_bytes, gemm_strided_batched_act, gemm_strided_batched_ex,
                   gemm_strided_batched_noalloc, gemm_strided_batched_ws, gemm_workspace_bytes,
                   load, rowsum, tsm_gemm_grouped_kernel_name, tsm_gemm_kernel_name, tsm_gemm_ws_kernel_name,
                   tsm_last_error_detail, tsm_rowsum_kernel_name, tsm_status_string)


def dtype_code(in_dtype, out_dtype) -> int:
    import torch

    table = {
        (torch.float16, torch.float32): TSM_F16_F32,
        (torch.float16, torch.float16): TSM_F16_F16,
        (torch.bfloat16, torch.float32): TSM_BF16_F32,
        (torch.bfloat16, torch.float16): TSM_BF16_F16,
        (torch.float16, torch.bfloat16): TSM_F16_BF16,
        (torch.bfloat16, torch.bfloat16): TSM_BF16_BF16,
    }
    try:
        return table[(in_dtype, out_dtype)]
    except KeyError:
        raise TsmError(TSM_ERROR_INVALID_VALUE, f"unsupported dtypes {in_dtype} -> {out_dtype}") from None


def _layout(t, rows_dim_size, cols_dim_size):
    """(layout, ld) of the last two dims of a logical rows x cols tensor view."""
    s_r, s_c = t.stride(-2), t.stride(-1)
    if s_c == 1 and (s_r >= max(1, cols_dim_size) or rows_dim_size <= 1):
        return TSM_ROW, max(s_r, max(1, cols_dim_size))
    if s_r == 1 and (s_c >= max(1, rows_dim_size) or cols_dim_size <= 1):
        return TSM_COL, max(s_c, max(1, rows_dim_size))
    raise TsmError(TSM_ERROR_INVALID_VALUE, "operand must be row- or column-major in its last two dims")


_ACTIVATIONS = {None: TSM_ACT_NONE, "relu": TSM_ACT_RELU, "leaky_relu": TSM_ACT_LEAKY_RELU}


def workspace_for(a, b):
    """A float32 CUDA tensor big enough for ``matmul(a, b, workspace=...)`` to split K, or None when the shape
    does not split.  Allocate it once and reuse it across calls of that shape on one stream."""
    import torch

    M, K, N = a.shape[-2], a.shape[-1], b.shape[-1]
    batch = max(a.shape[0] if a.dim() == 3 else 1, b.shape[0] if b.dim() == 3 else 1)
    nbytes = gemm_workspace_bytes(M, N, K, batch)
    return torch.empty((nbytes + 3) // 4, dtype=torch.float32, device=a.device) if nbytes else None


def matmul(a, b, *, out=None, out_dtype=None, activation=None, slope=0.01, workspace=None, stream=None):
    """C = act(A.B) for CUDA tensors ``a`` (..., M, K) and ``b`` (..., K, N) in float16 or bfloat16.

    2-D operands give one product, 3-D ones a strided batch (a batch dim of
    size 1 or stride 0 broadcasts).  Each operand may be row-major or
    column-major in its last two dims (e.g. ``w.t()``); the result is row-major
    float32 (default), float16 or bfloat16.  ``activation`` is None, "relu" or
    "leaky_relu" (with ``slope``), fused into the kernels' epilogue.  With a
    ``workspace`` (see ``workspace_for``) products with few output tiles and
    deep K split K through it.
    """
    import torch

    if a.dtype != b.dtype:
        raise TsmError(TSM_ERROR_INVALID_VALUE, "a and b must share a dtype")
    out_dtype = out_dtype or (out.dtype if out is not None else torch.float32)
    code = dtype_code(a.dtype, out_dtype)
    M, K = a.shape[-2], a.shape[-1]
    K2, N = b.shape[-2], b.shape[-1]
    if K != K2:
        raise TsmError(TSM_ERROR_INVALID_VALUE, f"inner sizes differ: {K} vs {K2}")
    batched = a.dim() == 3 or b.dim() == 3
    batch = max(a.shape[0] if a.dim() == 3 else 1, b.shape[0] if b.dim() == 3 else 1)
    if out is None:
        out = torch.empty((batch, M, N) if batched else (M, N), dtype=out_dtype, device=a.device)
    la, lda = _layout(a, M, K)
    lb, ldb = _layout(b, K, N)
    if out.stride(-1) != 1:
        raise TsmError(TSM_ERROR_INVALID_VALUE, "out must be row-major")
    ldc = out.stride(-2) if M > 1 else max(1, N)

    def bstride(t):
        return 0 if t.dim() == 2 or t.shape[0] == 1 else t.stride(0)

    if activation not in _ACTIVATIONS:
        raise TsmError(TSM_ERROR_INVALID_VALUE, f"unknown activation {activation!r}")
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    gemm_strided_batched_ws(M, N, K, a, lda, la, bstride(a), b, ldb, lb, bstride(b), out, ldc,
                            out.stride(0) if out.dim() == 3 else 0, batch, code, _ACTIVATIONS[activation], slope,
                            workspace, ws_bytes, stream)
    return out
