"""CPU oracle for C = A.B -- test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg
may import this package.  The GPU library never calls it, and the two share no
code: the oracle is plain C (``gemm_oracle.c``, built with gcc) plus this ctypes
wrapper, and it reads the same 16-bit patterns the GPU receives.

Functions:
  gemm_rows(...)   -> (C, S): full rows of every problem, float64
  gemm_points(...) -> (C, S): selected cells (sampled checks at full size)
  gemm_grouped(...) -> [(C_g, S_g)]: the first m_g rows of each problem
  rowsum(...)       -> (out, S): row sums of a strided matrix, float64
  decode(bits, fmt)         : the oracle's own exact 16-bit -> float64 decode
  bound(...)                : the per-element acceptance bound

``C`` is the exact-product float64 sum in increasing k and ``S`` the sum of the
products' magnitudes.  See ``gemm_oracle.c`` for the passages followed.
"""

from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "gemm_oracle.c")
LIBRARY = os.path.join(_HERE, "libtsm_oracle.so")
CFLAGS = ["-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall", "-Wextra"]

_FMT = {"f16": 0, "bf16": 1}
_LAYOUT = {"row": 0, "col": 1}

U = 2.0 ** -24  # unit roundoff of float32


def build(source: str = SOURCE, out: str = LIBRARY, extra=()) -> str:
    """Compile the oracle with gcc (no -ffast-math: the sums must stay in order)."""
    cmd = ["gcc", *CFLAGS, *extra, source, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


class Oracle:
    """ctypes handle on one build of the oracle library."""

    def __init__(self, path: str = LIBRARY):
        stale = path == LIBRARY and os.path.exists(path) and os.path.getmtime(SOURCE) > os.path.getmtime(path)
        if not os.path.exists(path) or stale:
            build(out=path)
        self.path = path
        lib = ctypes.CDLL(path)
        i64, ptr, i32 = ctypes.c_int64, ctypes.c_void_p, ctypes.c_int
        lib.tsm_oracle_gemm_rows.argtypes = [i64, i64, i64, i64, i32,
                                             ptr, i64, i64, i32,
                                             ptr, i64, i64, i32,
                                             i64, i64, ptr, ptr]
        lib.tsm_oracle_gemm_rows.restype = i32
        lib.tsm_oracle_gemm_points.argtypes = [i64, i64, i64, i32,
                                               ptr, i64, i64, i32,
                                               ptr, i64, i64, i32,
                                               i64, ptr, ptr, ptr, ptr, ptr]
        lib.tsm_oracle_gemm_points.restype = None
        lib.tsm_oracle_decode.argtypes = [ptr, i64, i32, ptr]
        lib.tsm_oracle_decode.restype = None
        lib.tsm_oracle_rowsum.argtypes = [i64, i64, ptr, i64, i64, i32, ptr, ptr]
        lib.tsm_oracle_rowsum.restype = None
        lib.tsm_oracle_threads.argtypes = []
        lib.tsm_oracle_threads.restype = i32
        self.lib = lib

    def threads(self) -> int:
        return int(self.lib.tsm_oracle_threads())

    def decode(self, bits, fmt: str) -> np.ndarray:
        bits = np.ascontiguousarray(bits, dtype=np.uint16)
        out = np.empty(bits.shape, dtype=np.float64)
        self.lib.tsm_oracle_decode(bits.ctypes.data, bits.size, _FMT[fmt], out.ctypes.data)
        return out

    def gemm_rows(self, A, B, M, N, K, fmt, *, batch=1, lda=None, ldb=None, strideA=None, strideB=None,
                  a_layout="row", b_layout="row", row_begin=0, row_end=None, want_s=True):
        """Rows [row_begin, row_end) of every problem; returns (C, S) of shape (batch, rows, N)."""
        A = np.ascontiguousarray(A, dtype=np.uint16)
        B = np.ascontiguousarray(B, dtype=np.uint16)
        if lda is None:
            lda = K if a_layout == "row" else M
        if ldb is None:
            ldb = N if b_layout == "row" else K
        strideA = A.size // max(batch, 1) if strideA is None else strideA
        strideB = B.size // max(batch, 1) if strideB is None else strideB
        row_end = M if row_end is None else min(row_end, M)
        rows = max(0, row_end - row_begin)
        C = np.zeros((batch, rows, N), dtype=np.float64)
        S = np.zeros((batch, rows, N), dtype=np.float64) if want_s else None
        rc = self.lib.tsm_oracle_gemm_rows(batch, M, N, K, _FMT[fmt],
                                           A.ctypes.data, lda, strideA, _LAYOUT[a_layout],
                                           B.ctypes.data, ldb, strideB, _LAYOUT[b_layout],
                                           row_begin, row_end, C.ctypes.data,
                                           S.ctypes.data if want_s else None)
        if rc != 0:
            raise MemoryError("oracle could not allocate its float64 operand copies")
        return C, S

    def gemm_points(self, A, B, M, N, K, fmt, z, i, j, *, lda=None, ldb=None, strideA=0, strideB=0,
                    a_layout="row", b_layout="row"):
        """Cells (z[t], i[t], j[t]); returns (C, S) as float64 vectors."""
        A = np.ascontiguousarray(A, dtype=np.uint16)
        B = np.ascontiguousarray(B, dtype=np.uint16)
        if lda is None:
            lda = K if a_layout == "row" else M
        if ldb is None:
            ldb = N if b_layout == "row" else K
        z = np.ascontiguousarray(z, dtype=np.int64)
        i = np.ascontiguousarray(i, dtype=np.int64)
        j = np.ascontiguousarray(j, dtype=np.int64)
        n = z.size
        C = np.empty(n, dtype=np.float64)
        S = np.empty(n, dtype=np.float64)
        self.lib.tsm_oracle_gemm_points(M, N, K, _FMT[fmt],
                                        A.ctypes.data, lda, strideA, _LAYOUT[a_layout],
                                        B.ctypes.data, ldb, strideB, _LAYOUT[b_layout],
                                        n, z.ctypes.data, i.ctypes.data, j.ctypes.data,
                                        C.ctypes.data, S.ctypes.data)
        return C, S


    def gemm_grouped(self, A, B, M, N, K, fmt, rows, *, lda=None, ldb=None, strideA=None, strideB=None,
                     a_layout="row", b_layout="row"):
        """Grouped product: for problem g, C_g = A_g[0:m_g] . B_g with m_g = rows[g] clamped to [0, M].

        The mixture-of-experts slice of the Intel XPU Triton README (section "Use
        Tensor Descriptors to load tl.dot arguments and save results"): expert g
        multiplies only its first m_g token rows.  Each group is gemm_rows on
        that problem alone, rows 0 .. m_g - 1.  Returns a list of (C_g, S_g) of
        shape (m_g, N).
        """
        groups = len(rows)
        Af = np.ascontiguousarray(A, dtype=np.uint16).reshape(-1)
        Bf = np.ascontiguousarray(B, dtype=np.uint16).reshape(-1)
        strideA = Af.size // max(groups, 1) if strideA is None else strideA
        strideB = Bf.size // max(groups, 1) if strideB is None else strideB
        out = []
        for g in range(groups):
            m = min(max(int(rows[g]), 0), M)
            C, S = self.gemm_rows(Af[g * strideA:], Bf[g * strideB:], M, N, K, fmt, batch=1, lda=lda, ldb=ldb,
                                  strideA=0, strideB=0, a_layout=a_layout, b_layout=b_layout, row_begin=0,
                                  row_end=m)
            out.append((C[0], S[0]))
        return out


    def rowsum(self, X, R, C, row_stride, col_stride, fmt):
        """Row sums out[r] = sum_c X[r*row_stride + c*col_stride] and S[r] = sum_c |.| (float64).

        X is the flat storage (uint16 patterns for "f16"/"bf16", float32 for "f32").
        """
        code = {"f16": 0, "bf16": 1, "f32": 2}[fmt]
        X = np.ascontiguousarray(X, dtype=np.float32 if fmt == "f32" else np.uint16).reshape(-1)
        out = np.zeros(R, dtype=np.float64)
        S = np.zeros(R, dtype=np.float64)
        self.lib.tsm_oracle_rowsum(R, C, X.ctypes.data, row_stride, col_stride, code, out.ctypes.data,
                                   S.ctypes.data)
        return out, S


_DEFAULT = None


def default() -> Oracle:
    global _DEFAULT
    if _DEFAULT is None:
        _DEFAULT = Oracle()
    return _DEFAULT


def half_ulp_f16(x) -> np.ndarray:
    """Half the spacing of f16 numbers at |x| (float64), 2^-25 at and below the subnormal range.

    For a value stored as f16 by round-to-nearest this is an upper bound on the
    rounding error of that store.
    """
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.where(ax > 0, np.maximum(e, -14.0), -14.0)
    return 0.5 * np.exp2(e - 10.0)


def half_ulp_bf16(x) -> np.ndarray:
    """Half the spacing of bf16 numbers at |x| (float64), 2^-134 at and below the subnormal range."""
    ax = np.abs(np.asarray(x, dtype=np.float64))
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    e = np.where(ax > 0, np.maximum(e, -126.0), -126.0)
    return 0.5 * np.exp2(e - 7.0)


ACT_NONE, ACT_RELU, ACT_LEAKY_RELU = 0, 1, 2


def activate(C, act: int, slope: float = 0.0) -> np.ndarray:
    """The epilogue activation on exact (float64) results: x, max(x, 0), or x > 0 ? x : slope * x."""
    C = np.asarray(C, dtype=np.float64)
    if act == ACT_NONE:
        return C
    if act == ACT_RELU:
        return np.where(C > 0, C, 0.0)
    return np.where(C > 0, C, float(slope) * C)


def bound(K: int, S, out_fmt: str, c_gpu=None, act: int = ACT_NONE, slope: float = 0.0) -> np.ndarray:
    """Per-element acceptance bound on |C_gpu - act(C_ref)|.

    K * 2^-24 * S bounds the float32 accumulation for any summation order under
    round-to-nearest.  An activation with Lipschitz constant L (1 for ReLU,
    max(1, |slope|) for leaky ReLU) scales it by L, and leaky ReLU's float32
    product adds half a float32 ulp of the result.  A 16-bit output adds half an
    ulp of its format at the stored value.
    """
    lip = max(1.0, abs(float(slope))) if act == ACT_LEAKY_RELU else 1.0
    b = lip * float(K) * U * np.asarray(S, dtype=np.float64)
    if act == ACT_LEAKY_RELU:
        b = b + U * np.abs(np.asarray(c_gpu, dtype=np.float64))
    if out_fmt == "f16":
        b = b + half_ulp_f16(c_gpu)
    elif out_fmt == "bf16":
        b = b + half_ulp_bf16(c_gpu)
    return b
