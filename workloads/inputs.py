"""Seeded synthetic operands for the blocked GEMM C = A.B.

This module is shared by the CPU oracle's tests and by the GPU path's tests and
benchmark.  It holds no GEMM arithmetic: it draws float64 values from a seeded
generator, rounds them to 16-bit storage formats and lays them out in memory.

Reading of the workload statement (the pages fix neither generator nor draw
order, so this is a plain fixed choice that can be drawn in parallel):
  * generator: numpy's PCG64 ``default_rng``, one per block of 64 logical rows,
    seeded with ``[seed, operand, problem, block]`` (operand 0 = A, 1 = B);
  * within a block, values are drawn in float64 row by row;
  * "uniform[lo,hi]" is ``rng.uniform(lo, hi)``; "normal(0,1) scaled by s" is
    ``rng.standard_normal() * s``;
  * rounding: round-to-nearest, ties-to-even, straight from float64 to f16 or bf16
    (no intermediate float32 step), subnormals kept;
  * a column-major operand is the storage transpose of the drawn logical matrix,
    so the layout never changes the values.

Blocks are independent streams, so the values never depend on how many
threads draw them, which the tests check.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

_WORKERS = max(1, min(8, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4))

F16 = "f16"
BF16 = "bf16"

# (explicit mantissa bits, minimum normal exponent, exponent bias, +inf pattern)
_FORMATS = {
    F16: (10, -14, 15, 0x7C00, 0x7E00),
    BF16: (7, -126, 127, 0x7F80, 0x7FC0),
}


def _round_bits_general(x: np.ndarray, fmt: str) -> np.ndarray:
    """Round float64 values to ``fmt`` (ties to even), any magnitude.

    Works on the IEEE-754 bit pattern of the double: the 53-bit significand is
    shifted right by the number of bits the target cannot hold at that exponent
    (more for values below the target's smallest normal), the dropped bits
    decide the rounding, and a carry out of the kept bits moves the value into
    the next binade by plain integer addition.
    """
    man, emin, bias, inf_bits, nan_bits = _FORMATS[fmt]
    b = x.view(np.uint64)
    sign = (b >> np.uint64(63)).astype(np.uint16)
    efield = ((b >> np.uint64(52)) & np.uint64(0x7FF)).astype(np.int64)
    frac = b & np.uint64((1 << 52) - 1)
    special = efield == 0x7FF
    tiny = efield == 0  # zero or a float64 subnormal: far below half the target's least subnormal
    e = efield - 1023
    sig = np.where(tiny, np.uint64(0), frac | np.uint64(1 << 52))
    drop = (52 - man) + np.maximum(0, emin - e)
    drop = np.minimum(drop, 62).astype(np.uint64)
    kept = sig >> drop
    rem = sig & ((np.uint64(1) << drop) - np.uint64(1))
    half = np.uint64(1) << (drop - np.uint64(1))
    up = (rem > half) | ((rem == half) & ((kept & np.uint64(1)) == np.uint64(1)))
    kept = kept + up.astype(np.uint64)
    normal = e >= emin
    ebits = np.where(normal, e + bias - 1, 0).astype(np.int64)
    mag = np.where(normal, (ebits.astype(np.uint64) << np.uint64(man)) + kept, kept)
    mag = np.minimum(mag, np.uint64(inf_bits))
    mag = np.where(special, np.where(frac == 0, np.uint64(inf_bits), np.uint64(nan_bits)), mag)
    return (mag.astype(np.uint16) | (sign << np.uint16(15))).astype(np.uint16)


def round_f64_to_bits(x, fmt: str) -> np.ndarray:
    """Round float64 values to the nearest ``fmt`` value (ties to even); uint16 patterns.

    Fast path for values whose result is a normal ``fmt`` number: adding
    (half - 1 + lowest kept bit) to the double's bit pattern and truncating
    rounds the significand to nearest-even (a carry moves into the exponent
    field by itself); the exponent is then re-biased.  Everything else (zero,
    subnormal results, overflow, inf/NaN) takes the general path.
    """
    man, emin, bias, inf_bits, nan_bits = _FORMATS[fmt]
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float64))
    shape = x.shape
    x = x.reshape(-1)
    drop = np.uint64(52 - man)
    b = x.view(np.uint64)
    r = (b + ((np.uint64(1) << (drop - np.uint64(1))) - np.uint64(1) + ((b >> drop) & np.uint64(1)))) >> drop
    e11 = ((r >> np.uint64(man)) & np.uint64(0x7FF)).astype(np.int64) - 1023
    emax = (inf_bits >> man) - bias  # exponent of inf; finite normals stay below it
    ok = (e11 >= emin) & (e11 < emax)
    out = (((r >> np.uint64(man + 11)) << np.uint64(15)) | (((e11 + bias).astype(np.uint64) & np.uint64(0xFF))
                                                            << np.uint64(man)) | (r & np.uint64((1 << man) - 1)))
    out = out.astype(np.uint16)
    if not ok.all():
        idx = np.nonzero(~ok)[0]
        out[idx] = _round_bits_general(np.ascontiguousarray(x[idx]), fmt)
    return out.reshape(shape)


def bits_to_f64(bits, fmt: str) -> np.ndarray:
    """Exact float64 values of 16-bit patterns, via numpy's own float types.

    f16 goes through ``numpy.float16``; bf16 is the upper half of a float32, so
    the pattern shifted left by 16 is reinterpreted as ``numpy.float32``.
    """
    bits = np.asarray(bits, dtype=np.uint16)
    if fmt == F16:
        return bits.view(np.float16).astype(np.float64)
    if fmt == BF16:
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(fmt)


def _draw(rng: np.random.Generator, dist: tuple, n: int) -> np.ndarray:
    kind = dist[0]
    if kind == "uniform" and len(dist) == 3:
        return rng.uniform(dist[1], dist[2], n)
    if kind == "normal" and len(dist) == 2:
        return rng.standard_normal(n) * dist[1]
    raise ValueError(f"distribution {dist!r}: expected ('uniform', lo, hi) or ('normal', scale)")


ROWS_PER_BLOCK = 64


def draw_matrix_bits(seed: int, operand: int, z: int, dist, rows: int, cols: int, fmt: str,
                     workers: int | None = None, out: np.ndarray | None = None):
    """Draw a logical rows x cols matrix and round it to ``fmt``.

    Row block b (rows [64*b, 64*b + 64)) comes from its own generator,
    ``numpy.random.default_rng([seed, operand, z, b])``, filled row by row.
    Blocks are independent, so they are drawn on a thread pool (numpy releases
    the GIL while filling); the values do not depend on the number of workers.
    """
    if out is None:
        out = np.empty((rows, cols), dtype=np.uint16)
    if rows == 0 or cols == 0:
        return out

    def work(b):
        r0 = b * ROWS_PER_BLOCK
        r1 = min(rows, r0 + ROWS_PER_BLOCK)
        rng = np.random.default_rng([seed, operand, z, b])
        # fill in pieces of about 64K values to keep temporaries in cache
        step = max(1, (1 << 16) // cols)
        for q0 in range(r0, r1, step):
            q1 = min(r1, q0 + step)
            out[q0:q1] = round_f64_to_bits(_draw(rng, dist, (q1 - q0) * cols), fmt).reshape(q1 - q0, cols)

    nblocks = (rows + ROWS_PER_BLOCK - 1) // ROWS_PER_BLOCK
    with ThreadPoolExecutor(max_workers=workers or _WORKERS) as pool:
        list(pool.map(work, range(nblocks)))
    return out


def make_operands(seed: int, batch: int, M: int, N: int, K: int, fmt: str, dist: tuple,
                  a_layout: str = "row", b_layout: str = "row", workers: int | None = None):
    """Seeded operands for a (batched) GEMM.

    Returns ``(A, B)`` as contiguous uint16 arrays in storage order:
      A: (batch, M, K) if ``a_layout == "row"``, else (batch, K, M);
      B: (batch, K, N) if ``b_layout == "row"``, else (batch, N, K).
    The logical A of problem z is operand 0, the logical B operand 1 (see
    ``draw_matrix_bits`` for the generator of each row block).
    """
    A = np.empty((batch, M, K), dtype=np.uint16)
    B = np.empty((batch, K, N), dtype=np.uint16)
    for z in range(batch):
        draw_matrix_bits(seed, 0, z, dist, M, K, fmt, workers, out=A[z])
        draw_matrix_bits(seed, 1, z, dist, K, N, fmt, workers, out=B[z])
    if a_layout == "col":
        A = np.ascontiguousarray(A.transpose(0, 2, 1))
    if b_layout == "col":
        B = np.ascontiguousarray(B.transpose(0, 2, 1))
    return A, B


def integer_operands(seed: int, batch: int, M: int, N: int, K: int, fmt: str, lo: int = -2, hi: int = 2,
                     a_layout: str = "row", b_layout: str = "row"):
    """Operands with integer entries in [lo, hi] (exact in f16 and bf16).

    With |entries| <= 2 every partial sum of a product is an integer of magnitude
    at most 4K, exact in float32 for K < 2**22, so any accumulation order gives
    the same float32 result.
    """
    rng = np.random.default_rng(seed)
    a = rng.integers(lo, hi + 1, size=(batch, M, K)).astype(np.float64)
    b = rng.integers(lo, hi + 1, size=(batch, K, N)).astype(np.float64)
    A = round_f64_to_bits(a, fmt).reshape(a.shape)
    B = round_f64_to_bits(b, fmt).reshape(b.shape)
    if a_layout == "col":
        A = np.ascontiguousarray(A.transpose(0, 2, 1))
    if b_layout == "col":
        B = np.ascontiguousarray(B.transpose(0, 2, 1))
    return A, B
