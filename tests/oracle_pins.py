"""Pins that tie the CPU oracle to facts outside itself.

Each ``pin_*`` takes an ``oracle.Oracle`` and raises AssertionError when the
oracle disagrees with something the pages or the mathematics fix: printed
values, closed forms, identities, exact integer arithmetic done by numpy,
library conversions, or exact rational arithmetic.  ``test_oracle.py`` runs them
on the real oracle; ``test_oracle_mutants.py`` runs them on copies of the oracle
with one planted mistake each and checks that every mistake is caught.
"""

from __future__ import annotations

import math
import os
from fractions import Fraction

import numpy as np

from workloads.inputs import BF16, F16, bits_to_f64, integer_operands, make_operands, round_f64_to_bits

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, _, v = line.partition("=")
            vals[key.strip()] = v.split()
    return vals


def _store(logical, layout):
    """Storage array for a logical (batch, rows, cols) matrix in the given layout."""
    return logical if layout == "row" else np.ascontiguousarray(logical.transpose(0, 2, 1))


# ---------------------------------------------------------------- decoding
def pin_decode_f16_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.decode(bits, F16)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


def pin_decode_bf16_all_patterns(orc):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = orc.decode(bits, BF16)
    with np.errstate(invalid="ignore"):
        ref = (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    assert np.array_equal(np.signbit(got[~nan]), np.signbit(ref[~nan]))


# ---------------------------------------------------------------- brute force
def _fraction_of_bits(b, fmt):
    return Fraction(float(bits_to_f64(np.array([b], dtype=np.uint16), fmt)[0]))


def pin_bruteforce_tiny(orc):
    """All shapes with M, N, K in {1, 2, 3}: exact products, float64 sum rounded step by step.

    ``float(Fraction)`` rounds correctly, so ``float(Fraction(acc) + a*b)`` is one
    float64 addition of an exactly represented product: the oracle must match
    it bit for bit, and S likewise.
    """
    rng = np.random.default_rng(1234)
    for fmt in (F16, BF16):
        for M in (1, 2, 3):
            for N in (1, 2, 3):
                for K in (1, 2, 3):
                    for a_layout, b_layout in (("row", "row"), ("col", "col"), ("row", "col")):
                        a = rng.uniform(-2, 2, (1, M, K)) * rng.choice([1.0, 2.0 ** -9, 2.0 ** 7], (1, M, K))
                        b = rng.uniform(-2, 2, (1, K, N))
                        A = round_f64_to_bits(a, fmt).reshape(a.shape)
                        B = round_f64_to_bits(b, fmt).reshape(b.shape)
                        C, S = orc.gemm_rows(_store(A, a_layout), _store(B, b_layout), M, N, K, fmt,
                                             a_layout=a_layout, b_layout=b_layout)
                        for i in range(M):
                            for j in range(N):
                                acc, sacc = 0.0, 0.0
                                for k in range(K):
                                    p = _fraction_of_bits(A[0, i, k], fmt) * _fraction_of_bits(B[0, k, j], fmt)
                                    acc = float(Fraction(acc) + p)
                                    sacc = float(Fraction(sacc) + abs(p))
                                assert C[0, i, j] == acc, (fmt, M, N, K, i, j, C[0, i, j], acc)
                                assert S[0, i, j] == sacc, (fmt, M, N, K, i, j, S[0, i, j], sacc)


# ---------------------------------------------------------------- identities
def pin_identity_and_zero(orc):
    for fmt in (F16, BF16):
        for a_layout, b_layout in (("row", "row"), ("row", "col"), ("col", "row")):
            M, K, N = 5, 7, 6
            A, B = make_operands(7, 1, M, N, K, fmt, ("uniform", -1.0, 1.0))
            a = bits_to_f64(A, fmt)
            b = bits_to_f64(B, fmt)
            eyeK = round_f64_to_bits(np.eye(K)[None], fmt).reshape(1, K, K)
            eyeM = round_f64_to_bits(np.eye(M)[None], fmt).reshape(1, M, M)
            C, _ = orc.gemm_rows(_store(A, a_layout), _store(eyeK, b_layout), M, K, K, fmt,
                                 a_layout=a_layout, b_layout=b_layout)
            assert np.array_equal(C, a)
            _, BM = make_operands(8, 1, M, N, M, fmt, ("uniform", -1.0, 1.0))  # B with M rows
            C, _ = orc.gemm_rows(_store(eyeM, a_layout), _store(BM, b_layout), M, N, M, fmt,
                                 a_layout=a_layout, b_layout=b_layout)
            assert np.array_equal(C, bits_to_f64(BM, fmt))
            assert b.shape == (1, K, N)
            Z = np.zeros((1, K, N), dtype=np.uint16)
            C, S = orc.gemm_rows(_store(A, a_layout), _store(Z, b_layout), M, N, K, fmt,
                                 a_layout=a_layout, b_layout=b_layout)
            assert not C.any() and not S.any()
    # K = 0: the empty sum is zero
    C, S = orc.gemm_rows(np.zeros((1, 3, 0), np.uint16), np.zeros((1, 0, 4), np.uint16), 3, 4, 0, F16)
    assert C.shape == (1, 3, 4) and not C.any() and not S.any()


# ---------------------------------------------------------------- printed example and closed forms
def pin_golden_rowsum_ones(orc):
    g = _read_golden("rowsum_ones_2x3.txt")
    M, K, N = int(g["M"][0]), int(g["K"][0]), int(g["N"][0])
    a = np.array([float(v) for v in g["A"]]).reshape(1, M, K)
    b = np.array([float(v) for v in g["B"]]).reshape(1, K, N)
    want = np.array([float(v) for v in g["C"]]).reshape(1, M, N)
    for fmt in (F16, BF16):
        A = round_f64_to_bits(a, fmt).reshape(a.shape)
        B = round_f64_to_bits(b, fmt).reshape(b.shape)
        C, _ = orc.gemm_rows(A, B, M, N, K, fmt)
        assert np.array_equal(C, want), (C, want)


def pin_ones_closed_forms(orc):
    """A = ones gives the column sums of B in every row; B = ones gives the row sums of A.

    ``math.fsum`` returns the correctly rounded exact sum; the oracle's ordered
    float64 sum may differ from it by at most (K-1) * 2^-53 * sum|terms|.
    """
    for fmt in (F16, BF16):
        M, N, K = 4, 5, 300
        A, B = make_operands(11, 1, M, N, K, fmt, ("uniform", -1.0, 1.0))
        a = bits_to_f64(A, fmt)[0]
        b = bits_to_f64(B, fmt)[0]
        ones_a = round_f64_to_bits(np.ones((1, M, K)), fmt).reshape(1, M, K)
        ones_b = round_f64_to_bits(np.ones((1, K, N)), fmt).reshape(1, K, N)
        C, _ = orc.gemm_rows(ones_a, B, M, N, K, fmt)
        for j in range(N):
            exact = math.fsum(b[:, j])
            tol = (K - 1) * 2.0 ** -53 * np.abs(b[:, j]).sum()
            assert abs(C[0, 0, j] - exact) <= tol
            assert np.all(C[0, :, j] == C[0, 0, j])  # independent of i
        C, _ = orc.gemm_rows(A, ones_b, M, N, K, fmt)
        for i in range(M):
            exact = math.fsum(a[i, :])
            tol = (K - 1) * 2.0 ** -53 * np.abs(a[i, :]).sum()
            assert abs(C[0, i, 0] - exact) <= tol
            assert np.all(C[0, i, :] == C[0, i, 0])  # independent of j
        # ones . ones = K exactly
        C, S = orc.gemm_rows(ones_a, ones_b, M, N, K, fmt)
        assert np.all(C == K) and np.all(S == K)
    # six ones summed across a ragged last tile: 6.0
    C, _ = orc.gemm_rows(round_f64_to_bits(np.ones((1, 1, 6)), F16).reshape(1, 1, 6),
                         round_f64_to_bits(np.ones((1, 6, 1)), F16).reshape(1, 6, 1), 1, 1, 6, F16)
    assert C[0, 0, 0] == 6.0


def pin_linearity_in_a(orc):
    """C(2*A1 + A2/4) = 2*C(A1) + C(A2)/4 exactly for A1, A2 of disjoint support.

    Each cell's terms come from exactly one of A1 and A2, and scaling by a power
    of two is exact, so the sums agree bit for bit when computed term by term;
    they are compared against the combination of the two separate sums with the
    float64 error bound, and exactly when A2 is zero in a row.
    """
    M, N, K = 6, 5, 40
    for fmt in (F16, BF16):
        A, B = make_operands(21, 1, M, N, K, fmt, ("uniform", -1.0, 1.0))
        a = bits_to_f64(A, fmt)
        mask = (np.arange(K)[None, None, :] + np.arange(M)[None, :, None]) % 3 == 0
        mask[:, 0, :] = True  # row 0 has A2 = 0 entirely
        a1 = np.where(mask, a, 0.0)
        a2 = np.where(mask, 0.0, a)
        comb = 2.0 * a1 + 0.25 * a2
        A1 = round_f64_to_bits(a1, fmt).reshape(a.shape)
        A2 = round_f64_to_bits(a2, fmt).reshape(a.shape)
        AC = round_f64_to_bits(comb, fmt).reshape(a.shape)
        assert np.array_equal(bits_to_f64(AC, fmt), comb)  # scaling stayed exact
        C1, S1 = orc.gemm_rows(A1, B, M, N, K, fmt)
        C2, S2 = orc.gemm_rows(A2, B, M, N, K, fmt)
        CC, _ = orc.gemm_rows(AC, B, M, N, K, fmt)
        want = 2.0 * C1 + 0.25 * C2
        tol = 2 * K * 2.0 ** -53 * (2.0 * S1 + 0.25 * S2)
        assert np.all(np.abs(CC - want) <= tol)
        assert np.array_equal(CC[0, 0], 2.0 * C1[0, 0])


# ---------------------------------------------------------------- exact integer arithmetic
def pin_integer_exact(orc):
    """Integer entries: every float64 partial sum is exact, so C and S equal numpy's int64 products.

    Covers both layouts of both operands, padded leading dimensions, strided
    batches with and without broadcast operands, a row window, and the cell
    sampler.
    """
    M, N, K, batch = 9, 11, 37, 3
    for fmt in (F16, BF16):
        for a_layout in ("row", "col"):
            for b_layout in ("row", "col"):
                A, B = integer_operands(5, batch, M, N, K, fmt, -3, 3)
                ai = bits_to_f64(A, fmt).astype(np.int64)
                bi = bits_to_f64(B, fmt).astype(np.int64)
                want = np.matmul(ai, bi)
                want_s = np.matmul(np.abs(ai), np.abs(bi))
                As, Bs = _store(A, a_layout), _store(B, b_layout)
                # padded leading dimensions: embed each stored matrix in a wider one
                pa, pb = 3, 5
                Ap = np.zeros((batch, As.shape[1], As.shape[2] + pa), np.uint16)
                Ap[:, :, :As.shape[2]] = As
                Bp = np.zeros((batch, Bs.shape[1], Bs.shape[2] + pb), np.uint16)
                Bp[:, :, :Bs.shape[2]] = Bs
                lda = As.shape[2] + pa
                ldb = Bs.shape[2] + pb
                C, S = orc.gemm_rows(Ap, Bp, M, N, K, fmt, batch=batch, lda=lda, ldb=ldb,
                                     strideA=Ap[0].size, strideB=Bp[0].size,
                                     a_layout=a_layout, b_layout=b_layout)
                assert np.array_equal(C, want) and np.array_equal(S, want_s)
                # a window of rows
                C, _ = orc.gemm_rows(Ap, Bp, M, N, K, fmt, batch=batch, lda=lda, ldb=ldb,
                                     strideA=Ap[0].size, strideB=Bp[0].size,
                                     a_layout=a_layout, b_layout=b_layout, row_begin=2, row_end=7)
                assert np.array_equal(C, want[:, 2:7])
                # broadcast B (stride 0): every problem uses B[0]
                C, _ = orc.gemm_rows(Ap, Bp, M, N, K, fmt, batch=batch, lda=lda, ldb=ldb,
                                     strideA=Ap[0].size, strideB=0,
                                     a_layout=a_layout, b_layout=b_layout)
                assert np.array_equal(C, np.matmul(ai, bi[0:1]))
                # sampled cells
                rng = np.random.default_rng(3)
                z = rng.integers(0, batch, 50)
                i = rng.integers(0, M, 50)
                j = rng.integers(0, N, 50)
                Cp, Sp = orc.gemm_points(Ap, Bp, M, N, K, fmt, z, i, j, lda=lda, ldb=ldb,
                                         strideA=Ap[0].size, strideB=Bp[0].size,
                                         a_layout=a_layout, b_layout=b_layout)
                assert np.array_equal(Cp, want[z, i, j]) and np.array_equal(Sp, want_s[z, i, j])


# ---------------------------------------------------------------- random values against a library product
def pin_random_vs_numpy(orc):
    """Random f16/bf16 operands: C within 2*K*2^-53*S of numpy's float64 matmul.

    numpy's product runs in float64 from exactly decoded values (the library's
    own decode), so the two differ only by float64 summation error.
    """
    for fmt, dist in ((F16, ("uniform", -1.0, 1.0)), (BF16, ("normal", 0.1))):
        for a_layout, b_layout in (("row", "row"), ("row", "col"), ("col", "row")):
            M, N, K, batch = 13, 17, 129, 2
            A, B = make_operands(99, batch, M, N, K, fmt, dist, a_layout, b_layout)
            la = bits_to_f64(A, fmt)
            lb = bits_to_f64(B, fmt)
            if a_layout == "col":
                la = la.transpose(0, 2, 1)
            if b_layout == "col":
                lb = lb.transpose(0, 2, 1)
            want = np.matmul(la, lb)
            C, S = orc.gemm_rows(A, B, M, N, K, fmt, batch=batch, a_layout=a_layout, b_layout=b_layout)
            assert np.all(np.abs(C - want) <= 2 * K * 2.0 ** -53 * S)
            assert np.allclose(S, np.matmul(np.abs(la), np.abs(lb)), rtol=1e-12, atol=0)
            z = np.array([0, 1, 1, 0])
            i = np.array([0, M - 1, 5, 7])
            j = np.array([N - 1, 0, 3, 16])
            Cp, _ = orc.gemm_points(A, B, M, N, K, fmt, z, i, j, strideA=A[0].size, strideB=B[0].size,
                                    a_layout=a_layout, b_layout=b_layout)
            assert np.all(np.abs(Cp - want[z, i, j]) <= 2 * K * 2.0 ** -53 * S[z, i, j])


# ---------------------------------------------------------------- grouped (per-problem row counts)
def pin_grouped_integer(orc):
    """Grouped products on integer entries: group g equals numpy's int64 product of A_g's first m_g rows
    with B_g, where m_g is rows[g] clamped to [0, M] (counts below 0, inside, at and above M)."""
    M, N, K, groups = 10, 7, 33, 5
    rows = [-3, 0, 4, M, M + 6]
    for fmt in (F16, BF16):
        for a_layout, b_layout in (("row", "row"), ("row", "col"), ("col", "row")):
            A, B = integer_operands(8, groups, M, N, K, fmt, -2, 2)
            ai = bits_to_f64(A, fmt).astype(np.int64)
            bi = bits_to_f64(B, fmt).astype(np.int64)
            As, Bs = _store(A, a_layout), _store(B, b_layout)
            # trailing zero slack keeps a wrongly indexed read (a planted mistake) inside the buffer
            slack = 4 * (M + N + K) ** 2
            Ap = np.zeros(As.size + slack, np.uint16)
            Ap[:As.size] = As.reshape(-1)
            Bp = np.zeros(Bs.size + slack, np.uint16)
            Bp[:Bs.size] = Bs.reshape(-1)
            got = orc.gemm_grouped(Ap, Bp, M, N, K, fmt, rows, strideA=As[0].size, strideB=Bs[0].size,
                                   a_layout=a_layout, b_layout=b_layout)
            assert len(got) == groups
            for g, (C, S) in enumerate(got):
                m = min(max(rows[g], 0), M)
                assert C.shape == (m, N) and S.shape == (m, N)
                assert np.array_equal(C, np.matmul(ai[g, :m], bi[g]))
                assert np.array_equal(S, np.matmul(np.abs(ai[g, :m]), np.abs(bi[g])))


# ---------------------------------------------------------------- row sums
def pin_rowsum_printed_examples(orc):
    """The 2x3 matrix of ones sums to [3.0, 3.0] ("A Dumb Triton Runtime Error", "What I ran"), in every
    input format; six ones across a ragged tile window sum to 6 (its Step 2, n_cols = 6)."""
    g = _read_golden("rowsum_ones_2x3.txt")
    R, C = int(g["M"][0]), int(g["K"][0])
    x = np.array([float(v) for v in g["A"]]).reshape(R, C)
    want = np.array([float(v) for v in g["C"]])
    for fmt in ("f32", F16, BF16):
        X = x.astype(np.float32) if fmt == "f32" else round_f64_to_bits(x, fmt).reshape(R, C)
        out, S = orc.rowsum(X, R, C, C, 1, fmt)
        assert np.array_equal(out, want) and np.array_equal(S, want)
        out, _ = orc.rowsum(np.ones(6, np.float32) if fmt == "f32" else round_f64_to_bits(np.ones(6), fmt),
                            1, 6, 6, 1, fmt)
        assert out[0] == 6.0


def pin_rowsum_integer_views(orc):
    """Integer entries: exact sums, equal to numpy's int64 row sums of the same logical matrix, through a
    contiguous, a padded, a column-strided and a transposed view (and empty rows give 0)."""
    rng = np.random.default_rng(12)
    R, C = 7, 45
    for fmt in ("f32", F16, BF16):
        vals = rng.integers(-50, 51, (R, C))
        store = (lambda a: a.astype(np.float32)) if fmt == "f32" else (lambda a: round_f64_to_bits(a.astype(float), fmt))
        want = vals.sum(axis=1)
        want_s = np.abs(vals).sum(axis=1)
        out, S = orc.rowsum(store(vals).reshape(-1), R, C, C, 1, fmt)
        assert np.array_equal(out, want) and np.array_equal(S, want_s)
        padded = np.zeros((R, C + 9), np.int64)
        padded[:, :C] = vals
        out, _ = orc.rowsum(store(padded).reshape(-1), R, C, C + 9, 1, fmt)
        assert np.array_equal(out, want)
        strided = np.zeros((R, 3 * C), np.int64)
        strided[:, ::3] = vals
        out, _ = orc.rowsum(store(strided).reshape(-1), R, C, 3 * C, 3, fmt)
        assert np.array_equal(out, want)
        # the transposed storage: element (r, c) at c*R + r
        out, _ = orc.rowsum(store(np.ascontiguousarray(vals.T)).reshape(-1), R, C, 1, R, fmt)
        assert np.array_equal(out, want)
        out, S = orc.rowsum(store(vals).reshape(-1), R, 0, C, 1, fmt)
        assert not out.any() and not S.any()


def pin_rowsum_random_vs_fsum(orc):
    """Random float32 rows (the page's 8 x 1000 shape): within the float64 summation bound of math.fsum,
    the correctly rounded exact sum."""
    rng = np.random.default_rng(13)
    R, C = 8, 1000
    x = rng.standard_normal((R, C)).astype(np.float32)
    out, S = orc.rowsum(x.reshape(-1), R, C, C, 1, "f32")
    for r in range(R):
        exact = math.fsum(float(v) for v in x[r])
        assert abs(out[r] - exact) <= (C - 1) * 2.0 ** -53 * S[r]
        assert abs(S[r] - math.fsum(abs(float(v)) for v in x[r])) <= (C - 1) * 2.0 ** -53 * S[r]


ALL_PINS = [
    pin_decode_f16_all_patterns,
    pin_decode_bf16_all_patterns,
    pin_bruteforce_tiny,
    pin_identity_and_zero,
    pin_golden_rowsum_ones,
    pin_ones_closed_forms,
    pin_linearity_in_a,
    pin_integer_exact,
    pin_random_vs_numpy,
    pin_grouped_integer,
    pin_rowsum_printed_examples,
    pin_rowsum_integer_views,
    pin_rowsum_random_vs_fsum,
]
