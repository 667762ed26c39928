/*
 * CPU oracle for the blocked matrix product C = A.B -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the package smoke check and the benchmark's CPU-baseline
 * leg load this file's library.  The GPU path never calls it and shares no code
 * with it.
 *
 * What it computes.  The K-tiled, scratchpad-staged kernel ("The PTSS Cliff",
 * sections "The Arithmetic of 'Fully Unrolled K'" and "The Idea: Stage in SLM,
 * Tile K") reorganises where operands live and in which order the K terms are
 * added, but its result is the plain matrix product: every output cell is the
 * sum over k of A[i][k] * B[k][j].  The oracle is that definition, written out:
 *
 *   1. decode the very 16-bit patterns the GPU receives (f16 or bf16) into
 *      float64 -- exactly, from the IEEE-754 field definitions;
 *   2. C[z][i][j] = sum_{k=0..K-1} A[z][i][k] * B[z][k][j], a naive triple loop
 *      summing in float64 in increasing k;
 *   3. S[z][i][j] = sum_k |A[z][i][k] * B[z][k][j]|, in the same loop; the
 *      acceptance bound of a float32-accumulating GEMM is proportional to it.
 *
 * A product of two f16 (11-bit significands) or two bf16 (8-bit) values is
 * exact in float64, and the float64 summation error is at most
 * (K-1) * 2^-53 * S, far below the float32 accumulation bound K * 2^-24 * S.
 *
 * Out-of-range K terms contribute the additive identity, the padding a masked
 * tile load must use ("A Dumb Triton Runtime Error", Step 2 on boundary masking
 * and the -inf padding trap); in this definition there are simply no such terms.
 *
 * Storage: matrices are 16-bit patterns.  Logical element (r, c) of a row-major
 * matrix with leading dimension ld is X[r*ld + c]; of a column-major one,
 * X[c*ld + r].  Problem z of a strided batch starts at X + z*stride.  All
 * offsets are 64-bit (the Intel XPU Triton README, "Avoid int32 Overflow").
 *
 * Threads: OpenMP over output rows; every cell is still one sequential sum.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* f16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.  Exponent field
 * 0 holds zero and subnormals (fraction * 2^-24); field 31 holds inf/NaN. */
static double decode_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* bf16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.  Exponent
 * field 0 holds zero and subnormals (fraction * 2^-133); 255 holds inf/NaN. */
static double decode_bf16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xff;
    int f = h & 0x7f;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);
    return sign ? -v : v;
}

static double decode(uint16_t h, int fmt) { return fmt ? decode_bf16(h) : decode_f16(h); }

/* Logical element (r, c) of a stored matrix. */
static uint16_t element(const uint16_t *X, int64_t r, int64_t c, int64_t ld, int col_major) {
    return col_major ? X[c * ld + r] : X[r * ld + c];
}

/* Decode every 16-bit pattern of an array (used by the tests to pin the two
 * decoders against library conversions). fmt: 0 = f16, 1 = bf16. */
void tsm_oracle_decode(const uint16_t *bits, int64_t n, int fmt, double *out) {
    for (int64_t t = 0; t < n; ++t) out[t] = decode(bits[t], fmt);
}

/*
 * Rows [row_begin, row_end) of every problem z in [0, batch): all N columns.
 * C and S (either may be NULL) receive (batch, row_end - row_begin, N) values,
 * dense row-major.  fmt: 0 = f16 operands, 1 = bf16 operands.
 * Returns 0, or -1 if scratch memory could not be allocated.
 *
 * Step 1 (decode) fills float64 copies of the A rows and of B; the copy of B is
 * kept column by column so step 2's sum over k walks memory in order.  This
 * changes where values sit, not which values are added or in what order.
 */
int tsm_oracle_gemm_rows(int64_t batch, int64_t M, int64_t N, int64_t K, int fmt,
                         const uint16_t *A, int64_t lda, int64_t strideA, int a_col,
                         const uint16_t *B, int64_t ldb, int64_t strideB, int b_col,
                         int64_t row_begin, int64_t row_end, double *C, double *S) {
    if (row_end > M) row_end = M;
    if (row_begin < 0) row_begin = 0;
    int64_t rows = row_end - row_begin;
    if (batch <= 0 || rows <= 0 || N <= 0) return 0;
    size_t kk = K > 0 ? (size_t)K : 1;
    double *a = (double *)malloc(sizeof(double) * (size_t)rows * kk);
    double *b = (double *)malloc(sizeof(double) * (size_t)N * kk);
    if (!a || !b) {
        free(a);
        free(b);
        return -1;
    }
    for (int64_t z = 0; z < batch; ++z) {
        const uint16_t *Az = A + z * strideA;
        const uint16_t *Bz = B + z * strideB;
        /* step 1: exact decode */
#pragma omp parallel for schedule(static)
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t k = 0; k < K; ++k)
                a[r * K + k] = decode(element(Az, row_begin + r, k, lda, a_col), fmt);
#pragma omp parallel for schedule(static)
        for (int64_t j = 0; j < N; ++j)
            for (int64_t k = 0; k < K; ++k)
                b[j * K + k] = decode(element(Bz, k, j, ldb, b_col), fmt);
        /* steps 2 and 3: the naive triple loop */
#pragma omp parallel for schedule(dynamic, 1)
        for (int64_t r = 0; r < rows; ++r) {
            for (int64_t j = 0; j < N; ++j) {
                double c = 0.0, s = 0.0;
                for (int64_t k = 0; k < K; ++k) {
                    double p = a[r * K + k] * b[j * K + k];
                    c += p;
                    s += fabs(p);
                }
                int64_t o = (z * rows + r) * N + j;
                if (C) C[o] = c;
                if (S) S[o] = s;
            }
        }
    }
    free(a);
    free(b);
    return 0;
}

/*
 * Selected cells: for t in [0, npts) the cell (z[t], i[t], j[t]); results go to
 * C[t] and S[t] (either may be NULL).  Decodes on the fly, so it needs no
 * memory beyond its arguments and suits sampled checks on very large problems.
 */
void tsm_oracle_gemm_points(int64_t M, int64_t N, int64_t K, int fmt,
                            const uint16_t *A, int64_t lda, int64_t strideA, int a_col,
                            const uint16_t *B, int64_t ldb, int64_t strideB, int b_col,
                            int64_t npts, const int64_t *zi, const int64_t *ii, const int64_t *ji,
                            double *C, double *S) {
    (void)M;
    (void)N;
#pragma omp parallel for schedule(dynamic, 16)
    for (int64_t t = 0; t < npts; ++t) {
        const uint16_t *Az = A + zi[t] * strideA;
        const uint16_t *Bz = B + zi[t] * strideB;
        double c = 0.0, s = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = decode(element(Az, ii[t], k, lda, a_col), fmt) *
                       decode(element(Bz, k, ji[t], ldb, b_col), fmt);
            c += p;
            s += fabs(p);
        }
        if (C) C[t] = c;
        if (S) S[t] = s;
    }
}

/* Number of OpenMP threads a parallel region of this library would use. */
int tsm_oracle_threads(void) {
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Row sums -- the reduction of "A Dumb Triton Runtime Error" (section "The
 * kernel itself": one sum per row of a strided matrix, each element widened
 * before it is added):
 *
 *   out[r] = sum_{c=0..C-1} X[r*row_stride + c*col_stride], in float64, in
 *            increasing c;   S[r] = sum_c |X[r][c]| (NULL: not wanted).
 *
 * fmt: 0 = f16, 1 = bf16, 2 = float32.  A float32 pattern widens to float64
 * exactly (C's float -> double conversion).  Past-the-end columns do not exist
 * in this definition, so the additive-identity padding of a tiled kernel is
 * implicit.  Threads: OpenMP over rows; each row is one sequential sum.
 */
static double widen_f32(uint32_t bits) {
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

void tsm_oracle_rowsum(int64_t R, int64_t C, const void *X, int64_t row_stride, int64_t col_stride, int fmt,
                       double *out, double *S) {
    #pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < R; ++r) {
        double total = 0.0, magnitude = 0.0;
        for (int64_t c = 0; c < C; ++c) {
            const int64_t at = r * row_stride + c * col_stride;
            const double v = fmt == 2 ? widen_f32(((const uint32_t *)X)[at]) : decode(((const uint16_t *)X)[at], fmt);
            total += v;
            magnitude += fabs(v);
        }
        out[r] = total;
        if (S) S[r] = magnitude;
    }
}
