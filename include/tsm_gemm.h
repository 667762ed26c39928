/*
 * tsm_gemm.h -- C ABI of the MI355X (gfx950) blocked GEMM library.
 *
 * The operation is the blocked matrix product C = A.B with 16-bit floating-point
 * operands (f16 or bf16), float32 accumulation and a float32 or f16 result.  It
 * is the computation of the 64x128x128 f16 example on "The PTSS Cliff: A Kernel
 * That Won't Build" (sections "The Arithmetic of 'Fully Unrolled K'" and "The
 * Idea: Stage in SLM, Tile K"): every output cell is sum_k A[i][k] * B[k][j],
 * computed by workgroups that each own an output tile and walk K in bounded
 * slices staged through on-chip shared memory (LDS on gfx950).  The masked
 * K-blocked loop with a float32 accumulator and zero padding outside the matrix
 * is the one of the Intel XPU Triton README, section "Use Tensor Descriptors to
 * load tl.dot arguments and save results".
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 *  - Sizes, leading dimensions and batch strides are counted in ELEMENTS, and
 *    are 64-bit ("A Dumb Triton Runtime Error", Step 1: strides in elements;
 *    Intel XPU Triton README, "Avoid int32 Overflow": offsets are formed in
 *    64 bits).
 *  - A is logically M x K, B is K x N, C is M x N.
 *      row-major A: A[i*lda + k], lda >= K      column-major A: A[k*lda + i], lda >= M
 *      row-major B: B[k*ldb + j], ldb >= N      column-major B: B[j*ldb + k], ldb >= K
 *      C is always row-major:  C[i*ldc + j], ldc >= N
 *  - C is OVERWRITTEN with A.B (no accumulate, no atomics): "A Dumb Triton
 *    Runtime Error", section "Making It Compile, and Why I'd Still Use the
 *    Original", shows read-modify-write into an output that was not zeroed
 *    giving wrong rows.  Elements of C outside the M x N region (the ld padding)
 *    are never written.  K = 0 with M, N > 0 writes zeros (the empty sum).
 *  - Operand elements outside M, N or K never contribute: tiles are loaded
 *    with zero padding ("A Dumb Triton Runtime Error", Step 2, on masking with
 *    the additive identity).
 *  - Pointers are device pointers owned by the caller (e.g. torch tensors).  The
 *    library allocates nothing, keeps no mutable global state and never
 *    synchronises: it enqueues kernels on `stream` (a hipStream_t; NULL = the
 *    null stream) and returns.  Results are valid once the stream reaches them.
 *  - Any 2-byte-aligned operand base and any leading dimension is accepted;
 *    the vector width of the loads is chosen inside the library.  C must be
 *    4-byte aligned for float32 output and 2-byte aligned for f16 output.
 *  - Errors: every argument check runs on the host before any HIP call; on an
 *    error nothing is enqueued and a status code is returned.  No C++ exception
 *    crosses this boundary.  tsm_last_error_detail() names the failed check.
 *
 * Status codes and enums are plain ints so that any FFI can call in.
 */
#ifndef TSM_GEMM_H
#define TSM_GEMM_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define TSM_SUCCESS 0
#define TSM_ERROR_INVALID_VALUE 1 /* an argument breaks the contract above      */
#define TSM_ERROR_NOT_SUPPORTED 2 /* valid, but beyond this library's limits     */
#define TSM_ERROR_LAUNCH 3        /* the HIP runtime refused or failed a launch */

/* dtype: operand format and output format.  Accumulation is always float32;
 * a 16-bit output is rounded to nearest even from the float32 result. */
#define TSM_F16_F32 0
#define TSM_F16_F16 1
#define TSM_BF16_F32 2
#define TSM_BF16_F16 3
#define TSM_F16_BF16 4
#define TSM_BF16_BF16 5

/* Epilogue activation of gemm_strided_batched_act, applied to the float32
 * result before the output conversion. */
#define TSM_ACT_NONE 0
#define TSM_ACT_RELU 1       /* x > 0 ? x : 0          */
#define TSM_ACT_LEAKY_RELU 2 /* x > 0 ? x : slope * x  */

/* Storage layout of an operand. */
#define TSM_ROW 0
#define TSM_COL 1

/*
 * gemm -- C := A.B for row-major A (M x K) and row-major B (K x N): the product
 * of "The PTSS Cliff", section "The Arithmetic of 'Fully Unrolled K'" (each
 * output cell the sum over k of A[i][k] * B[k][j]), with the K-tiled, LDS-staged
 * blocking of its section "The Idea: Stage in SLM, Tile K".
 *   M, N, K   : sizes, >= 0.
 *   A, lda    : operand A and its leading dimension (>= max(1, K)).
 *   B, ldb    : operand B and its leading dimension (>= max(1, N)).
 *   C, ldc    : result, leading dimension >= max(1, N).
 *   dtype     : operand -> output format: TSM_F16_F32, TSM_F16_F16, TSM_BF16_F32,
 *               TSM_BF16_F16, TSM_F16_BF16 or TSM_BF16_BF16.
 *   stream    : hipStream_t to enqueue on (NULL = null stream).
 * Returns a status code.  M = 0 or N = 0 succeeds without launching.
 * Errors (TSM_ERROR_INVALID_VALUE): negative size; NULL pointer with work to do;
 * leading dimension below the row length; unknown dtype; misaligned pointer;
 * C overlapping A or B.  TSM_ERROR_NOT_SUPPORTED: sizes whose tile grid or
 * element offsets exceed the launch limits (reported, never truncated).
 */
int gemm(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb, void *C,
         int64_t ldc, int dtype, void *stream);

/*
 * gemm_ex -- gemm with an explicit storage layout per operand
 * (layout_a, layout_b in {TSM_ROW, TSM_COL}); gemm is gemm_ex(TSM_ROW, TSM_ROW).
 * The Intel XPU Triton README's matmul signature ("Use Proper Type
 * Annotations") takes a row and a column stride per operand, so either storage
 * order of A and B is the same product; here the two orders that keep one
 * dimension contiguous are offered.
 * A column-major B (element (k, j) at B[j*ldb + k], ldb >= K) makes both operands
 * contiguous along K, the layout the square bf16 product uses.
 */
int gemm_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a, const void *B,
            int64_t ldb, int layout_b, void *C, int64_t ldc, int dtype, void *stream);

/*
 * gemm_strided_batched -- batch independent products, problem z using
 *   A + z*strideA, B + z*strideB, C + z*strideC   (strides in elements, 64-bit).
 * The per-problem slices follow the batched indexing of the Intel XPU Triton
 * README (section "Use Tensor Descriptors to load tl.dot arguments and save
 * results", one expert's slice of a 3-D operand per program); the offsets are
 * formed in 64 bits, as its section "Avoid int32 Overflow" requires once a
 * stride product passes 2^31 (the 8-problem skinny workload's B spans 2^31
 * bytes).
 * strideA or strideB may be 0 (the operand is shared by every problem).
 * strideC must keep the outputs disjoint: strideC >= (M-1)*ldc + N when batch > 1.
 * batch = 0 succeeds without launching.  Other rules as for gemm.
 */
int gemm_strided_batched(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int64_t strideA,
                         const void *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc, int64_t strideC,
                         int64_t batch, int dtype, void *stream);

/* gemm_strided_batched_ex -- gemm_strided_batched with per-operand layouts
 * (as gemm_ex: the README's per-operand strides, restricted to row- or
 * column-major storage).
 * Row bands: one problem (batch 1) of more than one round of 256 x 256 tiles
 * (a round: one tile per CU) whose last round is partly empty may run as two
 * launches on the stream, one after the other: the rows that fill whole rounds
 * on the 256 x 256 kernel, the remaining rows as a problem of their own on the
 * kernel chosen for that problem.  Each element of C is computed by one of the
 * two.  This applies to every plain entry point (gemm to
 * gemm_strided_batched_act, and gemm_strided_batched_ws and _noalloc when they
 * do not split). */
int gemm_strided_batched_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a,
                            int64_t strideA, const void *B, int64_t ldb, int layout_b, int64_t strideB, void *C,
                            int64_t ldc, int64_t strideC, int64_t batch, int dtype, void *stream);

/*
 * gemm_grouped -- `groups` independent products of different heights: problem g
 * uses the first m_g rows of A + g*strideA and C + g*strideC, and B + g*strideB,
 *     C_g[0:m_g, :] := A_g[0:m_g, :] . B_g,
 * where m_g = min(max(rows[g], 0), M).  This is the mixture-of-experts slice of
 * the Intel XPU Triton README (section "Use Tensor Descriptors to load tl.dot
 * arguments and save results", its A[expert, :tokens, :] example): each
 * expert's token count is read from device memory by the kernels, workgroups
 * whose tile starts at or past m_g exit early, and rows past m_g are masked.
 *   M         : the largest row count a problem may have (the row capacity of
 *               every A_g and C_g); sizes and strides are validated against it.
 *   rows      : DEVICE pointer to `groups` int32 counts, 4-byte aligned, read in
 *               stream order (a kernel earlier on `stream` may produce them).
 *               Values outside [0, M] are clamped, never an error: the host
 *               cannot see them.  Must be non-NULL when M, N and groups are > 0.
 *   Rows m_g .. M-1 of every C_g are not written.  Other arguments and rules as
 *   for gemm_strided_batched_ex (groups plays the role of batch).
 */
int gemm_grouped(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a, int64_t strideA,
                 const void *B, int64_t ldb, int layout_b, int64_t strideB, void *C, int64_t ldc, int64_t strideC,
                 const int32_t *rows, int64_t groups, int dtype, void *stream);

/* Element format of a row-sum input.  Sums are always float32. */
#define TSM_ROWSUM_F32 0
#define TSM_ROWSUM_F16 1
#define TSM_ROWSUM_BF16 2

/*
 * rowsum -- out[r] := sum_c X[r*row_stride + c*col_stride], r < R, c < C.
 * The tiled row-sum kernel of "A Dumb Triton Runtime Error" (sections "The
 * kernel itself" through "Step 3: Cross-Lane Tree Reduction (tl.sum) and Scalar
 * Store"): each element is converted to float32 and added into lane-local
 * float32 accumulators, tiles past the row end contribute 0, and one
 * cross-lane reduction per row is followed by one plain store.
 *   R, C        : rows and columns, >= 0.  C = 0 writes zeros.
 *   X           : device pointer, aligned to its element size (TSM_ROWSUM_*).
 *   row_stride,
 *   col_stride  : element strides, >= 0 (any view: transposed, sliced).
 *   out         : device float32 array of R sums, 4-byte aligned, OVERWRITTEN
 *                 (its previous contents never matter: "Making It Compile, and
 *                 Why I'd Still Use the Original").  Must not overlap X.
 * Accuracy: |out[r] - exact| <= C * 2^-24 * sum_c |X[r][c]|.  The reduction
 * order is fixed, so results are bitwise reproducible.
 * Errors and stream semantics as for gemm.
 */
int rowsum(int64_t R, int64_t C, const void *X, int64_t row_stride, int64_t col_stride, int xdtype, float *out,
           void *stream);

/* tsm_rowsum_kernel_name -- the kernel a rowsum call would launch, or NULL. */
const char *tsm_rowsum_kernel_name(int64_t R, int64_t C, const void *X, int64_t row_stride, int64_t col_stride,
                                   int xdtype, const float *out);

/*
 * gemm_strided_batched_act -- gemm_strided_batched_ex with an elementwise
 * activation fused into the epilogue: C := act(A.B), act applied to each
 * float32 result before it is converted and stored.  The ACTIVATION
 * meta-parameter of the Intel XPU Triton README's matmul signature ("Use
 * Proper Type Annotations") names such a fused activation; the pages do not
 * say which, so the plainest piecewise-linear ones are offered.
 *   activation: TSM_ACT_NONE, TSM_ACT_RELU or TSM_ACT_LEAKY_RELU.
 *   slope     : the factor leaky ReLU applies to negative values (finite);
 *               ignored otherwise.
 * Other arguments and rules as for gemm_strided_batched_ex.
 */
int gemm_strided_batched_act(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a,
                             int64_t strideA, const void *B, int64_t ldb, int layout_b, int64_t strideB, void *C,
                             int64_t ldc, int64_t strideC, int64_t batch, int dtype, int activation, float slope,
                             void *stream);

/*
 * gemm_workspace_bytes -- bytes of workspace with which gemm_strided_batched_ws
 * splits K for a problem of this shape: batch * S * M * N * 4 for S chunks of
 * K (the largest S the operands' layouts may lead to), or for the hybrid
 * r * s * 256 * 256 * 4 (see gemm_strided_batched_ws), or 0 when the shape
 * does not split (its output tiles already occupy the chip, K is below 512 or
 * not a multiple of 64, or N is not a multiple of 64 or 8).  With stream-K
 * requested (TSM_GEMM_SPLIT=streamk in the environment), also its need when
 * larger: 2 * R * 256 * 256 * 4 bytes for R runs (R = the CU count of the
 * current device, at most 256: 128 MiB).  Depends on the sizes (and then the
 * CU count) only.  Negative sizes give 0.
 */
int64_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t batch);

/*
 * gemm_strided_batched_ws -- gemm_strided_batched_act that may split K through
 * a caller's workspace, for products with few output tiles and deep K (e.g.
 * 256 x 256 x 8192, sixteen 64 x 64 tiles for 256 CUs).  The two-pass,
 * deterministic form of the split: pass 1 gives each workgroup one output tile
 * and one K chunk of 512 or more and stores its float32 partial sums into the
 * workspace; pass 2 adds the chunks of every output element in a fixed order,
 * applies the activation and the output conversion, and stores C once.  No
 * atomics, no zeroed memory: the store-once rule of "A Dumb Triton Runtime
 * Error" (section "The Takeaway and the Final Fix") holds across the split.
 *   workspace       : device memory owned by the caller, 16-byte aligned, not
 *                     overlapping A, B or C; its contents on entry do not
 *                     matter and on return are unspecified.  May be NULL
 *                     (with workspace_bytes = 0): the call then never splits.
 *   workspace_bytes : its size.  Below gemm_workspace_bytes(M, N, K, batch),
 *                     or for operands the split passes cannot read, the call
 *                     runs exactly as gemm_strided_batched_act.  The split
 *                     needs 16-byte aligned bases and rows (lda, ldb multiples
 *                     of 8, ldc of 4) and no grouped counts.  The streaming
 *                     kernel's split (up to 512 rows) needs row-major A, B
 *                     either way; the 256 x 256 tiles' split (above 128 rows,
 *                     one problem) takes any layout.
 * One problem of more than 256 tiles of 256 x 256 whose last round of 256 tiles
 * is at most half full (more than 128 rows, K a multiple of 128 from 2048 up)
 * takes the hybrid: the whole rounds run unsplit, and each of the r leftover
 * tiles is cut into s equal chunks of K (s r <= 256), whose float32 partial
 * tiles go to the workspace (r s * 256 * 256 * 4 bytes, at most 64 MiB) and
 * are added in K order before C is stored once.  Where row bands (see
 * gemm_strided_batched_ex) also apply, the hybrid is taken only for K above
 * 4096 with more than 64 rows past the whole rounds; TSM_GEMM_SPLIT=hybrid in
 * the environment takes it wherever it applies.
 * With TSM_GEMM_SPLIT=streamk in the environment, stream-K (the work-centric
 * decomposition of Osama et al., PPoPP 2023) replaces the tile split for 32
 * to 224 tiles of 256 x 256 (one problem or a strided batch, more than 128
 * rows, K a multiple of 128 from 2048 up): R workgroups, one per CU, take
 * equal runs of 128-deep slices of the tiles in order; every run meets at
 * most two tiles and stores a float32 partial tile for each into the
 * workspace, and a second kernel adds each tile's partials in K order and
 * stores C once.  The result is the same on every call on devices with the
 * same CU count.  It is not the default: on MI355X it is slower than the
 * plain kernel or the tile split for these shapes.  TSM_GEMM_SPLIT=none
 * keeps the kernel that needs no workspace.
 * Two calls in flight at once must not share a workspace.  Other arguments,
 * rules and errors as for gemm_strided_batched_act; additionally
 * TSM_ERROR_INVALID_VALUE for negative workspace_bytes, a NULL workspace with
 * workspace_bytes > 0, a misaligned workspace or one overlapping an operand.
 */
int gemm_strided_batched_ws(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a,
                            int64_t strideA, const void *B, int64_t ldb, int layout_b, int64_t strideB, void *C,
                            int64_t ldc, int64_t strideC, int64_t batch, int dtype, int activation, float slope,
                            void *workspace, int64_t workspace_bytes, void *stream);

/*
 * gemm_strided_batched_noalloc -- gemm_strided_batched_ws for callers that
 * cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid allocation): the K split's partial sums go to a
 * static scratch array of gemm_noalloc_scratch_bytes() (64 MiB) that the
 * library holds on each GPU from its load until the process ends.  The call
 * allocates nothing.  It splits K exactly when gemm_strided_batched_ws would
 * with a workspace of gemm_workspace_bytes(M, N, K, batch) bytes; shapes that
 * do not split run as gemm_strided_batched_act.
 * Calls on one GPU share its scratch: calls that overlap on one GPU (other
 * streams, other host threads) race and must not be issued.  The scratch
 * needs no clearing (every partial read back was written by the same call).
 * Arguments and errors as for gemm_strided_batched_act; additionally
 * TSM_ERROR_NOT_SUPPORTED when the split would need more than the scratch
 * holds (the detail names the size; use gemm_strided_batched_ws then), and
 * TSM_ERROR_LAUNCH when the scratch's device address cannot be obtained.
 */
int gemm_strided_batched_noalloc(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a,
                                 int64_t strideA, const void *B, int64_t ldb, int layout_b, int64_t strideB, void *C,
                                 int64_t ldc, int64_t strideC, int64_t batch, int dtype, int activation, float slope,
                                 void *stream);

/* Bytes of the static scratch gemm_strided_batched_noalloc splits K through. */
int64_t gemm_noalloc_scratch_bytes(void);

/* Static text for a status code ("success", "invalid value", ...). */
const char *tsm_status_string(int status);

/* Text naming the check that made the calling thread's last call fail
 * (thread-local; empty after a successful call). */
const char *tsm_last_error_detail(void);

/*
 * tsm_gemm_kernel_name -- name of the kernel variant a gemm_strided_batched_ex
 * call with these arguments would launch (same arguments, no stream), or NULL
 * if the call would be rejected or launch nothing.  Pure host logic: it
 * validates and selects, it never touches the GPU.  The returned string is
 * static.
 */
const char *tsm_gemm_kernel_name(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a,
                                 int64_t strideA, const void *B, int64_t ldb, int layout_b, int64_t strideB,
                                 void *C, int64_t ldc, int64_t strideC, int64_t batch, int dtype);

/* tsm_gemm_ws_kernel_name -- the same for a gemm_strided_batched_ws call (a
 * split names its pass-1 kernel followed by "+reduce"). */
const char *tsm_gemm_ws_kernel_name(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a,
                                    int64_t strideA, const void *B, int64_t ldb, int layout_b, int64_t strideB,
                                    void *C, int64_t ldc, int64_t strideC, int64_t batch, int dtype,
                                    const void *workspace, int64_t workspace_bytes);

/* tsm_gemm_grouped_kernel_name -- the same for a gemm_grouped call. */
const char *tsm_gemm_grouped_kernel_name(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a,
                                         int64_t strideA, const void *B, int64_t ldb, int layout_b, int64_t strideB,
                                         void *C, int64_t ldc, int64_t strideC, const int32_t *rows, int64_t groups,
                                         int dtype);

#ifdef __cplusplus
}
#endif

#endif /* TSM_GEMM_H */
