// Internal interface between the host dispatch (gemm_api.hip) and the kernel
// translation units.  Nothing here is part of the public C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tsm {

// One (possibly batched) product, already validated by the host code.
struct Problem {
  const uint16_t *A;
  const uint16_t *B;
  void *C;
  int64_t M, N, K;
  int64_t lda, ldb, ldc;
  int64_t sA, sB, sC;  // batch strides, elements
  int64_t batch;
  bool a_col;    // A stored column-major (M-contiguous) instead of row-major (K-contiguous)
  bool b_col;    // B stored column-major (K-contiguous) instead of row-major (N-contiguous)
  bool in_bf16;  // operands are bf16 (else f16)
  bool out16;     // C is 16-bit (else float32)
  bool out_bf16;  // the 16-bit output format is bf16 (else f16)
  int act;        // epilogue activation: 0 none, 1 ReLU, 2 leaky ReLU
  float slope;    // leaky ReLU slope
  const int32_t *rows;  // grouped products: device array of per-problem row counts (else null)
  int skinny_w;         // skinny kernel: workgroup width forced (64 or 256), or 0 to choose by the grid
};

// Kernel arguments, passed by value.  Offsets are 64-bit throughout.
struct KernelArgs {
  const uint16_t *A;
  const uint16_t *B;
  void *C;
  int64_t M, N, K;
  int64_t lda, ldb, ldc;
  int64_t sA, sB, sC;
  int32_t tiles_m, tiles_n;
  int32_t z0;  // first problem index covered by this launch
  const int32_t *rows;  // per-problem row counts in device memory, or null (every problem has M rows)
  int32_t compact_groups;  // large-tile kernel, grouped call: number of groups, tiles numbered over valid ones only
  int32_t flat_batch;      // large-tile and masked kernels, strided batch: number of problems, tiles numbered over all of them
  int32_t act;             // epilogue: 0 none, 1 ReLU, 2 leaky ReLU
  float slope;             // leaky ReLU slope
  int32_t out_bf16;        // 16-bit output is bf16 (else f16)
  // skinny kernel, K-split pass: grid.y enumerates (problem, row block, K chunk);
  // 0 splits means a plain launch
  int32_t splits, row_blocks;
  int64_t kchunk;  // K depth of every chunk but the last (a multiple of 64)
  // large-tile kernel, stream-K: the partial slots (2 per workgroup, 256 x 256 float32 each)
  float *sk_ws;
  // large-tile kernel, one problem, a range of its tiles in the grouped tile order: tiles
  // tile0 .. tile0 + tile_count - 1 (tile_count 0: all of them)
  int32_t tile0, tile_count;
  // stream-K with runs aligned to whole chunks of one tile (the hybrid's remainder): one
  // partial slot per run instead of two
  int32_t sk_aligned;
};

// Rows of problem z: M, or for a grouped product the caller's count for z
// clamped to [0, M].  Uniform across the workgroup (a scalar load).
__device__ __forceinline__ int64_t rows_of(const KernelArgs &p, int64_t z) {
  if (!p.rows) return p.M;
  const int64_t r = p.rows[z];
  return r < 0 ? 0 : (r > p.M ? p.M : r);
}

// The 8 XCDs take workgroups round-robin; re-deal index b of T so that each
// XCD gets a contiguous run of tiles (the last T % 8 keep their index).
__device__ __forceinline__ int xcd_remap(int b, int T) {
  const int T8 = T & ~7;
  return b < T8 ? (b & 7) * (T8 >> 3) + (b >> 3) : b;
}

// Tile (tm, tn) of run index pid over a tiles_m x tiles_n grid: groups of
// group_m tile rows, walked column by column (the grouped ordering of the
// Intel XPU Triton README's matmul signature, GROUP_SIZE_M), so consecutive
// tiles share A and B panels.
__device__ __forceinline__ void tile_order(int pid, int tiles_m, int tiles_n, int group_m, int &tm, int &tn) {
  const int per_group = group_m * tiles_n;
  const int group = pid / per_group;
  const int first_m = group * group_m;
  const int gm = min(tiles_m - first_m, group_m);
  const int in_group = pid - group * per_group;
  tm = first_m + in_group % gm;
  tn = in_group / gm;
}

// Largest grid.y a launch uses for the batch; bigger batches are split.
constexpr int64_t kMaxGridY = 65535;

// ---- kernel families -------------------------------------------------------
// Masked, register-staged LDS kernel: any layout, any alignment, ragged edges.
// vec = 8 needs 16-byte aligned rows along the contiguous dimension of both
// operands; vec = 1 accepts anything 2-byte aligned.
struct MaskedInfo {
  static constexpr int BM = 128, BN = 128, THREADS = 256;  // K slices of 32 (64 on 64 x 64 tiles)
  // largest leading dimension (elements, exclusive): a slice spans at most
  // 127 of them plus under 80 elements, below 2^31 bytes (bit 31 of a load's offset
  // marks an element outside the matrix)
  static constexpr int64_t kMaxLd = (int64_t)1 << 23;
};
// vec: 8 (16-byte aligned vectors) or 0 (realigned vectors at any 2-byte
// alignment); tile: 128 (128 x 128) or 64 (64 x 64, for problems with few 128-tiles).
hipError_t launch_masked(const Problem &p, int vec, int tile, hipStream_t stream);
const char *masked_name(int vec, int tile);

// Large-tile kernel: A row-major, B either layout, N a multiple of 8, K a
// multiple of 128, 16-byte aligned rows; any M (rows past M or N, or past a
// grouped problem's count, read as zero and are not stored).
// Variants (K slab depth, MFMA shape, A and B layouts): 0 = 32-deep, 32x32x16,
// column-major B; 1 = 32-deep, 16x16x32, column-major B; 2 = 32-deep,
// 16x16x32, row-major B (transposed out of LDS); 3, 4 = as 1, 2 with 64-deep
// slabs; 5, 6 = as 2, 1 with column-major A (also transposed out of LDS).
struct TileInfo {
  static constexpr int BM = 256, BN = 256, BK = 32, STAGES = 4;
};
bool tile_supports(const Problem &p, bool a_col, bool b_row);

// Skinny kernel: M <= 128 (in 1, 2, 4 or 8 blocks of 16 rows), row-major A,
// B either way, N a multiple of the workgroup width (256 columns when that
// grid fills the chip, else 64), K a multiple of 64, 16-byte aligned rows.
struct SkinnyInfo {
  static constexpr int BK = 64;
};
struct SkinnyPlan {
  int mb = 0;  // 16-row blocks (0: the kernel cannot run the problem)
  int w = 0;   // columns per workgroup
};
SkinnyPlan skinny_plan(const Problem &p);
// slices in one round of the kernel's LDS ring (it always runs whole rounds)
int skinny_ring_slices(const SkinnyPlan &pl);
bool skinny_supports(const Problem &p);

// K split through a caller's workspace, for problems whose tiles cannot fill
// the chip: pass 1 runs the skinny kernel (64 or 256 columns per workgroup,
// row blocks of 16 * mb rows) on each K chunk and writes float32 partial sums,
// one M x N slab per (problem, chunk); pass 2 adds the slabs in chunk order
// and applies the epilogue.
struct KSplit {
  int splits = 0;  // K chunks (0: no split)
  int64_t kchunk = 0;
  int mb = 0, row_blocks = 0;
  int w = 64;  // columns per pass-1 workgroup (64 or 256)
  int tile_variant = -1;  // >= 0: pass 1 is that 256 x 256 kernel (a batch of the K chunks), not the skinny one
  int sk_runs = 0;        // > 0: stream-K instead, tile_variant over this many runs (splits is then 2)
  // > 0: the hybrid instead: this many whole rounds of tiles data-parallel on dp_variant, the
  // remaining tiles in `splits` chunks of K on tile_variant (stream-K runs of one chunk each)
  int dp_tiles = 0, dp_variant = -1;
};
// Depends on the shape (and, through `wide`, on whether B is row-major);
// workspace bytes = batch * splits * M * N * 4.
KSplit ksplit_shape(int64_t M, int64_t N, int64_t K, int64_t batch, bool wide);
// The shape's split, if the operands' layouts and alignment allow it.
KSplit ksplit_plan(const Problem &p);
hipError_t launch_ksplit(const Problem &p, const KSplit &ks, float *ws, hipStream_t stream);
hipError_t launch_ksplit_pass1(const Problem &p, const KSplit &ks, float *ws, hipStream_t stream);
// The 256 x 256 kernels' split, for single products of 8-127 such tiles:
// pass 1 runs the K chunks as a strided batch of products into the workspace.
KSplit tsplit_shape(int64_t M, int64_t N, int64_t K, int64_t batch);
KSplit tsplit_plan(const Problem &p);
// Stream-K over the 256 x 256 kernels, for single products and strided
// batches of 256 x 256 tiles that leave part of the chip idle; `cus` is the
// device's CU count.  Workspace bytes = sk_workspace_bytes(sk_runs).
KSplit sk_shape(int64_t M, int64_t N, int64_t K, int64_t batch, int cus);
KSplit sk_plan(const Problem &p, int cus);
// The hybrid for one problem a little over whole rounds of 256 x 256 tiles.
// Workspace bytes = hybrid_workspace_bytes(ks).
KSplit hybrid_shape(int64_t M, int64_t N, int64_t K, int64_t batch, int cus);
KSplit hybrid_plan(const Problem &p, int cus, int dp_variant);
inline int64_t hybrid_workspace_bytes(const KSplit &ks) { return (int64_t)ks.sk_runs * TileInfo::BM * TileInfo::BN * 4; }
const char *ksplit_name(const KSplit &ks, bool b_col);

// Split-K kernel for small M x N and deep K: 16 x 16 tiles, K split across the
// 16 waves of a workgroup; row-major A, B either way, M, N multiples of 16, K
// a multiple of 2048.
struct SplitKInfo {
  static constexpr int WAVES = 16;
};
bool splitk_supports(const Problem &p);
hipError_t launch_splitk(const Problem &p, hipStream_t stream);
const char *splitk_name(bool b_col);
hipError_t launch_skinny(const Problem &p, hipStream_t stream);
const char *skinny_name(const Problem &p);
hipError_t launch_tile(const Problem &p, int variant, hipStream_t stream);
// Stream-K over P workgroups (variants 1, 2, 5 and 6), then the fix-up of the
// tiles that several workgroups share; ws holds 2 P partial tiles
// (sk_workspace_bytes).
hipError_t launch_tile_sk(const Problem &p, int variant, float *ws, int P, hipStream_t stream);
// One problem of more than one round of tiles: the first `dp_tiles` tiles (whole
// rounds) on the data-parallel kernel `variant`, and the remaining ones split
// `splits` ways in K as aligned stream-K runs on `sk_variant` (2, 5, 6 or 8; one run per chunk,
// one 256 x 256 float32 partial slot per run: (tiles - dp_tiles) * splits * 256 KiB
// of workspace), then their fix-up.
hipError_t launch_tile_hybrid(const Problem &p, int variant, int sk_variant, int dp_tiles, int splits, float *ws,
                              hipStream_t stream);
inline int64_t sk_workspace_bytes(int P) { return (int64_t)P * 2 * TileInfo::BM * TileInfo::BN * 4; }
const char *tile_name(int variant);

// ---- row sums ----------------------------------------------------------------
// out[r] = sum_c X[r*row_stride + c*col_stride], float32 accumulation.
struct RowsumInfo {
  enum { F32 = 0, F16 = 1, BF16 = 2 };  // element format of X
};
struct RowsumArgs {
  const void *X;
  float *out;
  int64_t R, C;
  int64_t r0;  // first row of this launch (launches cover at most kRowsPerLaunch rows)
  int64_t row_stride, col_stride;  // elements
  int fmt;
};
struct RowsumPlan {
  bool vec;    // 16-byte loads (contiguous, 16-byte aligned rows)
  bool block;  // one workgroup per row (few long rows), else one wave per row
};
RowsumPlan rowsum_plan(const RowsumArgs &a);
hipError_t launch_rowsum(const RowsumArgs &a, hipStream_t stream);
const char *rowsum_name(const RowsumArgs &a);

}  // namespace tsm
