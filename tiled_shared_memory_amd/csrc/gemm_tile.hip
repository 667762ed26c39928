// Large-tile MFMA GEMM for gfx950: operands contiguous along K, full tiles.
//
// This is the fast path for A row-major and B column-major (every K slice of
// both operands is a set of contiguous 128-byte row pieces), M and N multiples
// of 256 and K a multiple of 64, all rows 16-byte aligned.  The host routes
// every other problem to the masked kernel.
//
// Blocking ("The PTSS Cliff", sections "The Idea: Stage in SLM, Tile K" and
// "Choosing K_TILE"): a 256-thread workgroup owns a 256 x 256 tile of C and
// walks K in slices of 64.  Each wave owns a 128 x 128 quadrant as 4 x 4
// blocks of v_mfma_f32_32x32x16, i.e. 256 float32 accumulators per lane, a
// budget fixed by the tile alone; the live operand fragments are one 16-deep
// step of one slice (32 registers).  K never enters the register budget.
//
// Staging: the two operand slices (2 x 32 KiB) go global -> LDS with
// buffer loads that write straight into LDS (no VGPR round trip), double buffered: while the
// matrix cores consume slice s, slice s+1 is in flight (128 KiB of the CU's
// 160 KiB LDS).  Each slice row is 128 bytes = 8 chunks of 16 bytes; chunk c of
// row r is stored at position c ^ (r % 8), so the 32 rows a fragment read
// touches spread over all banks.  One wave-wide load fills 8 whole rows (1 KiB),
// each lane fetching the global chunk that belongs at its LDS slot.
//
// Tile order: workgroups are dealt to the 8 XCDs round-robin, so consecutive
// tile indices are first regrouped per XCD, then ordered in groups of 8 tile
// rows, column by column (the grouped ordering of the Intel XPU Triton
// README's matmul signature, GROUP_SIZE_M), so the workgroups resident on one
// XCD share A and B panels in that XCD's L2.
//
// Epilogue: the operands are fed to the MFMA as (B, A), which makes the
// accumulator layout hold 4 consecutive columns of one row per register
// group, so each lane stores 8 bytes (f16) or 16 bytes (float32) at a time.
#include "gemm_internal.hpp"
#include "mfma.hpp"

namespace tsm {
namespace {

constexpr int BM = TileInfo::BM;
constexpr int BN = TileInfo::BN;
constexpr int BK = TileInfo::BK;
constexpr int THREADS = TileInfo::THREADS;
constexpr int ROW_BYTES = BK * 2;             // 128
constexpr int TILE_BYTES = BM * ROW_BYTES;    // 32 KiB per operand slice
constexpr int GROUP_M = 8;

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(1))) void global_void;

// Buffer resource over `bytes` bytes starting at `base` (raw addressing,
// dword 3 = the gfx9 default data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Per-lane byte offsets, relative to the slice origin, of the 8 chunks a lane
// fetches for one 256 x 64 operand slice (rows ld elements apart).  Lane l of
// wave w fills LDS slot l of 8-row groups w*8 .. w*8+7; the chunk that belongs
// at that slot under the XOR swizzle is chunk (l % 8) ^ (l / 8) of its row.
__device__ __forceinline__ void slice_offsets(uint32_t (&off)[8], int64_t ld, int wave, int lane) {
  const int r_in = lane >> 3;
  const int c = (lane & 7) ^ r_in;
#pragma unroll
  for (int g = 0; g < 8; ++g) off[g] = (uint32_t)(((wave * 8 + g) * 8 + r_in) * ld + c * 8) * 2u;
}

// Issue the asynchronous copy of one slice into LDS: 8 buffer loads per wave,
// each writing 1 KiB (8 rows) of LDS.  kbytes is the slice's K offset in bytes.
__device__ __forceinline__ void issue_slice(__amdgpu_buffer_rsrc_t rsrc, const uint32_t (&off)[8], uint32_t kbytes,
                                            char *lds, int wave) {
#pragma unroll
  for (int g = 0; g < 8; ++g)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)(lds + (wave * 8 + g) * 1024), 16, off[g], kbytes, 0,
                                             0);
}

// Fragments of one 16-deep step: 4 A blocks and 4 B blocks of 32 rows.
__device__ __forceinline__ void read_frags(const char *sa, const char *sb, u32x4 (&fa)[4], u32x4 (&fb)[4], int ks,
                                           int wm, int wn, int lane) {
  const int row = lane & 31;
  const int chunk = ((2 * ks + (lane >> 5)) ^ (lane & 7)) * 16;  // rows read here have row % 8 == lane % 8
#pragma unroll
  for (int i = 0; i < 4; ++i)
    fa[i] = *reinterpret_cast<const u32x4 *>(sa + (wm * 128 + i * 32 + row) * ROW_BYTES + chunk);
#pragma unroll
  for (int j = 0; j < 4; ++j)
    fb[j] = *reinterpret_cast<const u32x4 *>(sb + (wn * 128 + j * 32 + row) * ROW_BYTES + chunk);
}

// Scheduling hints (instruction classes of __builtin_amdgcn_sched_group_barrier).
constexpr int SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100;

// One 64-deep slice from LDS (sa, sb), while the next slice is fetched into the
// other stage: 4 steps of 16, each 8 fragment reads and 16 MFMAs.  The
// fragments of step ks+1 are read while the MFMAs of step ks run, and the 16
// buffer loads of the next slice are spread over the first step's MFMAs.
template <bool BF16, bool ISSUE>
__device__ __forceinline__ void slice(const char *sa, const char *sb, f32x16 (&acc)[4][4], int wm, int wn, int lane,
                                      __amdgpu_buffer_rsrc_t ra, __amdgpu_buffer_rsrc_t rb,
                                      const uint32_t (&offA)[8], const uint32_t (&offB)[8], uint32_t kbytes,
                                      char *na, char *nb, int wave) {
  u32x4 fa[2][4], fb[2][4];
  read_frags(sa, sb, fa[0], fb[0], 0, wm, wn, lane);
  if constexpr (ISSUE) {
    issue_slice(ra, offA, kbytes, na, wave);
    issue_slice(rb, offB, kbytes, nb, wave);
  }
#pragma unroll
  for (int ks = 0; ks < BK / 16; ++ks) {
    const int cur = ks & 1;
    if (ks + 1 < BK / 16) read_frags(sa, sb, fa[cur ^ 1], fb[cur ^ 1], ks + 1, wm, wn, lane);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = mfma_32x32x16<BF16>(fb[cur][j], fa[cur][i], acc[i][j]);
  }
  // schedule: step-0 reads first; then interleave MFMAs with the remaining reads and loads
  __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 8, 0);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
    if constexpr (ISSUE) __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 2, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
  }
  __builtin_amdgcn_sched_group_barrier(SG_MFMA, 8, 0);
#pragma unroll
  for (int ks = 1; ks < 3; ++ks) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      __builtin_amdgcn_sched_group_barrier(SG_MFMA, 1, 0);
      __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 8, 0);
  }
  __builtin_amdgcn_sched_group_barrier(SG_MFMA, 16, 0);
}

__device__ __forceinline__ void wait_slices() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

template <bool BF16, bool OUT_F16>
__global__ __launch_bounds__(THREADS, 1) void gemm_tile_kernel(KernelArgs p) {
  // separate arrays per stage so the compiler can tell the in-flight slice
  // from the one being read
  __shared__ __attribute__((aligned(1024))) char sA0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB0[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sA1[TILE_BYTES];
  __shared__ __attribute__((aligned(1024))) char sB1[TILE_BYTES];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 1, wn = wave & 1;

  // ---- tile order: per-XCD regrouping, then GROUP_M rows column by column
  const int T = p.tiles_m * p.tiles_n;
  int pid = blockIdx.x;
  if ((T & 7) == 0) pid = (pid & 7) * (T >> 3) + (pid >> 3);
  const int per_group = GROUP_M * p.tiles_n;
  const int group = pid / per_group;
  const int first_m = group * GROUP_M;
  const int gm = min(p.tiles_m - first_m, GROUP_M);
  const int in_group = pid - group * per_group;
  const int tm = first_m + in_group % gm;
  const int tn = in_group / gm;

  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t z = (int64_t)p.z0 + blockIdx.y;
  const uint16_t *A = p.A + z * p.sA + m0 * p.lda;  // row m0, k = 0 (row-major A)
  const uint16_t *B = p.B + z * p.sB + n0 * p.ldb;  // column n0, k = 0 (column-major B)

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x16{};

  // Buffer resources cover exactly the 256 rows of each operand panel; the
  // host keeps that extent below 4 GiB, so all offsets are 32-bit.
  const __amdgpu_buffer_rsrc_t ra = make_rsrc(A, (uint32_t)((255 * p.lda + p.K) * 2));
  const __amdgpu_buffer_rsrc_t rb = make_rsrc(B, (uint32_t)((255 * p.ldb + p.K) * 2));
  uint32_t offA[8], offB[8];
  slice_offsets(offA, p.lda, wave, lane);
  slice_offsets(offB, p.ldb, wave, lane);
  constexpr uint32_t SLICE = BK * 2;  // bytes between consecutive K slices of one row

  // The host guarantees K is a positive multiple of 128, so slices come in
  // pairs: the steady-state loop has no branches, which keeps the 256
  // accumulators of each lane in place across iterations.
  const int nk = (int)(p.K / BK);
  issue_slice(ra, offA, 0, sA0, wave);
  issue_slice(rb, offB, 0, sB0, wave);
  wait_slices();
  int kt = 0;
  for (; kt + 2 < nk; kt += 2) {
    // slice kt is in stage 0: multiply it while kt+1 loads into stage 1, then the reverse
    slice<BF16, true>(sA0, sB0, acc, wm, wn, lane, ra, rb, offA, offB, (kt + 1) * SLICE, sA1, sB1, wave);
    wait_slices();
    slice<BF16, true>(sA1, sB1, acc, wm, wn, lane, ra, rb, offA, offB, (kt + 2) * SLICE, sA0, sB0, wave);
    wait_slices();
  }
  // last pair: slices nk-2 (stage 0) and nk-1
  slice<BF16, true>(sA0, sB0, acc, wm, wn, lane, ra, rb, offA, offB, (kt + 1) * SLICE, sA1, sB1, wave);
  wait_slices();
  slice<BF16, false>(sA1, sB1, acc, wm, wn, lane, ra, rb, offA, offB, 0, sA0, sB0, wave);

  // ---- epilogue: lane holds C[m][n + 0..3] for m = block row + lane % 32
  const int64_t ldc = p.ldc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + wm * 128 + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int64_t n = n0 + wn * 128 + j * 32 + 8 * g + 4 * (lane >> 5);
        const f32x16 &a = acc[i][j];
        if constexpr (OUT_F16) {
          uint16_t *C = (uint16_t *)p.C + z * p.sC;
          u32x2 v;
          v[0] = (uint32_t)f32_to_f16_bits(a[4 * g + 0]) | ((uint32_t)f32_to_f16_bits(a[4 * g + 1]) << 16);
          v[1] = (uint32_t)f32_to_f16_bits(a[4 * g + 2]) | ((uint32_t)f32_to_f16_bits(a[4 * g + 3]) << 16);
          *reinterpret_cast<u32x2 *>(C + m * ldc + n) = v;
        } else {
          float *C = (float *)p.C + z * p.sC;
          f32x4 v = {a[4 * g + 0], a[4 * g + 1], a[4 * g + 2], a[4 * g + 3]};
          *reinterpret_cast<f32x4 *>(C + m * ldc + n) = v;
        }
      }
    }
  }
}

template <bool BF16, bool OUT_F16>
hipError_t launch_t(const KernelArgs &base, int64_t batch, hipStream_t stream) {
  const int64_t tiles = (int64_t)base.tiles_m * base.tiles_n;
  for (int64_t z0 = 0; z0 < batch; z0 += kMaxGridY) {
    KernelArgs a = base;
    a.z0 = (int32_t)z0;
    const int64_t nz = batch - z0 < kMaxGridY ? batch - z0 : kMaxGridY;
    hipLaunchKernelGGL((gemm_tile_kernel<BF16, OUT_F16>), dim3((unsigned)tiles, (unsigned)nz), dim3(THREADS), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

bool tile_supports(const Problem &p) {
  if (p.a_col || !p.b_col) return false;  // both operands must be K-contiguous
  if (p.M % BM || p.N % BN || p.K % (2 * BK) || p.K == 0) return false;
  // one operand panel (256 rows) must span less than 4 GiB: 32-bit buffer offsets
  if (255 * p.lda + p.K >= (int64_t)1 << 31 || 255 * p.ldb + p.K >= (int64_t)1 << 31) return false;
  if (((uintptr_t)p.A & 15) || ((uintptr_t)p.B & 15) || ((uintptr_t)p.C & 15)) return false;
  if (p.lda % 8 || p.ldb % 8) return false;
  if (p.ldc % (p.out_f16 ? 4 : 4)) return false;  // 8-byte (f16) / 16-byte (f32) row stores
  if (p.batch > 1 && (p.sA % 8 || p.sB % 8 || p.sC % 4)) return false;
  return true;
}

hipError_t launch_tile(const Problem &p, hipStream_t stream) {
  KernelArgs a{};
  a.A = p.A;
  a.B = p.B;
  a.C = p.C;
  a.M = p.M;
  a.N = p.N;
  a.K = p.K;
  a.lda = p.lda;
  a.ldb = p.ldb;
  a.ldc = p.ldc;
  a.sA = p.sA;
  a.sB = p.sB;
  a.sC = p.sC;
  a.tiles_m = (int32_t)(p.M / BM);
  a.tiles_n = (int32_t)(p.N / BN);
  if (p.in_bf16)
    return p.out_f16 ? launch_t<true, true>(a, p.batch, stream) : launch_t<true, false>(a, p.batch, stream);
  return p.out_f16 ? launch_t<false, true>(a, p.batch, stream) : launch_t<false, false>(a, p.batch, stream);
}

const char *tile_name() { return "tile_256x256x64_kk"; }

}  // namespace tsm
