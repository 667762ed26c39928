// Large-tile MFMA GEMM for gfx950: operands contiguous along K, full tiles.
//
// This is the fast path for A row-major and B column-major (every K slice of
// both operands is a set of contiguous 64-byte row pieces), M and N multiples
// of 256 and K a multiple of 128, all rows 16-byte aligned.  The host routes
// every other problem to the masked kernel.
//
// Blocking ("The PTSS Cliff", sections "The Idea: Stage in SLM, Tile K" and
// "Choosing K_TILE"): a 256-thread workgroup owns a 256 x 256 tile of C and
// walks K in slices of 32.  Each wave owns a 128 x 128 quadrant as 4 x 4
// blocks of v_mfma_f32_32x32x16, i.e. 256 float32 accumulators per lane, a
// budget fixed by the tile alone; the live operand fragments are two 16-deep
// steps (64 registers).  K never enters the register budget.
//
// Staging: operand slices (2 x 16 KiB) go global -> LDS with buffer loads that
// write straight into LDS (no VGPR round trip), through a ring of 4 stages
// (128 KiB of the CU's 160 KiB): a slice is requested three slices before it
// is multiplied, which covers HBM latency at full MFMA rate.  Each slice row
// is 64 bytes = 4 chunks of 16 bytes, XOR-swizzled per row (see swz) so that
// fragment reads are free of bank conflicts.  One wave-wide load fills
// 16 whole rows (1 KiB), each lane fetching the global chunk that belongs at
// its LDS slot.
//
// Per slice: wait for the slice and a workgroup barrier, read the first
// step's fragments, refill the freed stage, run the previous slice's last
// step (deferred so it covers the fragment-read latency), read the second
// step's fragments, run the first step.
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
constexpr int BK = TileInfo::BK;              // 32
constexpr int NS = TileInfo::STAGES;          // 4
constexpr int ROW_BYTES = BK * 2;             // 64: 4 chunks of 16 bytes
constexpr int TILE_BYTES = BM * ROW_BYTES;    // 16 KiB per operand slice
constexpr int GROUP_M = 8;

typedef __attribute__((address_space(3))) void lds_void;

// The LDS ring: one array per stage and operand, so that the compiler can tell
// the slice in flight from the one being read.
__shared__ __attribute__((aligned(1024))) char g_a0[TILE_BYTES], g_b0[TILE_BYTES];
__shared__ __attribute__((aligned(1024))) char g_a1[TILE_BYTES], g_b1[TILE_BYTES];
__shared__ __attribute__((aligned(1024))) char g_a2[TILE_BYTES], g_b2[TILE_BYTES];
__shared__ __attribute__((aligned(1024))) char g_a3[TILE_BYTES], g_b3[TILE_BYTES];

template <int S> struct Ring;
template <> struct Ring<0> {
  __device__ static char *a() { return g_a0; }
  __device__ static char *b() { return g_b0; }
};
template <> struct Ring<1> {
  __device__ static char *a() { return g_a1; }
  __device__ static char *b() { return g_b1; }
};
template <> struct Ring<2> {
  __device__ static char *a() { return g_a2; }
  __device__ static char *b() { return g_b2; }
};
template <> struct Ring<3> {
  __device__ static char *a() { return g_a3; }
  __device__ static char *b() { return g_b3; }
};

// Buffer resource over `bytes` bytes starting at `base` (raw addressing,
// dword 3 = the gfx9 default data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// LDS position of 16-byte chunk c of slice row r: chunk c ^ (3 * bit 3 of r).
// gfx950 serves a 64-lane 16-byte read in two halves of 32 lanes (lanes 0-15
// with 32-47, then 16-31 with 48-63) across 512 bytes of banks; with 64-byte
// rows, rows r and r + 8 share a bank window, and this XOR sends their chunks
// to complementary positions, so both fragment shapes (32 rows x 2 chunks,
// 16 rows x 2 chunks per half) read without bank conflicts.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (((r >> 3) & 1) * 3); }

// Per-lane byte offsets, relative to the slice origin, of the chunks a lane
// fetches for one 256 x 32 operand slice (rows ld elements apart).  One
// wave-wide load fills 16 whole rows (1 KiB): lane l writes LDS slot l, i.e.
// row l / 4 of its group at position l % 4, so it fetches the chunk whose
// swizzled position that is.
template <int LOADS>
__device__ __forceinline__ void slice_offsets(uint32_t (&off)[LOADS], int64_t ld, int wave, int lane) {
  const int r_in = lane >> 2;
  const int c = swz(r_in, lane & 3);  // swz is an involution in its chunk argument
#pragma unroll
  for (int g = 0; g < LOADS; ++g) off[g] = (uint32_t)(((wave * LOADS + g) * 16 + r_in) * ld + c * 8) * 2u;
}

// Asynchronous copy of one operand slice into LDS: 16 buffer loads shared by
// the waves, each writing 1 KiB of LDS; kbytes is the slice's K offset in bytes.
template <int LOADS>
__device__ __forceinline__ void issue(__amdgpu_buffer_rsrc_t rsrc, const uint32_t *off, uint32_t kbytes, char *lds,
                                      int wave) {
#pragma unroll
  for (int g = 0; g < LOADS; ++g)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_void *)(lds + (wave * LOADS + g) * 1024), 16, off[g],
                                             kbytes, 0, 0);
}

// Fragments of one whole 32-deep slice for one wave (128 x 128 of C):
//  MI = 32: two 16-deep steps, each 4 A and 4 B blocks of 32 rows
//           (v_mfma_f32_32x32x16 operands);
//  MI = 16: one 32-deep step, 8 A and 8 B blocks of 16 rows
//           (v_mfma_f32_16x16x32 operands).
// Either way 16 reads of 16 bytes per lane, 64 registers.
template <int MI>
struct Frags {
  static constexpr int NA = MI == 32 ? 4 : 8;  // blocks per operand per step
  static constexpr int NSTEP = MI == 32 ? 2 : 1;
  u32x4 a[NSTEP][NA], b[NSTEP][NA];
};

template <int MI>
__device__ __forceinline__ void read_frags(const char *sa, const char *sb, Frags<MI> &f, int wm, int wn, int lane) {
  constexpr int NA = Frags<MI>::NA;
  // lane reads row (lane % MI) of each block, K chunk (lane / MI) of the step;
  // block rows are multiples of 16, so the swizzle sees row % 16 == lane % 16
  const int row = lane % MI;
#pragma unroll
  for (int s = 0; s < Frags<MI>::NSTEP; ++s) {
    const int chunk = swz(lane, s * (4 / Frags<MI>::NSTEP) + lane / MI) * 16;
#pragma unroll
    for (int i = 0; i < NA; ++i)
      f.a[s][i] = *reinterpret_cast<const u32x4 *>(sa + (wm * 128 + i * MI + row) * ROW_BYTES + chunk);
#pragma unroll
    for (int j = 0; j < NA; ++j)
      f.b[s][j] = *reinterpret_cast<const u32x4 *>(sb + (wn * 128 + j * MI + row) * ROW_BYTES + chunk);
  }
}

// Accumulators of one wave: 128 x 128 float32 = 256 registers per lane.
template <int MI>
struct Acc;
template <>
struct Acc<32> {
  f32x16 v[4][4];
};
template <>
struct Acc<16> {
  f32x4 v[8][8];
};

// All MFMAs of one slice.  Operands go in as (B, A) so that each accumulator
// register group holds 4 consecutive columns of one row of C.
template <bool BF16, int MI>
__device__ __forceinline__ void mma(const Frags<MI> &f, Acc<MI> &acc) {
  constexpr int NA = Frags<MI>::NA;
#pragma unroll
  for (int s = 0; s < Frags<MI>::NSTEP; ++s)
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int j = 0; j < NA; ++j) {
        if constexpr (MI == 32)
          acc.v[i][j] = mfma_32x32x16<BF16>(f.b[s][j], f.a[s][i], acc.v[i][j]);
        else
          acc.v[i][j] = mfma_16x16x32<BF16>(f.b[s][j], f.a[s][i], acc.v[i][j]);
      }
}

// Scheduling classes of __builtin_amdgcn_sched_group_barrier.
constexpr int SG_MFMA = 0x008, SG_VMEM_READ = 0x020, SG_DS_READ = 0x100;
constexpr int LOADS = 4;  // 1 KiB wave-loads per operand slice per wave

struct Ctx {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t offA[LOADS], offB[LOADS];
  int nk, wave, wm, wn, lane;
};

// Slice j, resident in stage S: after its barrier, read all of its fragments
// into one register set while the MFMAs of slice j-1 run from the other set,
// and refill the stage that slice j-1 freed with slice j+3.
template <bool BF16, int MI, int S>
__device__ __forceinline__ void slice(Ctx &c, int j, Frags<MI> (&fr)[2], Acc<MI> &acc) {
  // Keep every MFMA of the previous slice above this point: sinking them past
  // the fragment reads below would need a third fragment register set.
  __builtin_amdgcn_sched_barrier(0);
  // Slice j has landed once at most the two younger slices' loads are pending;
  // this wave's reads of stage S-1 (refilled below) are complete.  The empty
  // asm keeps LDS reads from moving above the barrier.
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(2 * 2 * LOADS) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  read_frags<MI>(Ring<S>::a(), Ring<S>::b(), fr[S & 1], c.wm, c.wn, c.lane);
  // the last slice again near the end keeps the load count per slice uniform
  const int next = min(j + NS - 1, c.nk - 1);
  issue<LOADS>(c.ra, c.offA, (uint32_t)next * ROW_BYTES, Ring<(S + NS - 1) % NS>::a(), c.wave);
  issue<LOADS>(c.rb, c.offB, (uint32_t)next * ROW_BYTES, Ring<(S + NS - 1) % NS>::b(), c.wave);
  mma<BF16, MI>(fr[(S & 1) ^ 1], acc);  // slice j-1
  // schedule: one fragment read or load after every other MFMA, spread over
  // the whole slice (bursts of memory instructions stall the in-order wave
  // and with it the MFMA pipe)
  constexpr int NMFMA = MI == 32 ? 32 : 64;
  constexpr int G = NMFMA / 8;  // MFMAs per group of 2 reads + 1 load
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, G / 4, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, G / 4, 0);
    __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, G / 4, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, G / 4, 0);
  }
}

template <bool BF16, bool OUT_F16, int MI>
__global__ __launch_bounds__(256, 1) void gemm_tile_kernel(KernelArgs p) {
  Ctx c;
  const int tid = threadIdx.x;
  c.lane = tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  c.wm = c.wave >> 1;  // 2 x 2 waves of 128 x 128
  c.wn = c.wave & 1;
  const int lane = c.lane, wm = c.wm, wn = c.wn;

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

  Acc<MI> acc;
  if constexpr (MI == 32) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc.v[i][j] = f32x16{};
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) acc.v[i][j] = f32x4{};
  }

  // Buffer resources cover exactly the 256 rows of each operand panel; the
  // host keeps that extent below 1 GiB, so all offsets are 32-bit.
  c.ra = make_rsrc(A, (uint32_t)((255 * p.lda + p.K) * 2));
  c.rb = make_rsrc(B, (uint32_t)((255 * p.ldb + p.K) * 2));
  slice_offsets<LOADS>(c.offA, p.lda, c.wave, lane);
  slice_offsets<LOADS>(c.offB, p.ldb, c.wave, lane);
  c.nk = (int)(p.K / BK);  // the host guarantees K is a positive multiple of NS * BK

  // prologue: slices 0 .. NS-2 in flight
  issue<LOADS>(c.ra, c.offA, 0 * ROW_BYTES, Ring<0>::a(), c.wave);
  issue<LOADS>(c.rb, c.offB, 0 * ROW_BYTES, Ring<0>::b(), c.wave);
  issue<LOADS>(c.ra, c.offA, 1 * ROW_BYTES, Ring<1>::a(), c.wave);
  issue<LOADS>(c.rb, c.offB, 1 * ROW_BYTES, Ring<1>::b(), c.wave);
  issue<LOADS>(c.ra, c.offA, 2 * ROW_BYTES, Ring<2>::a(), c.wave);
  issue<LOADS>(c.rb, c.offB, 2 * ROW_BYTES, Ring<2>::b(), c.wave);

  // Before slice 0 there is no previous slice: zero fragments add exactly 0.
  Frags<MI> fr[2];
#pragma unroll
  for (int s = 0; s < Frags<MI>::NSTEP; ++s)
#pragma unroll
    for (int i = 0; i < Frags<MI>::NA; ++i) fr[1].a[s][i] = fr[1].b[s][i] = u32x4{0, 0, 0, 0};

  // The steady-state loop has no data-dependent branches, which keeps the
  // 256 accumulators of each lane in place across iterations.
  for (int j = 0; j < c.nk; j += NS) {
    slice<BF16, MI, 0>(c, j + 0, fr, acc);
    slice<BF16, MI, 1>(c, j + 1, fr, acc);
    slice<BF16, MI, 2>(c, j + 2, fr, acc);
    slice<BF16, MI, 3>(c, j + 3, fr, acc);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  mma<BF16, MI>(fr[1], acc);  // the last slice (nk is a multiple of 4, so it sits in set 1)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the duplicate tail loads

  // ---- epilogue: each register group holds C[m][n + 0..3]
  const int64_t ldc = p.ldc;
#pragma unroll
  for (int i = 0; i < 128 / MI; ++i) {
    const int64_t m = m0 + wm * 128 + i * MI + (lane % MI);
#pragma unroll
    for (int j = 0; j < 128 / MI; ++j) {
#pragma unroll
      for (int g = 0; g < (MI == 32 ? 4 : 1); ++g) {
        // 32x32: group g covers columns 8g + 4*(lane/32) .. +3; 16x16: 4*(lane/16) .. +3
        const int64_t n = n0 + wn * 128 + j * MI + (MI == 32 ? 8 * g + 4 * (lane >> 5) : 4 * (lane >> 4));
        float v0, v1, v2, v3;
        if constexpr (MI == 32) {
          v0 = acc.v[i][j][4 * g + 0];
          v1 = acc.v[i][j][4 * g + 1];
          v2 = acc.v[i][j][4 * g + 2];
          v3 = acc.v[i][j][4 * g + 3];
        } else {
          v0 = acc.v[i][j][0];
          v1 = acc.v[i][j][1];
          v2 = acc.v[i][j][2];
          v3 = acc.v[i][j][3];
        }
        if constexpr (OUT_F16) {
          uint16_t *C = (uint16_t *)p.C + z * p.sC;
          u32x2 v;
          v[0] = (uint32_t)f32_to_f16_bits(v0) | ((uint32_t)f32_to_f16_bits(v1) << 16);
          v[1] = (uint32_t)f32_to_f16_bits(v2) | ((uint32_t)f32_to_f16_bits(v3) << 16);
          *reinterpret_cast<u32x2 *>(C + m * ldc + n) = v;
        } else {
          float *C = (float *)p.C + z * p.sC;
          *reinterpret_cast<f32x4 *>(C + m * ldc + n) = f32x4{v0, v1, v2, v3};
        }
      }
    }
  }
}

template <bool BF16, bool OUT_F16, int MI>
hipError_t launch_t(const KernelArgs &base, int64_t batch, hipStream_t stream) {
  const int64_t tiles = (int64_t)base.tiles_m * base.tiles_n;
  for (int64_t z0 = 0; z0 < batch; z0 += kMaxGridY) {
    KernelArgs a = base;
    a.z0 = (int32_t)z0;
    const int64_t nz = batch - z0 < kMaxGridY ? batch - z0 : kMaxGridY;
    hipLaunchKernelGGL((gemm_tile_kernel<BF16, OUT_F16, MI>), dim3((unsigned)tiles, (unsigned)nz), dim3(256), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int MI>
hipError_t launch_mi(const Problem &p, const KernelArgs &a, hipStream_t stream) {
  if (p.in_bf16)
    return p.out_f16 ? launch_t<true, true, MI>(a, p.batch, stream) : launch_t<true, false, MI>(a, p.batch, stream);
  return p.out_f16 ? launch_t<false, true, MI>(a, p.batch, stream) : launch_t<false, false, MI>(a, p.batch, stream);
}

}  // namespace

bool tile_supports(const Problem &p) {
  if (p.a_col || !p.b_col) return false;  // both operands must be K-contiguous
  if (p.M % BM || p.N % BN || p.K % (NS * BK) || p.K == 0) return false;
  // one operand panel (256 rows) must span less than 2 GiB: 32-bit buffer offsets
  if (255 * p.lda + p.K >= (int64_t)1 << 30 || 255 * p.ldb + p.K >= (int64_t)1 << 30) return false;
  if (((uintptr_t)p.A & 15) || ((uintptr_t)p.B & 15) || ((uintptr_t)p.C & 15)) return false;
  if (p.lda % 8 || p.ldb % 8) return false;
  if (p.ldc % 4) return false;  // 8-byte (f16) / 16-byte (float32) row stores
  if (p.batch > 1 && (p.sA % 8 || p.sB % 8 || p.sC % 4)) return false;
  return true;
}

hipError_t launch_tile(const Problem &p, int mi, hipStream_t stream) {
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
  return mi == 16 ? launch_mi<16>(p, a, stream) : launch_mi<32>(p, a, stream);
}

const char *tile_name(int mi) { return mi == 16 ? "tile_256x256x32_mi16" : "tile_256x256x32_mi32"; }

}  // namespace tsm
