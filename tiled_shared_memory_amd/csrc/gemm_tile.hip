// Large-tile MFMA GEMM for gfx950.
//
// The fast path for K a multiple of 128, N a multiple of 8 and 16-byte
// aligned rows, in every layout pair (A row- or column-major, B either way),
// for problems whose 256 x 256 tiles fill most of the chip.  M and N need not
// be multiples of 256: rows and columns past them load as zero and are not
// stored (and a grouped call's rows past each problem's count likewise).  The
// host sends everything else to the masked kernel.
//
// Blocking ("The PTSS Cliff", sections "The Idea: Stage in SLM, Tile K" and
// "Choosing K_TILE"): a 256-thread workgroup owns a 256 x 256 tile of C and
// walks K in slabs.  Each wave owns a 128 x 128 quadrant, i.e. 256 float32
// accumulators per lane (8 x 8 blocks of v_mfma_f32_16x16x32, or 4 x 4 of
// v_mfma_f32_32x32x16), a budget fixed by the tile alone; the live operand
// fragments are two 32-deep sub-slices (128 registers).  K never enters the
// register budget.
//
// Staging: operand slabs go global -> LDS with buffer loads that write
// straight into LDS (no VGPR round trip); one wave-wide load fills 1 KiB of
// LDS, each lane fetching the global chunk that belongs at its LDS slot.  Rows
// are XOR-swizzled in 16-byte chunks (see swz, swz_row) so that fragment reads
// are free of bank conflicts.  Three ring shapes:
//  * 32-deep slices, 4 stages: a slice is requested three slices before it is
//    multiplied.  K-contiguous rows are 64 bytes.
//  * 64-deep slabs, 2 stages: a slab is requested one slab (two 32-deep
//    sub-slices) before use.  K-contiguous rows are 128 bytes, so every L2
//    request carries a whole 128-byte line: half the requests of 64-byte rows
//    for the same bytes, which is what limits the 32-deep ring on K-contiguous
//    operands.
//  * 64-deep slabs with staggered refills (the default for K-contiguous A and
//    B): A on 3 stages, B on 2 (the whole 160 KiB); each half of a slab issues
//    half of the copies (see substep_st).
// Row-major B slices are 256 columns wide (512-byte rows); the B operand is
// transposed on its way out of LDS by ds_read_b64_tr_b16.
//
// Per 32-deep sub-slice: (at a slab boundary) wait for the slab and a
// workgroup barrier, then refill the freed stage; read the sub-slice's
// fragments into one register set while the previous sub-slice's MFMAs run
// from the other, reads and loads interleaved with the MFMAs.
//
// Tile order: workgroups are dealt to the 8 XCDs round-robin, so consecutive
// tile indices are first regrouped per XCD, then ordered in groups of 8 tile
// rows (4 from 32 tile rows up), column by column (the grouped ordering of the
// Intel XPU Triton README's matmul signature, GROUP_SIZE_M), so the workgroups
// resident on one XCD share A and B panels in that XCD's L2.
//
// K ranges: the tile body (tile_run) takes any K range that is a multiple of
// 128, so the same kernels also run stream-K (equal runs of 128-deep units
// over the tiles, float32 partial tiles, then sk_reduce_kernel's fixed-order
// fix-up) and the hybrid (whole rounds of tiles data-parallel, the last
// round's tiles in equal chunks of K).
//
// Epilogue: the operands are fed to the MFMA as (B, A), which makes the
// accumulator layout hold 4 consecutive columns of one row per register
// group, so each lane stores 8 bytes (f16) or 16 bytes (float32) at a time,
// through a buffer resource over the tile's valid part of C (no per-row
// branches, one 32-bit lane offset per column block).
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

// Tile rows per group of the tile order: 4 from 32 tile rows up (8192 x 8192
// x 8192: 0.764 ms against 0.778 with 8, and 0.795 with 2), else 8 (4096^3:
// 0.110 ms against 0.112 with 4).
__device__ __forceinline__ int group_rows(int tiles_m) { return tiles_m >= 32 ? 4 : GROUP_M; }
constexpr int64_t kMaxCompactGroups = 256;  // groups whose counts every workgroup scans

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// The LDS ring: one array per stage and operand, so that the compiler can tell
// the slice in flight from the one being read.
__shared__ __attribute__((aligned(1024))) char g_a0[TILE_BYTES], g_b0[TILE_BYTES];
__shared__ __attribute__((aligned(1024))) char g_a1[TILE_BYTES], g_b1[TILE_BYTES];
__shared__ __attribute__((aligned(1024))) char g_a2[TILE_BYTES], g_b2[TILE_BYTES];
__shared__ __attribute__((aligned(1024))) char g_a3[TILE_BYTES], g_b3[TILE_BYTES];

// Wide variant: 64-deep slabs (128-byte rows, 32 KiB per operand), 2 stages.
constexpr int WROW_BYTES = 128;
constexpr int WTILE_BYTES = BM * WROW_BYTES;
__shared__ __attribute__((aligned(1024))) char w_a0[WTILE_BYTES], w_b0[WTILE_BYTES];
__shared__ __attribute__((aligned(1024))) char w_a1[WTILE_BYTES], w_b1[WTILE_BYTES];

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

// A third 64-deep A stage: with it the A slabs ride a 3-stage ring (160 KiB of
// LDS with the two B stages), see substep_st.
__shared__ __attribute__((aligned(1024))) char w_a2[WTILE_BYTES];
__device__ __forceinline__ char *wa3(int s) { return s == 0 ? w_a0 : s == 1 ? w_a1 : w_a2; }

template <int S> struct WRing;
template <> struct WRing<0> {
  __device__ static char *a() { return w_a0; }
  __device__ static char *b() { return w_b0; }
};
template <> struct WRing<1> {
  __device__ static char *a() { return w_a1; }
  __device__ static char *b() { return w_b1; }
};

// A per-lane offset past every buffer resource (which the host keeps below
// 1 GiB): such a load returns zeros.  Slice offsets added to it stay below 2^32.
constexpr uint32_t kOutside = 0x80000000u;

// Buffer resource over `bytes` bytes starting at `base` (raw addressing,
// dword 3 = the gfx9 default data format).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// LDS position of 16-byte chunk c of row r of a K-contiguous slab, KB = slab
// depth / 32.  The fragment reads take rows (lane % 16) + 16i at chunk
// 4U + lane / 16 (16x16x32 operands).  Both swizzles were chosen by measuring
// the LDS bank-conflict counter on that read pattern, over every swizzle of
// the form c ^ (XOR-linear function of row bits 0..3) and random ones: with
// these, the reads are conflict-free (4 LDS cycles per 64-lane 16-byte read);
// unswizzled rows cost 2x (64-byte rows) and 4x (128-byte rows).
//  KB = 1 (64-byte rows): c ^ (3 * bit 3 of r).
//  KB = 2 (128-byte rows): c ^ ((r / 2) % 8).
template <int KB>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (KB == 1) {
    return c ^ (((r >> 3) & 1) * 3);
  } else {
    return c ^ ((r >> 1) & 7);
  }
}

// Row-major B: a slice is 32 rows of k, 256 columns (512 bytes); position of
// 16-byte chunk c (0..31) of row r.  One transpose read covers rows
// {0..3, 8..11, 16..19, 24..27} + 4h and a 32-byte column block; the XOR
// sends those 16 rows to 16 distinct even offsets (32 distinct positions).
__device__ __forceinline__ int swz_row(int r, int c) { return c ^ (2 * ((r & 3) | ((r >> 1) & 12))); }

// Per-lane byte offsets of the chunks a lane fetches for one row-major B
// slice: wave-load g of wave w fills rows 2*(w*LOADS+g) + lane/32, position
// lane % 32, i.e. the chunk whose swizzled position that is.  A chunk's
// columns are the same in every slice, so chunks at or past the panel's
// `vcols` valid columns get an offset beyond the buffer resource: they load
// as zero (and never touch memory past the matrix).
template <int LOADS>
__device__ __forceinline__ void slice_offsets_row(uint32_t (&off)[LOADS], int64_t ld, int wave, int lane, int vcols) {
#pragma unroll
  for (int g = 0; g < LOADS; ++g) {
    const int r = 2 * (wave * LOADS + g) + (lane >> 5);
    const int c = swz_row(r, lane & 31);
    off[g] = c * 8 < vcols ? (uint32_t)(r * ld + c * 8) * 2u : kOutside;
  }
}

// Per-lane byte offsets, relative to the slab origin, of the chunks a lane
// fetches for one 256 x 32KB K-contiguous operand slab (rows ld elements
// apart).  One wave-wide load fills 1 KiB = 16 / KB whole rows: lane l writes
// LDS slot l, i.e. row l / (4 KB) of its group at position l % (4 KB), so it
// fetches the chunk whose swizzled position that is (swz is an involution in
// its chunk argument).
template <int LOADS, int KB>
__device__ __forceinline__ void slice_offsets(uint32_t (&off)[LOADS], int64_t ld, int wave, int lane) {
  constexpr int CPR = 4 * KB;  // chunks per row
#pragma unroll
  for (int g = 0; g < LOADS; ++g) {
    const int r = (wave * LOADS + g) * (64 / CPR) + lane / CPR;
    off[g] = (uint32_t)(r * ld + swz<KB>(r, lane % CPR) * 8) * 2u;
  }
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

// A 16x16x32 operand from a slice stored k-row by k-row (512-byte rows of
// 256 columns, swizzled by swz_row): lane needs X[8*(lane/16) .. +7][column
// col0 + lane % 16]; two ds_read_b64_tr_b16, each 4 rows deep (in each 16-lane
// group, lane j points at row 4h + j/4 of the group's 8 rows, columns
// 4*(j%4) .. +3).  Sub-slice U of the slab is a constant offset of 32 rows.
template <int U>
__device__ __forceinline__ u32x4 read_tr_operand(const char *s, int col0, int lane) {
  u32x4 f;
  const int col = col0 + 4 * (lane & 3);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int r = 8 * (lane >> 4) + 4 * h + ((lane & 15) >> 2);
    const int off = (32 * U + r) * 512 + swz_row(r, col >> 3) * 16 + (col & 7) * 2;
    const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)((lds_char *)s + off));
    const u32x2 d = __builtin_bit_cast(u32x2, v);
    f[2 * h] = d[0];
    f[2 * h + 1] = d[1];
  }
  return f;
}

// Fragments of sub-slice U (k = 32U .. 32U + 31) of a slab of depth 32 KB.
// ACOL: A is column-major (its slices are k rows of 256 m); BROW: B is
// row-major (k rows of 256 n).  Both are transposed on the way out of LDS.
template <int MI, bool ACOL, bool BROW, int KB, int U>
__device__ __forceinline__ void read_frags(const char *sa, const char *sb, Frags<MI> &f, int wm, int wn, int lane) {
  constexpr int NA = Frags<MI>::NA;
  constexpr int RB = 64 * KB;  // bytes per K-contiguous row
  static_assert(!BROW || MI == 16, "row-major B is read with 16x16x32 operands");
  static_assert(!ACOL || MI == 16, "column-major A is read with 16x16x32 operands");
  static_assert(KB == 1 || MI == 16, "64-deep slabs are read with 16x16x32 operands");
  // lane reads row (lane % MI) of each block, K chunk (lane / MI) of the step;
  // block rows are multiples of 16, so the swizzle sees row % 16 == lane % 16
  const int row = lane % MI;
#pragma unroll
  for (int s = 0; s < Frags<MI>::NSTEP; ++s) {
    const int chunk = swz<KB>(lane, 4 * U + s * (4 / Frags<MI>::NSTEP) + lane / MI) * 16;
    if constexpr (!ACOL) {
#pragma unroll
      for (int i = 0; i < NA; ++i)
        f.a[s][i] = *reinterpret_cast<const u32x4 *>(sa + (wm * 128 + i * MI + row) * RB + chunk);
    } else {
#pragma unroll
      for (int i = 0; i < NA; ++i) f.a[s][i] = read_tr_operand<U>(sa, wm * 128 + i * 16, lane);
    }
    if constexpr (!BROW) {
#pragma unroll
      for (int j = 0; j < NA; ++j)
        f.b[s][j] = *reinterpret_cast<const u32x4 *>(sb + (wn * 128 + j * MI + row) * RB + chunk);
    } else {
      // B operand of 16x16x32 from row-major B: column lane % 16 of its block
#pragma unroll
      for (int j = 0; j < NA; ++j) f.b[s][j] = read_tr_operand<U>(sb, wn * 128 + j * 16, lane);
    }
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
constexpr int LOADS = 4;  // 1 KiB wave-loads per operand slice per wave (8 per 64-deep slab)

template <int L>
struct CtxT {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t offA[L], offB[L];
  uint32_t kstepA;  // bytes between consecutive slabs of A (row bytes if K-contiguous, 32 KB rows if column-major)
  uint32_t kstepB;  // bytes between consecutive slabs of B (row bytes if K-contiguous, 32 KB rows if row-major)
  int nk, wave, wm, wn, lane;
};
using Ctx = CtxT<LOADS>;
using CtxW = CtxT<2 * LOADS>;

// Slice j, resident in stage S: after its barrier, read all of its fragments
// into one register set while the MFMAs of slice j-1 run from the other set,
// and refill the stage that slice j-1 freed with slice j+3.
template <bool BF16, int MI, bool ACOL, bool BROW, int S>
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
  read_frags<MI, ACOL, BROW, 1, 0>(Ring<S>::a(), Ring<S>::b(), fr[S & 1], c.wm, c.wn, c.lane);
  // the last slice again near the end keeps the load count per slice uniform
  const int next = min(j + NS - 1, c.nk - 1);
  issue<LOADS>(c.ra, c.offA, (uint32_t)next * c.kstepA, Ring<(S + NS - 1) % NS>::a(), c.wave);
  issue<LOADS>(c.rb, c.offB, (uint32_t)next * c.kstepB, Ring<(S + NS - 1) % NS>::b(), c.wave);
  mma<BF16, MI>(fr[(S & 1) ^ 1], acc);  // slice j-1
  // schedule: one fragment read or load after every other MFMA, spread over
  // the whole slice (bursts of memory instructions stall the in-order wave
  // and with it the MFMA pipe)
  constexpr int NMFMA = MI == 32 ? 32 : 64;
  constexpr int G = NMFMA / 8;          // MFMAs per group of reads + 1 load
  // reads per group: (16 or 8) A reads + (16 or 8) B reads over 8 groups
  constexpr int R = ((ACOL ? 16 : 8) + (BROW ? 16 : 8)) / 8;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, G / 4, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, R - R / 2, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, G / 4, 0);
    __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, G / 4, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, R / 2, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, G / 4, 0);
  }
}

// Tile-rows of 256 that hold rows of problem g of a grouped call.
__device__ __forceinline__ int work_rows(const KernelArgs &p, int g) { return (int)((rows_of(p, g) + BM - 1) / BM); }

// Wide variant, sub-slice U of slab j (resident in stage S): U = 0 waits for
// the slab and the barrier, reads sub-slice 0's fragments and refills the
// other stage (freed by that barrier) with slab j+1 while the previous
// sub-slice's MFMAs run; U = 1 only reads and multiplies.  A slab is thus
// requested one slab (two sub-slices) before it is used.
template <bool BF16, bool ACOL, bool BROW, int S, int U>
__device__ __forceinline__ void substep_w(CtxW &c, int j, Frags<16> (&fr)[2], Acc<16> &acc) {
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (U == 0) {
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  read_frags<16, ACOL, BROW, 2, U>(WRing<S>::a(), WRing<S>::b(), fr[U], c.wm, c.wn, c.lane);
  if constexpr (U == 0) {
    // the last slab again at the end keeps the load count per slab uniform
    const int next = min(j + 1, c.nk - 1);
    issue<2 * LOADS>(c.ra, c.offA, (uint32_t)next * c.kstepA, WRing<S ^ 1>::a(), c.wave);
    issue<2 * LOADS>(c.rb, c.offB, (uint32_t)next * c.kstepB, WRing<S ^ 1>::b(), c.wave);
  }
  mma<BF16, 16>(fr[U ^ 1], acc);  // the previous sub-slice
  constexpr int R = ((ACOL ? 16 : 8) + (BROW ? 16 : 8)) / 8;  // fragment reads per group of 8 MFMAs
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 2, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, R - R / 2, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 2, 0);
    if constexpr (U == 0) __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 2, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, R / 2, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 2, 0);
    if constexpr (U == 0) __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
  }
}

// Staggered refills (K-contiguous A and B, 64-deep slabs): A on a 3-stage
// ring, B on a 2-stage one.  Sub-slice U of slab j (A in stage SA = j % 3, B
// in stage SB = j % 2): U = 0 waits for slab j (only the A copies of slab j+1
// may still be in flight), passes the barrier and refills the B stage freed by
// slab j-1 with B's slab j+1; U = 1 refills the A stage freed by slab j-1 with
// A's slab j+2.  Each half of a slab thus issues half of the copies (32
// wave-loads per CU, where the two-stage ring issues all 64 in the first
// half), and A's copies are requested two slabs ahead.
// The first MFMAs of a tile: from a zero accumulator operand (an inline
// constant), so the accumulators need no zeroing.
template <bool BF16>
__device__ __forceinline__ void mma_init(const Frags<16> &f, Acc<16> &acc) {
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc.v[i][j] = mfma_16x16x32<BF16>(f.b[0][j], f.a[0][i], f32x4{});
}
// MODE 1: the tile's first sub-slice, which has no previous one to multiply;
// MODE 2: the second, whose multiply starts the accumulators.
template <bool BF16, int SA, int SB, int U, int MODE = 0>
__device__ __forceinline__ void substep_st(CtxW &c, int j, Frags<16> (&fr)[2], Acc<16> &acc) {
  __builtin_amdgcn_sched_barrier(0);
  if constexpr (U == 0) {
    asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(2 * LOADS) : "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  }
  read_frags<16, false, false, 2, U>(wa3(SA), WRing<SB>::b(), fr[U], c.wm, c.wn, c.lane);
  if constexpr (U == 0) {
    const int next = min(j + 1, c.nk - 1);  // the last slab again at the end keeps the copy count uniform
    issue<2 * LOADS>(c.rb, c.offB, (uint32_t)next * c.kstepB, WRing<SB ^ 1>::b(), c.wave);
  } else {
    const int next = min(j + 2, c.nk - 1);
    issue<2 * LOADS>(c.ra, c.offA, (uint32_t)next * c.kstepA, wa3((SA + 2) % 3), c.wave);
  }
  if constexpr (MODE == 0) mma<BF16, 16>(fr[U ^ 1], acc);  // the previous sub-slice
  else if constexpr (MODE == 2) mma_init<BF16>(fr[U ^ 1], acc);
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 2, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 2, 0);
    __builtin_amdgcn_sched_group_barrier(SG_VMEM_READ, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 2, 0);
    __builtin_amdgcn_sched_group_barrier(SG_DS_READ, 1, 0);
    __builtin_amdgcn_sched_group_barrier(SG_MFMA, 2, 0);
  }
}

// Slab 0 (A and B in stage 0): the peeled first trip of the ring.
template <bool BF16>
__device__ __forceinline__ void slab_first(CtxW &c, Frags<16> (&fr)[2], Acc<16> &acc) {
  substep_st<BF16, 0, 0, 0, 1>(c, 0, fr, acc);
  substep_st<BF16, 0, 0, 1, 2>(c, 0, fr, acc);
}
template <bool BF16, int J>
__device__ __forceinline__ void slab_st(CtxW &c, int j, Frags<16> (&fr)[2], Acc<16> &acc) {
  substep_st<BF16, J % 3, J % 2, 0>(c, j, fr, acc);
  substep_st<BF16, J % 3, J % 2, 1>(c, j, fr, acc);
}

// ---- Staged 16-bit epilogue.  Each wave converts its 128 x 128 quadrant into
// LDS (128 rows of 256 bytes, free once every wave is past its last fragment
// read), then stores it back 4 rows x 256 bytes per instruction: 16 B per lane,
// whole 128-byte lines, non-temporal.  A store straight from the 16 x 16
// accumulator layout touches 16 rows of C, 32 bytes each: on the 8192^3
// product that cost 64 L1 accesses per store instruction (TCP accesses
// 1.53e8 per call against 1.38e8 now) and serialized address translations
// (TCP_UTCL1_SERIALIZATION_STALL 1.0e7 cycles, now 0), and the call took 2.4%
// longer.
//
// The 16-byte chunk c of quadrant row r sits at chunk c ^ (r % 16), so that
// the 8-byte writes of 16 rows at one column group spread over the banks and
// each 256-byte row is read back whole by 16 lanes (the epilogue's LDS bank
// conflicts come to 1.5% of the kernel's LDS cycles).

// Wave w's staging area: a 64-deep ring's 32 KiB stage (w_a0, w_a1, w_b0 and
// w_b1 exist in both such rings), or for the 32-deep ring two 16 KiB stages,
// A stage w for quadrant rows 0..63 and B stage w for rows 64..127.
template <int KB>
__device__ __forceinline__ char *stage_lo(int wave) {
  if constexpr (KB == 1) return wave == 0 ? g_a0 : wave == 1 ? g_a1 : wave == 2 ? g_a2 : g_a3;
  return wave == 0 ? w_a0 : wave == 1 ? w_a1 : wave == 2 ? w_b0 : w_b1;
}
template <int KB>
__device__ __forceinline__ char *stage_hi(int wave) {
  if constexpr (KB == 1) return (wave == 0 ? g_b0 : wave == 1 ? g_b1 : wave == 2 ? g_b2 : g_b3) - 64 * 256;
  return stage_lo<KB>(wave);
}

// Two values of C as a 32-bit pair of f16 (FMT = 0) or bf16 (FMT = 1), each
// rounded to nearest even by the hardware's packed conversion.
template <int FMT>
__device__ __forceinline__ uint32_t pack16(float a, float b) {
  typedef float f2 __attribute__((ext_vector_type(2)));
  if constexpr (FMT == 0) {
    typedef _Float16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, h2));
  } else {
    typedef __bf16 h2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f2{a, b}, h2));
  }
}

// Cache-policy bit "nt" of a buffer store (non-temporal: C is written once
// and not read again by the kernel).  With whole-line stores it shortened the
// 8192^3 product by 1.8% (0.724 against 0.738 ms, one box, interleaved); the
// write-back policies sc0 / sc1 changed nothing.
constexpr int kNonTemporal = 2;

// One tile's product over k0 .. k0+kd (a multiple of 128): the whole K for
// a data-parallel tile, one stream-K segment otherwise.  PART = false: the
// sums go through the epilogue into C; PART = true: raw into the 256 x 256
// float32 partial at `part`.
template <bool BF16, int OUT, int MI, bool ACOL, bool BROW, int KB, bool PART>
__device__ __forceinline__ void tile_run(const KernelArgs &p, int64_t z, int tm, int tn, int64_t k0, int64_t kd,
                                         float *part) {
  static_assert(KB == 1 || MI == 16, "64-deep slabs use 16x16x32 operands");
  static_assert(KB != 3 || (!ACOL && !BROW), "staggered refills: K-contiguous operands");
  constexpr bool OUT16 = OUT != 0;
  constexpr int KD = KB == 3 ? 2 : KB;  // slab depth / 32 (KB == 3: 64-deep slabs, staggered refills)
  CtxT<LOADS * KD> c;
  const int tid = threadIdx.x;
  c.lane = tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  c.wm = c.wave >> 1;  // 2 x 2 waves of 128 x 128
  c.wn = c.wave & 1;
  const int lane = c.lane, wm = c.wm, wn = c.wn;

  const int64_t m0 = (int64_t)tm * BM, n0 = (int64_t)tn * BN;
  const int64_t M = rows_of(p, z);  // this problem's rows
  if (m0 >= M) return;              // the whole tile lies past them (uniform)
  const int64_t vrows = M - m0 < BM ? M - m0 : BM;
  const int vcols = (int)(p.N - n0 < BN ? p.N - n0 : BN);  // valid columns of this tile (N is a multiple of 8)
  // row m0, k = k0: row-major A starts its panel at row m0, column-major A at column m0
  const uint16_t *A = p.A + z * p.sA + (ACOL ? m0 + k0 * p.lda : m0 * p.lda + k0);
  // column n0, k = k0: column-major B starts its panel at row n0, row-major B at column n0
  const uint16_t *B = p.B + z * p.sB + (BROW ? n0 + k0 * p.ldb : n0 * p.ldb + k0);

  Acc<MI> acc;  // the staggered ring's first multiply defines it (mma_init); the others start from zeros
  if constexpr (KB == 3) {
  } else if constexpr (MI == 32) {
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

  // Buffer resources cover exactly the operand panels over k0 .. k0+kd: the
  // tile's valid rows of A (rows past M load as zero) and 256 rows, or kd
  // rows x 256 columns, of B.  The host keeps each extent below 1 GiB, so all
  // offsets are 32-bit.
  c.ra = make_rsrc(A, (uint32_t)((ACOL ? (kd - 1) * p.lda + vrows : (vrows - 1) * p.lda + kd) * 2));
  c.rb = make_rsrc(B, (uint32_t)((BROW ? (kd - 1) * p.ldb + vcols : (vcols - 1) * p.ldb + kd) * 2));
  if constexpr (ACOL) {
    slice_offsets_row<LOADS * KD>(c.offA, p.lda, c.wave, lane, (int)vrows);
    c.kstepA = (uint32_t)(32 * KD * p.lda * 2);
  } else {
    slice_offsets<LOADS * KD, KD>(c.offA, p.lda, c.wave, lane);
    c.kstepA = 64 * KD;
  }
  if constexpr (BROW) {
    slice_offsets_row<LOADS * KD>(c.offB, p.ldb, c.wave, lane, vcols);
    c.kstepB = (uint32_t)(32 * KD * p.ldb * 2);
  } else {
    slice_offsets<LOADS * KD, KD>(c.offB, p.ldb, c.wave, lane);
    c.kstepB = 64 * KD;
  }
  // kd is a positive multiple of 128 (the host checks K, stream-K cuts it in 128s)
  c.nk = (int)(kd / (BK * KD));

  if constexpr (KB == 3) {
    // prologue: A slabs 0 and 1, B slab 0 (the issue order the waits count on:
    // A(0), B(0), A(1), then per slab j: B(j+1) in its first half, A(j+2) in its second)
    issue<2 * LOADS>(c.ra, c.offA, 0, w_a0, c.wave);
    issue<2 * LOADS>(c.rb, c.offB, 0, WRing<0>::b(), c.wave);
    issue<2 * LOADS>(c.ra, c.offA, min(1, c.nk - 1) * c.kstepA, w_a1, c.wave);
    Frags<16> fr[2];
    slab_first<BF16>(c, fr, acc);
    // six slabs per trip: A's stage repeats every 3, B's every 2
    int j = 1;
    for (; j + 6 <= c.nk; j += 6) {
      slab_st<BF16, 1>(c, j, fr, acc);
      slab_st<BF16, 2>(c, j + 1, fr, acc);
      slab_st<BF16, 3>(c, j + 2, fr, acc);
      slab_st<BF16, 4>(c, j + 3, fr, acc);
      slab_st<BF16, 5>(c, j + 4, fr, acc);
      slab_st<BF16, 6>(c, j + 5, fr, acc);
    }
    // the remaining 1, 3 or 5 slabs (nk is even)
    slab_st<BF16, 1>(c, j, fr, acc);
    if (j + 1 < c.nk) {
      slab_st<BF16, 2>(c, j + 1, fr, acc);
      slab_st<BF16, 3>(c, j + 2, fr, acc);
      if (j + 3 < c.nk) {
        slab_st<BF16, 4>(c, j + 3, fr, acc);
        slab_st<BF16, 5>(c, j + 4, fr, acc);
      }
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    mma<BF16, 16>(fr[1], acc);  // the last sub-slice
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the duplicate tail copies
  } else if constexpr (KB == 2) {
    issue<2 * LOADS>(c.ra, c.offA, 0, WRing<0>::a(), c.wave);
    issue<2 * LOADS>(c.rb, c.offB, 0, WRing<0>::b(), c.wave);
    Frags<16> fr[2];
#pragma unroll
    for (int i = 0; i < Frags<16>::NA; ++i) fr[1].a[0][i] = fr[1].b[0][i] = u32x4{0, 0, 0, 0};
    for (int j = 0; j < c.nk; j += 2) {
      substep_w<BF16, ACOL, BROW, 0, 0>(c, j, fr, acc);
      substep_w<BF16, ACOL, BROW, 0, 1>(c, j, fr, acc);
      substep_w<BF16, ACOL, BROW, 1, 0>(c, j + 1, fr, acc);
      substep_w<BF16, ACOL, BROW, 1, 1>(c, j + 1, fr, acc);
    }
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    mma<BF16, 16>(fr[1], acc);  // the last sub-slice
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the duplicate tail loads
  } else {
  // prologue: slices 0 .. NS-2 in flight
  issue<LOADS>(c.ra, c.offA, 0 * c.kstepA, Ring<0>::a(), c.wave);
  issue<LOADS>(c.rb, c.offB, 0 * c.kstepB, Ring<0>::b(), c.wave);
  issue<LOADS>(c.ra, c.offA, 1 * c.kstepA, Ring<1>::a(), c.wave);
  issue<LOADS>(c.rb, c.offB, 1 * c.kstepB, Ring<1>::b(), c.wave);
  issue<LOADS>(c.ra, c.offA, 2 * c.kstepA, Ring<2>::a(), c.wave);
  issue<LOADS>(c.rb, c.offB, 2 * c.kstepB, Ring<2>::b(), c.wave);

  // Before slice 0 there is no previous slice: zero fragments add exactly 0.
  Frags<MI> fr[2];
#pragma unroll
  for (int s = 0; s < Frags<MI>::NSTEP; ++s)
#pragma unroll
    for (int i = 0; i < Frags<MI>::NA; ++i) fr[1].a[s][i] = fr[1].b[s][i] = u32x4{0, 0, 0, 0};

  // The steady-state loop has no data-dependent branches, which keeps the
  // 256 accumulators of each lane in place across iterations.
  for (int j = 0; j < c.nk; j += NS) {
    slice<BF16, MI, ACOL, BROW, 0>(c, j + 0, fr, acc);
    slice<BF16, MI, ACOL, BROW, 1>(c, j + 1, fr, acc);
    slice<BF16, MI, ACOL, BROW, 2>(c, j + 2, fr, acc);
    slice<BF16, MI, ACOL, BROW, 3>(c, j + 3, fr, acc);
  }
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  mma<BF16, MI>(fr[1], acc);  // the last slice (nk is a multiple of 4, so it sits in set 1)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the duplicate tail loads
  }

  // ---- epilogue: each register group holds C[m][n + 0..3]
  if constexpr (PART) {
    // a stream-K partial: the raw float32 sums of the whole 256 x 256 tile
    // (rows and columns past M and N hold zeros), row-major, through a buffer
    // resource: one lane offset, the block row in a scalar offset, the block
    // column in the instruction's immediate
    const __amdgpu_buffer_rsrc_t rp = make_rsrc(part, BM * BN * 4);
    const uint32_t lo = (uint32_t)(((wm * 128 + (lane % MI)) * BN + wn * 128 + (MI == 32 ? 4 * (lane >> 5) : 4 * (lane >> 4))) * 4);
#pragma unroll
    for (int i = 0; i < 128 / MI; ++i)
#pragma unroll
      for (int j = 0; j < 128 / MI; ++j)
#pragma unroll
        for (int g = 0; g < (MI == 32 ? 4 : 1); ++g) {
          f32x4 v;
          if constexpr (MI == 32)
            v = f32x4{acc.v[i][j][4 * g + 0], acc.v[i][j][4 * g + 1], acc.v[i][j][4 * g + 2], acc.v[i][j][4 * g + 3]};
          else
            v = acc.v[i][j];
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), rp, lo + (j * MI + (MI == 32 ? 8 * g : 0)) * 4,
                                                 i * MI * BN * 4, 0);
        }
    return;
  }
  // C through a buffer resource that ends at the tile's last valid element:
  // rows past M (ragged or grouped problems) lie beyond it, and column groups
  // past N (N is a multiple of 8: groups of 4 or 8 lie wholly on one side) get
  // an offset beyond it, so every store is unconditional.  The host keeps
  // 256 rows of C below 2^31 bytes.
  if constexpr ((OUT == 1 || OUT == 2) && MI == 16) {
    __syncthreads();  // every wave is past its last fragment read and copy
    char *const lo = stage_lo<KB == 1 ? 1 : 2>(c.wave), *const hi = stage_hi<KB == 1 ? 1 : 2>(c.wave);
    const int t = lane & 15, g = lane >> 4;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        u32x2 v;
        v[0] = pack16<OUT - 1>(acc.v[i][j][0], acc.v[i][j][1]);
        v[1] = pack16<OUT - 1>(acc.v[i][j][2], acc.v[i][j][3]);
        *reinterpret_cast<u32x2 *>((i < 4 ? lo : hi) + (16 * i + t) * 256 + ((32 * j + 8 * g) ^ (16 * t))) = v;
      }
    // a wave reads back only what it wrote, and its LDS operations complete in order
    const int64_t ldc = p.ldc;
    const int64_t vr = M - m0 < BM ? M - m0 : BM;
    const int vc = (int)(p.N - n0 < BN ? p.N - n0 : BN);
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc((char *)p.C + (z * p.sC + m0 * ldc + n0) * 2, (uint32_t)(((vr - 1) * ldc + vc) * 2));
    const int col = wn * 128 + 8 * t;  // this lane's 8 columns in every row it stores
    const uint32_t coff = col < vc ? (uint32_t)(col * 2) : kOutside;
#pragma unroll
    for (int k = 0; k < 32; ++k) {
      const int row = 4 * k + g;  // quadrant row
      const u32x4 d = *reinterpret_cast<const u32x4 *>((k < 16 ? lo : hi) + row * 256 + (t ^ (row & 15)) * 16);
      __builtin_amdgcn_raw_buffer_store_b128(d, rc, coff + (uint32_t)((wm * 128 + row) * ldc * 2), 0, kNonTemporal);
    }
    return;
  }
  // float32 output (and the 32x32 variant): straight from the accumulators,
  // one lane offset per column block, the row block added as a constant.
  const Epilogue ep = epilogue_of(p);
  constexpr int ES = OUT16 ? 2 : 4;
  const int64_t ldc = p.ldc;
  const int64_t vr = M - m0 < BM ? M - m0 : BM;
  const int vc = (int)(p.N - n0 < BN ? p.N - n0 : BN);
  const __amdgpu_buffer_rsrc_t rc =
      make_rsrc((char *)p.C + (z * p.sC + m0 * ldc + n0) * ES, (uint32_t)(((vr - 1) * ldc + vc) * ES));
  const int lr = wm * 128 + (lane % MI);
  const int lcol = wn * 128 + (MI == 32 ? 4 * (lane >> 5) : 4 * (lane >> 4));
  uint32_t coff[128 / MI][MI == 32 ? 4 : 1];
#pragma unroll
  for (int j = 0; j < 128 / MI; ++j)
#pragma unroll
    for (int g = 0; g < (MI == 32 ? 4 : 1); ++g) {
      // 32x32: group g covers columns 8g + 4*(lane/32) .. +3; 16x16: 4*(lane/16) .. +3
      const int col = lcol + j * MI + (MI == 32 ? 8 * g : 0);
      coff[j][g] = col < vc ? (uint32_t)((lr * ldc + col) * ES) : kOutside;
    }
#pragma unroll
  for (int i = 0; i < 128 / MI; ++i) {
    const uint32_t roff = (uint32_t)(i * MI * ldc * ES);
#pragma unroll
    for (int j = 0; j < 128 / MI; ++j) {
#pragma unroll
      for (int g = 0; g < (MI == 32 ? 4 : 1); ++g) {
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
        v0 = ep.apply(v0);
        v1 = ep.apply(v1);
        v2 = ep.apply(v2);
        v3 = ep.apply(v3);
        if constexpr (OUT16) {
          u32x2 v;
          v[0] = (uint32_t)ep.to16(v0) | ((uint32_t)ep.to16(v1) << 16);
          v[1] = (uint32_t)ep.to16(v2) | ((uint32_t)ep.to16(v3) << 16);
          __builtin_amdgcn_raw_buffer_store_b64(v, rc, coff[j][g] + roff, 0, 0);
        } else {
          __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, f32x4{v0, v1, v2, v3}), rc,
                                                 coff[j][g] + roff, 0, 0);
        }
      }
    }
  }
}


// Tile (z, tm, tn) of linear index t over every tile of a launch: the tiles
// of the groups' valid row blocks in a grouped call (group after group), else
// problem after problem; within a problem, the grouped tile order.
__device__ __forceinline__ void tile_of(const KernelArgs &p, int t, int64_t &z, int &tm, int &tn) {
  t += p.tile0;
  if (p.compact_groups) {
    int g = 0;
    for (; g < p.compact_groups - 1; ++g) {
      const int c = work_rows(p, g) * p.tiles_n;
      if (t < c) break;
      t -= c;
    }
    tile_order(t, work_rows(p, g), p.tiles_n, GROUP_M, tm, tn);
    z = g;
  } else {
    const int T = p.tiles_m * p.tiles_n;
    z = t / T;
    tile_order(t - (int)z * T, p.tiles_m, p.tiles_n, group_rows(p.tiles_m), tm, tn);
  }
}

// Tiles of a launch (grouped calls: the valid ones, from the counts in device memory).
__device__ __forceinline__ int launch_tiles(const KernelArgs &p) {
  if (p.tile_count) return p.tile_count;
  if (!p.compact_groups) return p.tiles_m * p.tiles_n * p.flat_batch;
  int V = 0;
  for (int g = 0; g < p.compact_groups; ++g) V += work_rows(p, g);
  return V * p.tiles_n;
}

// Stream-K: the 128-deep units of every tile (unit u is tile u / U, K from
// 128 (u % U)), dealt to P workgroups as contiguous runs, the first r of
// E + 1 units and the rest of E (the work-centric decomposition of Osama et
// al., "Stream-K", PPoPP 2023).  Every segment (the part of a run inside one
// tile) writes float32 partial sums; sk_reduce_kernel adds each tile's
// partials in run order and stores the tile once: no atomics, no zeroed
// memory, the same bits on every call ("A Dumb Triton Runtime Error", "The
// Takeaway and the Final Fix": reduce, then store once).
struct SkRuns {
  int64_t U, E, r;
  __device__ SkRuns(int64_t T, int64_t units, int P) : U(units) {
    E = T * units / P;
    r = T * units - E * P;
  }
  __device__ int64_t start(int64_t w) const { return w * E + (w < r ? w : r); }
  __device__ int64_t owner(int64_t u) const {  // run holding unit u
    const int64_t h = r * (E + 1);
    return u < h ? u / (E + 1) : r + (u - h) / E;
  }
};

// SK: 0 data-parallel; 1 stream-K, runs of up to two segments; 2 stream-K runs
// that are one whole chunk of one tile (the hybrid's leftover tiles).
template <bool BF16, int OUT, int MI, bool ACOL, bool BROW, int KB, int SK>
__global__ __launch_bounds__(256, 1) void gemm_tile_kernel(KernelArgs p) {
  if constexpr (SK == 2) {
    // Aligned run w: exactly one chunk of one tile (the host makes the chunk
    // count divide the tile's units, so e - b = U / chunks and the run starts
    // on a chunk boundary), its partial in slot w (sk_aligned tells the
    // fix-up).
    const int P = gridDim.x;
    const int w = xcd_remap(blockIdx.x, P);
    const SkRuns runs(launch_tiles(p), p.K / 128, P);
    const int U = (int)runs.U;
    const int b = (int)runs.start(w), e = (int)runs.start(w + 1);
    const int t = b / U;
    const int k0 = b - t * U;
    int64_t z;
    int tm, tn;
    tile_of(p, t, z, tm, tn);
    tile_run<BF16, OUT, MI, ACOL, BROW, KB, true>(p, z, tm, tn, 128 * (int64_t)k0, 128 * (int64_t)(e - b),
                                                    p.sk_ws + (int64_t)w * (BM * BN));
    return;
  } else if constexpr (SK == 1) {
    // Run w (the per-XCD regrouping keeps consecutive runs, and so
    // consecutive tiles, on one XCD).  The host launches at most one run per
    // tile (T <= P), so a run has E + 1 <= U units and meets at most two
    // tiles: its segment in the first goes to partial slot 2w, the one in the
    // second to slot 2w + 1.  The two are written out (not a loop): a loop
    // around the tile body holds its scalars across both and spills them.
    const int P = gridDim.x;
    const int w = xcd_remap(blockIdx.x, P);
    const SkRuns runs(launch_tiles(p), p.K / 128, P);
    const int U = (int)runs.U;  // the host keeps tiles x units below 2^31
    const int b = (int)runs.start(w), e = (int)runs.start(w + 1);
    // at most two segments (the host keeps a run within two tiles)
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const int u = s == 0 ? b : (b / U + 1) * U;  // the second segment starts at the next tile
      if (u >= e) break;
      const int t = u / U;
      const int k0 = u - t * U;
      const int k1 = k0 + (e - u) < U ? k0 + (e - u) : U;
      int64_t z;
      int tm, tn;
      tile_of(p, t, z, tm, tn);
      float *part = p.sk_ws + (2 * (int64_t)w + s) * (BM * BN);
      tile_run<BF16, OUT, MI, ACOL, BROW, KB, true>(p, z, tm, tn, 128 * (int64_t)k0, 128 * (int64_t)(k1 - k0), part);
      // the next segment's copies overwrite LDS stages whose last fragment
      // reads other waves may not have made yet
      __syncthreads();
    }
    return;
  } else {
    // ---- tile order: per-XCD regrouping, then groups of tile rows column by column
    int tm, tn;
    int64_t z;
    if (p.compact_groups) {
      // Grouped call: number only the tiles that hold rows, group after group,
      // so the per-XCD regrouping spreads the real work evenly over the XCDs
      // (the counts are in device memory; every workgroup reads them).
      const int G = p.compact_groups;
      int V = 0;
      for (int g = 0; g < G; ++g) V += work_rows(p, g);
      V *= p.tiles_n;
      if ((int)blockIdx.x >= V) return;  // uniform
      int pid = xcd_remap(blockIdx.x, V);
      int g = 0;
      for (; g < G - 1; ++g) {
        const int t = work_rows(p, g) * p.tiles_n;
        if (pid < t) break;
        pid -= t;
      }
      tile_order(pid, work_rows(p, g), p.tiles_n, GROUP_M, tm, tn);
      z = g;
    } else if (p.flat_batch) {
      // Strided batch: one 1-D grid over every tile of every problem, so the
      // per-XCD regrouping gives each XCD a run of tiles of one problem (a
      // 2-D grid would regroup within each problem only, and the 32 tiles
      // resident on an XCD would come from several problems' panels:
      // 8 x 2048 x 2048 x 4096 took 0.261 ms that way against 0.217 ms)
      const int T = p.tiles_m * p.tiles_n;
      const int pid = xcd_remap(blockIdx.x, T * p.flat_batch);
      z = pid / T;
      tile_order(pid - (int)z * T, p.tiles_m, p.tiles_n, group_rows(p.tiles_m), tm, tn);
    } else {
      // (a hybrid launch covers the first tile_count tiles of the order)
      tile_order(xcd_remap(blockIdx.x, p.tile_count ? p.tile_count : p.tiles_m * p.tiles_n), p.tiles_m, p.tiles_n,
                 group_rows(p.tiles_m), tm, tn);
      z = (int64_t)p.z0 + blockIdx.y;
    }

    tile_run<BF16, OUT, MI, ACOL, BROW, KB, false>(p, z, tm, tn, 0, p.K, nullptr);
  }
}

// Stream-K fix-up: each tile gets the sum of its segments' partials, added
// in run order (which is K order), through the epilogue into C.  Block b
// covers rows 16 (b % 16) .. +15 of tile b / 16, each thread 4 rows of 4
// consecutive columns (a wave reads 1 KiB of one row at a time).
template <bool OUT16>
__global__ __launch_bounds__(256) void sk_reduce_kernel(KernelArgs p, int P) {
  const int t = (int)(blockIdx.x >> 4);
  const int T = launch_tiles(p);
  if (t >= T) return;  // uniform (a grouped call's grid counts every tile)
  const SkRuns runs(T, p.K / 128, P);
  const int64_t u0 = (int64_t)t * runs.U;
  const int64_t w0 = runs.owner(u0), w1 = runs.owner(u0 + runs.U - 1);
  int64_t z;
  int tm, tn;
  tile_of(p, t, z, tm, tn);
  const int tid = threadIdx.x;
  const int col = 4 * (tid & 63);
  const int row0 = 16 * (int)(blockIdx.x & 15) + 4 * (tid >> 6);
  f32x4 acc[4] = {};
  for (int64_t w = w0; w <= w1; ++w) {
    // run w's segment in its first tile is in slot 2w, in its second in 2w + 1
    // (aligned runs, one segment each: slot w)
    const int64_t slot = p.sk_aligned ? w : 2 * w + (runs.start(w) < u0 ? 1 : 0);
    const float *src = p.sk_ws + slot * (BM * BN) + row0 * BN + col;
    f32x4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) v[q] = *reinterpret_cast<const f32x4 *>(src + q * BN);
#pragma unroll
    for (int q = 0; q < 4; ++q) acc[q] += v[q];
  }
  const int64_t n = (int64_t)tn * BN + col;
  if (n >= p.N) return;  // N is a multiple of 8: groups of 4 lie wholly on one side
  const int64_t M = rows_of(p, z);
  const Epilogue ep = epilogue_of(p);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t m = (int64_t)tm * BM + row0 + q;
    if (m >= M) break;
    const int64_t at = z * p.sC + m * p.ldc + n;
    store4<OUT16>(OUT16 ? (void *)((uint16_t *)p.C + at) : (void *)((float *)p.C + at), ep, acc[q][0], acc[q][1],
                  acc[q][2], acc[q][3]);
  }
}

template <bool BF16, int OUT, int MI, bool ACOL, bool BROW, int KB, int SK>
hipError_t launch_t(const KernelArgs &base, int64_t batch, int P, hipStream_t stream) {
  // (a data-parallel launch over the first tile_count tiles of one problem covers just those)
  const int64_t tiles = !SK && base.tile_count ? base.tile_count : (int64_t)base.tiles_m * base.tiles_n;
  if constexpr (SK != 0) {
    // P runs over every tile of every problem (valid tiles of a grouped
    // call), then the fix-up over the same tiles
    KernelArgs a = base;
    a.z0 = 0;
    if (base.rows)
      a.compact_groups = (int32_t)batch;
    else
      a.flat_batch = (int32_t)batch;
    hipLaunchKernelGGL((gemm_tile_kernel<BF16, OUT, MI, ACOL, BROW, KB, SK>), dim3((unsigned)P), dim3(256), 0,
                       stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((sk_reduce_kernel<OUT != 0>), dim3((unsigned)(tiles * batch * 16)), dim3(256), 0, stream, a, P);
    return hipGetLastError();
  }
  // 1-D grids while their work-items stay below 2^32, else a 2-D grid
  if (base.rows && batch <= kMaxCompactGroups && tiles * batch * 256 <= 0xffffffffLL) {
    // grouped call: one 1-D grid over every tile of every group; the kernel
    // maps the first (valid) ones to real tiles and the rest exit
    KernelArgs a = base;
    a.z0 = 0;
    a.compact_groups = (int32_t)batch;
    hipLaunchKernelGGL((gemm_tile_kernel<BF16, OUT, MI, ACOL, BROW, KB, 0>), dim3((unsigned)(tiles * batch)), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
  }
  if (!base.rows && batch > 1 && tiles * batch * 256 <= 0xffffffffLL) {
    KernelArgs a = base;
    a.z0 = 0;
    a.flat_batch = (int32_t)batch;
    hipLaunchKernelGGL((gemm_tile_kernel<BF16, OUT, MI, ACOL, BROW, KB, 0>), dim3((unsigned)(tiles * batch)), dim3(256), 0,
                       stream, a);
    return hipGetLastError();
  }
  for (int64_t z0 = 0; z0 < batch; z0 += kMaxGridY) {
    KernelArgs a = base;
    a.z0 = (int32_t)z0;
    const int64_t nz = batch - z0 < kMaxGridY ? batch - z0 : kMaxGridY;
    hipLaunchKernelGGL((gemm_tile_kernel<BF16, OUT, MI, ACOL, BROW, KB, 0>), dim3((unsigned)tiles, (unsigned)nz), dim3(256), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

// Output mode of a launch (a template parameter, so that each kernel carries
// one epilogue): 0 float32; 1 f16 and 2 bf16, no activation (the staged
// epilogue); 3 16-bit with an activation, the format read at run time.
// Stream-K launches write float32 partials: 0 or 3 (their fix-up stores).
template <bool BF16, int MI, bool ACOL, bool BROW, int KB, int SK>
hipError_t launch_out(const Problem &p, const KernelArgs &a, hipStream_t stream, int P) {
  if (!p.out16) return launch_t<BF16, 0, MI, ACOL, BROW, KB, SK>(a, p.batch, P, stream);
  if constexpr (SK == 0) {
    if (p.act == 0)
      return p.out_bf16 ? launch_t<BF16, 2, MI, ACOL, BROW, KB, SK>(a, p.batch, P, stream)
                        : launch_t<BF16, 1, MI, ACOL, BROW, KB, SK>(a, p.batch, P, stream);
  }
  return launch_t<BF16, 3, MI, ACOL, BROW, KB, SK>(a, p.batch, P, stream);
}

template <int MI, bool ACOL, bool BROW, int KB, int SK = 0>
hipError_t launch_mi(const Problem &p, const KernelArgs &a, hipStream_t stream, int P = 0) {
  return p.in_bf16 ? launch_out<true, MI, ACOL, BROW, KB, SK>(p, a, stream, P)
                   : launch_out<false, MI, ACOL, BROW, KB, SK>(p, a, stream, P);
}

KernelArgs tile_args(const Problem &p) {
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
  a.rows = p.rows;
  a.act = p.act;
  a.slope = p.slope;
  a.out_bf16 = p.out_bf16;
  a.tiles_m = (int32_t)((p.M + BM - 1) / BM);
  a.tiles_n = (int32_t)((p.N + BN - 1) / BN);
  return a;
}

}  // namespace

bool tile_supports(const Problem &p, bool a_col, bool b_row) {
  if (p.a_col != a_col || p.b_col == b_row) return false;  // the requested layouts
  // any M and any N that is a multiple of 8: rows and columns past them load
  // as zero and are not stored; a column-major A needs M % 8 too (its chunks
  // of 8 rows lie wholly inside or outside) and no grouped row counts
  if (p.N % 8 || p.K % (NS * BK) || p.K == 0) return false;
  if (a_col && (p.M % 8 || p.rows)) return false;
  // 32-bit buffer offsets: an A panel (256 rows, or K rows x 256 columns) and
  // a B panel (256 rows, or K rows x 256 columns) must span less than 1 GiB
  if ((a_col ? (p.K - 1) * p.lda + 256 : 255 * p.lda + p.K) >= (int64_t)1 << 29) return false;
  if ((b_row ? (p.K - 1) * p.ldb + 256 : 255 * p.ldb + p.K) >= (int64_t)1 << 29) return false;
  if (((uintptr_t)p.A & 15) || ((uintptr_t)p.B & 15) || ((uintptr_t)p.C & 15)) return false;
  if (p.lda % 8 || p.ldb % 8) return false;
  if (p.ldc % 4) return false;  // 8-byte (f16) / 16-byte (float32) row stores
  // 32-bit store offsets: 256 rows of C below 2^31 bytes
  if (256 * p.ldc * (p.out16 ? 2 : 4) >= (int64_t)1 << 31) return false;
  if (p.batch > 1 && (p.sA % 8 || p.sB % 8 || p.sC % 4)) return false;
  return true;
}

hipError_t launch_tile_args(const Problem &p, const KernelArgs &a, int variant, hipStream_t stream) {
  switch (variant) {
    case 0:
      return launch_mi<32, false, false, 1>(p, a, stream);
    case 1:
      return launch_mi<16, false, false, 1>(p, a, stream);
    case 2:
      return launch_mi<16, false, true, 1>(p, a, stream);
    case 3:
      return launch_mi<16, false, false, 2>(p, a, stream);
    case 4:
      return launch_mi<16, false, true, 2>(p, a, stream);
    case 5:
      return launch_mi<16, true, true, 1>(p, a, stream);
    case 6:
      return launch_mi<16, true, false, 1>(p, a, stream);
    case 7:
      return launch_mi<16, true, false, 2>(p, a, stream);
    default:
      return launch_mi<16, false, false, 3>(p, a, stream);
  }
}

hipError_t launch_tile(const Problem &p, int variant, hipStream_t stream) {
  return launch_tile_args(p, tile_args(p), variant, stream);
}

hipError_t launch_tile_sk(const Problem &p, int variant, float *ws, int P, hipStream_t stream) {
  KernelArgs a = tile_args(p);
  a.sk_ws = ws;
  switch (variant) {
    case 2:
      return launch_mi<16, false, true, 1, 1>(p, a, stream, P);
    case 5:
      return launch_mi<16, true, true, 1, 1>(p, a, stream, P);
    case 6:
      return launch_mi<16, true, false, 1, 1>(p, a, stream, P);
    case 1:
      return launch_mi<16, false, false, 1, 1>(p, a, stream, P);
    default:
      return hipErrorInvalidValue;
  }
}

hipError_t launch_tile_hybrid(const Problem &p, int variant, int sk_variant, int dp_tiles, int splits, float *ws,
                              hipStream_t stream) {
  const int64_t tiles = ((p.M + BM - 1) / BM) * ((p.N + BN - 1) / BN);
  if (p.batch != 1 || p.rows || dp_tiles <= 0 || dp_tiles >= tiles || splits < 1) return hipErrorInvalidValue;
  // whole rounds: the first dp_tiles tiles of the order, one workgroup each
  {
    KernelArgs a = tile_args(p);
    a.tile_count = dp_tiles;
    const hipError_t e = launch_tile_args(p, a, variant, stream);
    if (e != hipSuccess) return e;
  }
  // the rest: splits aligned runs per tile (stream-K runs of exactly one chunk)
  Problem q = p;
  KernelArgs a = tile_args(q);
  a.sk_ws = ws;
  a.tile0 = dp_tiles;
  a.tile_count = (int32_t)(tiles - dp_tiles);
  a.sk_aligned = 1;
  if ((p.K / 128) % splits) return hipErrorInvalidValue;  // every run one whole chunk of one tile
  const int P = (int)(tiles - dp_tiles) * splits;
  // one segment per run: the data-parallel kernel of the layout fits (the
  // staggered-refill one included)
  switch (sk_variant) {
    case 2:
      return launch_mi<16, false, true, 1, 2>(q, a, stream, P);
    case 5:
      return launch_mi<16, true, true, 1, 2>(q, a, stream, P);
    case 6:
      return launch_mi<16, true, false, 1, 2>(q, a, stream, P);
    case 8:
      return launch_mi<16, false, false, 3, 2>(q, a, stream, P);
    default:
      return hipErrorInvalidValue;
  }
}

const char *tile_name(int variant) {
  // suffix: n = stored as used (A row-major, B row-major), t = transposed storage;
  // no suffix = A row-major, B column-major
  static const char *const names[] = {"tile_256x256x32_mi32",    "tile_256x256x32_mi16",   "tile_256x256x32_mi16_nn",
                                      "tile_256x256x64_mi16",    "tile_256x256x64_mi16_nn", "tile_256x256x32_mi16_tn",
                                      "tile_256x256x32_mi16_tt", "tile_256x256x64_mi16_tt",
                                      "tile_256x256x64_mi16_st"};
  return names[variant];
}

}  // namespace tsm
