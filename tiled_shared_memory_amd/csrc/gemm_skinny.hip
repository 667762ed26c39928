// Skinny GEMM for gfx950: M <= 16, row-major A and B, strided batch.
//
// Decode-like products (an activation of at most 16 rows times a weight) are
// bound by streaming B from HBM: every B element is used by at most 16 output
// rows, so the kernel's job is to keep enough bytes in flight.  Each
// 256-thread workgroup owns 256 columns of C and walks all of K in slices of
// 64 ("The PTSS Cliff", section "The Idea: Stage in SLM, Tile K": one K
// slice live at a time, float32 accumulators carried across the loop):
//
//  * B slices (64 x 256 x 2 = 32 KiB) go HBM -> LDS with buffer loads that
//    write LDS directly, through a ring of 4 stages, three slices ahead: with
//    one workgroup per CU that is 96 KiB in flight per CU.
//  * The MFMA wants 8 consecutive k per lane for one column, while row-major
//    B is contiguous along n.  ds_read_b64_tr_b16 transposes on the way out
//    of LDS: in each group of 16 lanes, lane j points at row k0 + j/4, columns
//    n0 + 4*(j%4) .. +3, and lane i receives B[k0 .. k0+3][n0 + i].  Two such
//    reads give one 16x16x32 operand.
//  * A (16 x K, a few hundred KiB per problem, shared by every workgroup of
//    the problem and L2-resident) rides along: each stage also holds the
//    16 x 64 A slice (2 KiB, filled with 4-byte buffer loads into LDS), so
//    the only waits on loads are the explicit per-slice ones.
//  * LDS rows are 512 bytes (32 chunks of 16 bytes), XOR-swizzled per row
//    (see swz) so that the 16 rows one transpose read touches land on 32
//    distinct 16-byte positions.
//
// Strided batches use gridDim.y and 64-bit problem offsets (Intel XPU Triton
// README, "Avoid int32 Overflow": the B block of the 8-problem workload spans
// 2 GiB).  Rows of A at or beyond M read as zero and are never stored.
#include "gemm_internal.hpp"
#include "mfma.hpp"

namespace tsm {
namespace {

constexpr int BN = SkinnyInfo::BN;        // 256 columns per workgroup
constexpr int BK = SkinnyInfo::BK;        // 64-deep slices
constexpr int NS = 4;                     // LDS ring stages
constexpr int ROW_BYTES = BN * 2;         // 512
constexpr int SLICE_BYTES = BK * ROW_BYTES;  // 32 KiB
constexpr int LOADS = SLICE_BYTES / 1024 / 4;  // 1 KiB wave-loads of B per slice per wave (8)
constexpr int A_ROW_BYTES = BK * 2;            // 128
constexpr int A_BYTES = 16 * A_ROW_BYTES;      // 2 KiB of A per slice
constexpr int A_LOADS = A_BYTES / 256 / 4;     // 256-byte wave-loads of A per slice per wave (2)

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

__shared__ __attribute__((aligned(1024))) char g_s0[SLICE_BYTES];
__shared__ __attribute__((aligned(1024))) char g_s1[SLICE_BYTES];
__shared__ __attribute__((aligned(1024))) char g_s2[SLICE_BYTES];
__shared__ __attribute__((aligned(1024))) char g_s3[SLICE_BYTES];
__shared__ __attribute__((aligned(256))) char g_a0[A_BYTES];
__shared__ __attribute__((aligned(256))) char g_a1[A_BYTES];
__shared__ __attribute__((aligned(256))) char g_a2[A_BYTES];
__shared__ __attribute__((aligned(256))) char g_a3[A_BYTES];

template <int S> __device__ __forceinline__ char *stage();
template <> __device__ __forceinline__ char *stage<0>() { return g_s0; }
template <> __device__ __forceinline__ char *stage<1>() { return g_s1; }
template <> __device__ __forceinline__ char *stage<2>() { return g_s2; }
template <> __device__ __forceinline__ char *stage<3>() { return g_s3; }
template <int S> __device__ __forceinline__ char *astage();
template <> __device__ __forceinline__ char *astage<0>() { return g_a0; }
template <> __device__ __forceinline__ char *astage<1>() { return g_a1; }
template <> __device__ __forceinline__ char *astage<2>() { return g_a2; }
template <> __device__ __forceinline__ char *astage<3>() { return g_a3; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Swizzled position of 16-byte chunk c (0..31) of slice row r.  One
// transpose read covers rows {0..3, 8..11, 16..19, 24..27} + 4h (+ 32t) and a
// 32-byte column block (chunks 2b, 2b+1); the XOR maps those 16 rows to 16
// distinct even offsets, so the 32 chunks read land on 32 distinct positions.
__device__ __forceinline__ int swz(int r, int c) { return c ^ (2 * ((r & 3) | ((r >> 1) & 12))); }

struct Ctx {
  __amdgpu_buffer_rsrc_t rb, ra;
  uint32_t offB[LOADS];   // per-lane byte offsets of this wave's B chunks within a slice
  uint32_t offA[A_LOADS];  // per-lane byte offsets of this wave's A dwords (k = 0); out of range past M
  uint32_t ldb_bytes;     // bytes between consecutive k rows of B
  int nk, wave, lane;
};

// Cache-policy operand of the buffer loads: non-temporal.  B is read exactly
// once, and streaming it past the caches measured 6.83 TB/s against 6.62 TB/s
// with the default policy on the skinny batch.
constexpr int kNonTemporal = 2;

// Issue the loads of slice `k` into LDS stage (s, sa): B rows k*64 .. +63 of
// the panel and the matching 16 x 64 A slice.
__device__ __forceinline__ void issue(const Ctx &c, int k, char *s, char *sa) {
  const uint32_t krow = (uint32_t)k * BK * c.ldb_bytes;  // byte offset of the slice's first row
#pragma unroll
  for (int g = 0; g < LOADS; ++g)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rb, (lds_void *)(s + (c.wave * LOADS + g) * 1024), 16, c.offB[g], krow,
                                             0, kNonTemporal);
  const uint32_t kbytes = (uint32_t)k * A_ROW_BYTES;
#pragma unroll
  for (int g = 0; g < A_LOADS; ++g)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(c.ra, (lds_void *)(sa + (c.wave * A_LOADS + g) * 256), 4,
                                             c.offA[g] + kbytes, 0, 0, 0);
}

// One slice from stage S: for each 32-deep step and each of the wave's four
// 16-column blocks, two transpose reads and one MFMA.  The MFMA takes B as its
// first operand, so each lane's 4 accumulators are 4 consecutive columns of
// one row of C.
template <bool BF16, int S>
__device__ __forceinline__ void slice(Ctx &c, int j, f32x4 (&acc)[4]) {
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(2 * (LOADS + A_LOADS)) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // refill the stage (and A slot) freed by slice j-1 with slice j+3, the last
  // slice again near the end so the count of loads per slice stays uniform
  const int next = min(j + NS - 1, c.nk - 1);
  issue(c, next, stage<(S + NS - 1) % NS>(), astage<(S + NS - 1) % NS>());

  const char *s = stage<S>();
  const char *sa = astage<S>();
  const int g16 = c.lane & 15;          // lane within its 16-lane group
  const int kq = c.lane >> 4;           // which 8-deep quarter of the 32-deep step
  const int rin = g16 >> 2;             // row inside the 4-row transpose block
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    // A operand: row lane % 16, k = 32t + 8 * (lane / 16) .. +7
    const u32x4 af = *reinterpret_cast<const u32x4 *>(sa + g16 * A_ROW_BYTES + t * 64 + kq * 16);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int col = c.wave * 64 + nb * 16 + 4 * (g16 & 3);  // first of the 4 columns this lane points at
      u32x4 bf;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int r = t * 32 + kq * 8 + h * 4 + rin;            // k row inside the slice
        const int off = r * ROW_BYTES + swz(r, col >> 3) * 16 + (col & 7) * 2;
        const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)((__attribute__((address_space(3))) char *)s + off));
        const u32x2 w = __builtin_bit_cast(u32x2, v);
        bf[2 * h] = w[0];
        bf[2 * h + 1] = w[1];
      }
      acc[nb] = mfma_16x16x32<BF16>(bf, af, acc[nb]);
    }
  }
}

template <bool BF16, bool OUT16>
__global__ __launch_bounds__(256, 1) void gemm_skinny_kernel(KernelArgs p) {
  Ctx c;
  const int tid = threadIdx.x;
  c.lane = tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = c.lane;

  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const int64_t z = (int64_t)p.z0 + blockIdx.y;
  const int64_t M = rows_of(p, z);  // this problem's rows (<= 16)
  if (M == 0) return;               // uniform: nothing to compute or store
  const uint16_t *A = p.A + z * p.sA;
  const uint16_t *B = p.B + z * p.sB + n0;

  c.ldb_bytes = (uint32_t)(p.ldb * 2);
  // B resource: K rows of the 256-column panel (host keeps it below 2 GiB)
  c.rb = make_rsrc(B, (uint32_t)(((p.K - 1) * p.ldb + BN) * 2));
  // A resource: the M (<= 16) rows of A
  c.ra = make_rsrc(A, (uint32_t)(((M - 1) * p.lda + p.K) * 2));
  // rows at or beyond M point past the end of the resource: the hardware
  // returns zeros for them
  // A dwords: wave-load g of this wave fills LDS bytes [(wave*A_LOADS+g)*256, +256),
  // i.e. row 2*(wave*A_LOADS+g) + lane/32, k = 2*(lane%32)
  const int m = lane & 15;
#pragma unroll
  for (int g = 0; g < A_LOADS; ++g) {
    const int r = 2 * (c.wave * A_LOADS + g) + (lane >> 5);
    c.offA[g] = r < M ? (uint32_t)(r * p.lda + 2 * (lane & 31)) * 2u : 0x80000000u;
  }
  // B chunks: wave-load g of this wave fills LDS bytes [(wave*LOADS+g)*1024, +1024),
  // i.e. rows 2*(wave*LOADS+g) + lane/32, positions lane%32
#pragma unroll
  for (int g = 0; g < LOADS; ++g) {
    const int r = 2 * (c.wave * LOADS + g) + (lane >> 5);
    const int chunk = swz(r, lane & 31);  // swz is an involution in the chunk
    c.offB[g] = (uint32_t)r * c.ldb_bytes + (uint32_t)chunk * 16u;
  }
  c.nk = (int)(p.K / BK);  // the host guarantees K is a positive multiple of NS * BK

  f32x4 acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = f32x4{};

  issue(c, 0, stage<0>(), astage<0>());
  issue(c, 1, stage<1>(), astage<1>());
  issue(c, 2, stage<2>(), astage<2>());
  for (int j = 0; j < c.nk; j += NS) {
    slice<BF16, 0>(c, j + 0, acc);
    slice<BF16, 1>(c, j + 1, acc);
    slice<BF16, 2>(c, j + 2, acc);
    slice<BF16, 3>(c, j + 3, acc);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the duplicate tail loads

  // ---- epilogue: lane holds C[m][n .. n+3], m = lane % 16
  const Epilogue ep = epilogue_of(p);
  if (m < M) {
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int64_t n = n0 + c.wave * 64 + nb * 16 + 4 * (lane >> 4);
      const int64_t at = z * p.sC + (int64_t)m * p.ldc + n;
      store4<OUT16>(OUT16 ? (void *)((uint16_t *)p.C + at) : (void *)((float *)p.C + at), ep, acc[nb][0], acc[nb][1],
                    acc[nb][2], acc[nb][3]);
    }
  }
}

template <bool BF16, bool OUT16>
hipError_t launch_t(const KernelArgs &base, int64_t batch, hipStream_t stream) {
  for (int64_t z0 = 0; z0 < batch; z0 += kMaxGridY) {
    KernelArgs a = base;
    a.z0 = (int32_t)z0;
    const int64_t nz = batch - z0 < kMaxGridY ? batch - z0 : kMaxGridY;
    hipLaunchKernelGGL((gemm_skinny_kernel<BF16, OUT16>), dim3((unsigned)base.tiles_n, (unsigned)nz), dim3(256), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

bool skinny_supports(const Problem &p) {
  if (p.a_col || p.b_col) return false;  // row-major A and B
  if (p.M > 16 || p.M < 1) return false;
  if (p.N % BN || p.K % (NS * BK) || p.K == 0) return false;
  if (((uintptr_t)p.A & 15) || ((uintptr_t)p.B & 15) || ((uintptr_t)p.C & 15)) return false;
  if (p.lda % 8 || p.ldb % 8 || p.ldc % 4) return false;
  if (p.batch > 1 && (p.sA % 8 || p.sB % 8 || p.sC % 4)) return false;
  // 32-bit buffer offsets: one B panel (K rows) and A's M rows below 2 GiB
  if ((p.K - 1) * p.ldb + BN >= ((int64_t)1 << 30)) return false;
  if ((p.M - 1) * p.lda + p.K >= ((int64_t)1 << 30)) return false;
  return true;
}

hipError_t launch_skinny(const Problem &p, hipStream_t stream) {
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
  a.tiles_m = 1;
  a.tiles_n = (int32_t)(p.N / BN);
  if (p.in_bf16)
    return p.out16 ? launch_t<true, true>(a, p.batch, stream) : launch_t<true, false>(a, p.batch, stream);
  return p.out16 ? launch_t<false, true>(a, p.batch, stream) : launch_t<false, false>(a, p.batch, stream);
}

const char *skinny_name() { return "skinny_m16_n256_k64"; }

}  // namespace tsm
