// Skinny GEMM for gfx950: at most 128 rows, row-major A and B, strided batch.
//
// Decode-like products (an activation of a few rows times a weight) are bound
// by streaming B from HBM: every B element is used by at most M output rows,
// so the kernel's job is to read B exactly once with enough bytes in flight.
// Each 256-thread workgroup owns W columns of C for all M rows and walks all
// of K in slices of 64 ("The PTSS Cliff", section "The Idea: Stage in SLM,
// Tile K": one K slice live at a time, float32 accumulators carried across the
// loop).  Three shapes:
//  * W = 256 (each wave 64 columns): 32 KiB B slices, one workgroup per CU;
//  * W = 64 (each wave 16 columns): 8 KiB B slices, four times the
//    workgroups, for problems whose W = 256 grid cannot fill the chip (a
//    single 16 x 16384 x 8192 product has only 64 such column blocks);
//  * W = 128 (each wave 32 columns): 16 KiB B slices, when its grid fills
//    the chip and W = 256 does not apply (65-128 rows, or a batch of two
//    16384-column weights): every workgroup reads all of A from L2, so it
//    moves half the A bytes of W = 64.
// Rows come in MB blocks of 16 (MB = 1, 2, 4 or 8; 8 not with W = 256).
//
//  * B slices go HBM -> LDS with non-temporal buffer loads that write LDS
//    directly, through a ring of NS stages, NS - 1 slices ahead (NS = 4 for
//    W = 256; 6, or 4 for MB = 8, for W = 128; 8, or 6 for MB = 8, for W = 64).
//  * K-split mode (pass 1 of the workspace path): grid.y also enumerates row
//    blocks and K chunks; each workgroup covers one chunk of one row block
//    and stores raw float32 partial sums, which a second kernel adds.
//  * The MFMA wants 8 consecutive k per lane for one column, while row-major
//    B is contiguous along n.  ds_read_b64_tr_b16 transposes on the way out
//    of LDS: in each group of 16 lanes, lane j points at row k0 + j/4, columns
//    n0 + 4*(j%4) .. +3, and lane i receives B[k0 .. k0+3][n0 + i].  Two such
//    reads give one 16x16x32 operand.
//  * A (a few MiB at most, shared by every workgroup of the problem and
//    L2-resident) rides along in each stage: 16 * MB rows x 64 k with 16-byte
//    loads into LDS, rows at or past M pointing outside the buffer resource
//    (they load as zero and are never stored).
//  * LDS rows are XOR-swizzled in 16-byte chunks (see swz_b, swz_a) so that
//    fragment reads spread over the banks.
//
// Strided batches use gridDim.y and 64-bit problem offsets (Intel XPU Triton
// README, "Avoid int32 Overflow": the B block of the 8-problem workload spans
// 2 GiB).
#include "gemm_internal.hpp"
#include "mfma.hpp"

namespace tsm {
namespace {

constexpr int BK = SkinnyInfo::BK;  // 64-deep slices
constexpr int A_ROW_BYTES = BK * 2;  // 128
constexpr uint32_t kOutside = 0x80000000u;  // a per-lane offset past every buffer resource

// Compile-time shape of one variant.
template <int MB, int W>
struct Shape {
  static_assert(W == 256 || W == 128 || W == 64, "workgroup widths");
  static_assert(MB == 1 || MB == 2 || MB == 4 || (MB == 8 && W != 256), "row blocks");
  static constexpr int CPW = W / 4;                   // columns per wave
  static constexpr int CB = CPW / 16;                 // 16-column MFMA blocks per wave
  static constexpr int ROW_BYTES = W * 2;             // one k row of the B slice
  static constexpr int SLICE_BYTES = BK * ROW_BYTES;  // B slice per stage
  static constexpr int LOADS = SLICE_BYTES / 1024 / 4;  // 1 KiB B wave-loads per wave per slice
  static constexpr int ROWS_PER_LOAD = 1024 / ROW_BYTES;
  static constexpr int CHUNKS = ROW_BYTES / 16;       // 16-byte chunks per B row
  static constexpr int A_BYTES = MB * 16 * A_ROW_BYTES;
  static constexpr int A_BLOCKS = A_BYTES / 1024;     // 1 KiB (8-row) A wave-loads per slice
  static constexpr int A_LOADS = A_BLOCKS < 4 ? 1 : A_BLOCKS / 4;  // per wave (MB = 1: two waves repeat a block)
  static constexpr int STAGE_BYTES = SLICE_BYTES + A_BYTES;
  // Ring depth: the bytes of B in flight per CU are (NS - 1) slices.  W = 256
  // runs one workgroup per CU with 3 x 32 KiB ahead; W = 64 and 128 are
  // chosen when there are about as many workgroups as CUs, so their rings are
  // deeper to keep 40-80 KiB of B in flight (and stay within the 160 KiB of
  // LDS).
  static constexpr int NS = W == 256 ? 4 : W == 128 ? (MB == 8 ? 4 : 6) : (MB == 8 ? 6 : 8);
  static_assert(NS * STAGE_BYTES <= 160 * 1024, "LDS");
  // loads a wave may leave outstanding at the wait for a slice: those of the
  // NS - 2 slices issued after it
  static constexpr int IN_FLIGHT = (NS - 2) * (LOADS + A_LOADS);
  static_assert(IN_FLIGHT < 64, "vmcnt range");
};

typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) char lds_char;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;

// Stage S of a ring of BYTES-byte stages.  Each stage is an LDS object of its
// own, so the compiler can tell the stage being filled by the direct-to-LDS
// loads from the one being read, and does not wait for the former before
// reading the latter.
template <int BYTES, int S>
__device__ __forceinline__ char *ring_stage() {
  __shared__ __attribute__((aligned(1024))) char buf[BYTES];
  return buf;
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

// Swizzled position of 16-byte chunk c of B slice row r.  One transpose read
// covers rows {0..3, 8..11, 16..19, 24..27} + 4h (+ 32t) and one 32-byte
// column block (chunks 2b, 2b+1).
//  W = 256 (32 chunks): the XOR sends those 16 rows to 16 distinct even
//    offsets, so the 32 chunks read land on 32 distinct positions;
//  W = 128 (16 chunks, rows 64 banks apart): the XOR sends the 8 rows a
//    half-wave reads (r % 4 and bit 3 of r) to 8 distinct even offsets, so
//    its 16 chunks fall on 64 distinct banks;
//  W = 64 (8 chunks, two rows per 64 banks): the 8 rows a half-wave reads
//    split by r % 2 into the two halves of the banks, and the 4 rows of
//    either half differ in bits 1 and 3 of r, which the XOR sends to 4
//    distinct even offsets, so its 16 chunks fall on 64 distinct banks (the
//    XOR on bits 3 and 4 used before left 1 conflict cycle in 6:
//    SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE 0.167 on 256 x 256 x 8192, now 0).
template <int W>
__device__ __forceinline__ int swz_b(int r, int c) {
  if constexpr (W == 256) return c ^ (2 * ((r & 3) | ((r >> 1) & 12)));
  else if constexpr (W == 128) return c ^ (2 * ((r & 3) | ((r >> 1) & 4)));
  else return c ^ (2 * (((r >> 1) & 1) | ((r >> 2) & 2)));
}

// Position of chunk c of A slice row r (128-byte rows): c ^ ((r / 2) % 8), the
// swizzle measured conflict-free for 16x16x32 operand reads of 128-byte rows.
__device__ __forceinline__ int swz_a(int r, int c) { return c ^ ((r >> 1) & 7); }

template <int MB, int W, bool BCOL>
struct Ctx {
  using SH = Shape<MB, W>;
  __amdgpu_buffer_rsrc_t rb, ra;
  uint32_t offB[SH::LOADS];    // per-lane byte offsets of this wave's B chunks within a slice
  uint32_t offA[SH::A_LOADS];  // per-lane byte offsets of this wave's A chunks (k = 0); outside past M
  uint32_t kstep_b;            // bytes between consecutive slices of B (64 rows, or 128 bytes if K-contiguous)
  int nk, wave, lane;
};

// Cache-policy operand of the B loads: non-temporal.  B is read exactly once,
// and streaming it past the caches measured 6.83 TB/s against 6.62 TB/s with
// the default policy on the skinny batch.
constexpr int kNonTemporal = 2;

// One 16-byte direct-to-LDS load per lane: lane i writes lds + 16 i.  Plain
// (not templated) functions, so that the host pass of the compiler never
// instantiates the device builtin.
__device__ __forceinline__ void dma16_nt(__amdgpu_buffer_rsrc_t r, char *lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voff, soff, 0, kNonTemporal);
}
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char *lds, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds, 16, voff, soff, 0, 0);
}

// Transposing 8-byte LDS read (see the header comment).
__device__ __forceinline__ u32x2 read_tr(const char *p) {
  const v4s v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(lds_char *)p);
  return __builtin_bit_cast(u32x2, v);
}

// Issue the loads of slice `k` into LDS stage s: B rows k*64 .. +63 of the
// panel, then the matching A slice behind it.  Slices at or past the end of K
// (the loop runs whole rounds of the ring) get per-lane offsets outside both
// buffer resources, so they load as zero and add nothing.
template <int MB, int W, bool BCOL>
__device__ __forceinline__ void issue(const Ctx<MB, W, BCOL> &c, int k, char *s) {
  using SH = Shape<MB, W>;
  const bool in = k < c.nk;
  const uint32_t past = in ? 0u : kOutside;              // per-lane offsets stay below 1 GiB
  const uint32_t krow = in ? (uint32_t)k * c.kstep_b : 0u;  // byte offset of the slice's first k
#pragma unroll
  for (int g = 0; g < SH::LOADS; ++g) dma16_nt(c.rb, s + (c.wave * SH::LOADS + g) * 1024, c.offB[g] | past, krow);
  const uint32_t kbytes = in ? (uint32_t)k * A_ROW_BYTES : 0u;
#pragma unroll
  for (int g = 0; g < SH::A_LOADS; ++g) {
    const int q = (c.wave * SH::A_LOADS + g) % SH::A_BLOCKS;
    dma16(c.ra, s + SH::SLICE_BYTES + q * 1024, c.offA[g] | past, kbytes);
  }
}

// One slice from stage S: for each 32-deep step, the MB A fragments, then per
// 16-column block two transpose reads and MB MFMAs.  The MFMA takes B as its
// first operand, so each lane's 4 accumulators are 4 consecutive columns of
// one row of C.
template <bool BF16, int MB, int W, bool BCOL, int S>
__device__ __forceinline__ void slice(Ctx<MB, W, BCOL> &c, int j, f32x4 (&acc)[MB][Shape<MB, W>::CB]) {
  using SH = Shape<MB, W>;
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"(SH::IN_FLIGHT) : "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  // refill the stage freed by slice j-1 with slice j+NS-1
  constexpr int NS = SH::NS;
  issue<MB, W, BCOL>(c, j + NS - 1, ring_stage<SH::STAGE_BYTES, (S + NS - 1) % NS>());

  const char *s = ring_stage<SH::STAGE_BYTES, S>();
  const char *sa = s + SH::SLICE_BYTES;
  const int g16 = c.lane & 15;  // lane within its 16-lane group
  const int kq = c.lane >> 4;   // which 8-deep quarter of the 32-deep step
  const int rin = g16 >> 2;     // row inside the 4-row transpose block
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    // A operands: row 16*mb + lane % 16, k = 32t + 8 * (lane / 16) .. +7
    u32x4 af[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const int r = mb * 16 + g16;
      af[mb] = *reinterpret_cast<const u32x4 *>(sa + r * A_ROW_BYTES + swz_a(r, t * 4 + kq) * 16);
    }
#pragma unroll
    for (int cb = 0; cb < SH::CB; ++cb) {
      u32x4 bf;
      if constexpr (BCOL) {
        // K-contiguous B: column n = wave*CPW + 16 cb + lane % 16 is LDS row n,
        // laid out like an A row: one 16-byte read
        const int r = c.wave * SH::CPW + cb * 16 + g16;
        bf = *reinterpret_cast<const u32x4 *>(s + r * A_ROW_BYTES + swz_a(r, t * 4 + kq) * 16);
      } else {
        const int col = c.wave * SH::CPW + cb * 16 + 4 * (g16 & 3);  // first of the 4 columns this lane points at
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int r = t * 32 + kq * 8 + h * 4 + rin;  // k row inside the slice
          const int off = r * SH::ROW_BYTES + swz_b<W>(r, col >> 3) * 16 + (col & 7) * 2;
          const u32x2 w = read_tr(s + off);
          bf[2 * h] = w[0];
          bf[2 * h + 1] = w[1];
        }
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb][cb] = mfma_16x16x32<BF16>(bf, af[mb], acc[mb][cb]);
    }
  }
}

// Fill stages 0 .. NS-2 with slices 0 .. NS-2.
template <int MB, int W, bool BCOL, int S>
__device__ __forceinline__ void prologue(const Ctx<MB, W, BCOL> &c) {
  if constexpr (S < Shape<MB, W>::NS - 1) {
    issue<MB, W, BCOL>(c, S, ring_stage<Shape<MB, W>::STAGE_BYTES, S>());
    prologue<MB, W, BCOL, S + 1>(c);
  }
}

// One round of the ring: slices j+S .. j+NS-1 from stages S .. NS-1.
template <bool BF16, int MB, int W, bool BCOL, int S>
__device__ __forceinline__ void round_from(Ctx<MB, W, BCOL> &c, int j, f32x4 (&acc)[MB][Shape<MB, W>::CB]) {
  if constexpr (S < Shape<MB, W>::NS) {
    slice<BF16, MB, W, BCOL, S>(c, j + S, acc);
    round_from<BF16, MB, W, BCOL, S + 1>(c, j, acc);
  }
}

// BCOL: B is K-contiguous (column-major, element (k, n) at B[n*ldb + k], the
// layout of a weight stored output-feature by output-feature); its slices are
// W rows of 64 k, staged and read like A.
template <bool BF16, bool OUT16, int MB, int W, bool BCOL>
__global__ __launch_bounds__(256) void gemm_skinny_kernel(KernelArgs p) {
  using SH = Shape<MB, W>;
  Ctx<MB, W, BCOL> c;
  const int tid = threadIdx.x;
  c.lane = tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = c.lane;

  int64_t n0 = (int64_t)blockIdx.x * W;
  int64_t zz = (int64_t)p.z0 + blockIdx.y;
  // K-split pass: grid.y enumerates (problem z, K chunk s, row block), and
  // the workgroup computes rows r0 .. r0+16*MB-1 over k0 .. k0+K-1.
  // Workgroup i of a launch runs on XCD i % 8; numbering the work so that
  // each XCD's share is contiguous (column block fastest, then row block,
  // then chunk) lets the workgroups on one XCD share their chunk's A and B
  // panels in its L2.
  int64_t z = zz, s = 0, r0 = 0;
  if (p.splits) {
    const int64_t gx = gridDim.x, total = gx * gridDim.y;
    int64_t id = blockIdx.x + (int64_t)blockIdx.y * gx;
    if (total % 8 == 0) id = (id % 8) * (total / 8) + id / 8;
    n0 = (id % gx) * W;
    zz = p.z0 + id / gx;
    r0 = (zz % p.row_blocks) * (16 * MB);
    const int64_t t = zz / p.row_blocks;
    s = t % p.splits;
    z = t / p.splits;
  }
  int64_t M = rows_of(p, z) - r0;  // this workgroup's rows (<= 16 * MB)
  if (M > 16 * MB) M = 16 * MB;
  if (M <= 0) return;  // uniform: nothing to compute or store
  const int64_t k0 = s * p.kchunk;
  const int64_t K = p.splits ? (p.K - k0 < p.kchunk ? p.K - k0 : p.kchunk) : p.K;  // a positive multiple of 64
  const uint16_t *A = p.A + z * p.sA + r0 * p.lda + k0;
  const uint16_t *B = p.B + z * p.sB + (BCOL ? n0 * p.ldb + k0 : k0 * p.ldb + n0);

  // B resource: the W-column panel over this K range, K rows of W columns or
  // W rows of K (host keeps it below 1 GiB)
  c.rb = make_rsrc(B, (uint32_t)((BCOL ? (W - 1) * p.ldb + K : (K - 1) * p.ldb + W) * 2));
  c.kstep_b = BCOL ? (uint32_t)A_ROW_BYTES : (uint32_t)(BK * p.ldb * 2);
  // A resource: the M rows of A; rows at or past M point outside it
  c.ra = make_rsrc(A, (uint32_t)(((M - 1) * p.lda + K) * 2));
  // A chunks: block q = 8 rows; lane l fills row 8q + l/8 at position l%8
#pragma unroll
  for (int g = 0; g < SH::A_LOADS; ++g) {
    const int q = (c.wave * SH::A_LOADS + g) % SH::A_BLOCKS;
    const int r = 8 * q + (lane >> 3);
    c.offA[g] = r < M ? (uint32_t)(r * p.lda + swz_a(r, lane & 7) * 8) * 2u : kOutside;
  }
  // B chunks: wave-load g of this wave fills LDS bytes [(wave*LOADS+g)*1024, +1024),
  // i.e. rows ROWS_PER_LOAD*(wave*LOADS+g) + lane/CHUNKS, position lane%CHUNKS
#pragma unroll
  for (int g = 0; g < SH::LOADS; ++g) {
    if constexpr (BCOL) {
      // column-major B: 128-byte rows (one per column), 8 per wave-load, like A
      const int r = 8 * (c.wave * SH::LOADS + g) + (lane >> 3);
      c.offB[g] = (uint32_t)(r * p.ldb + swz_a(r, lane & 7) * 8) * 2u;
    } else {
      const int r = SH::ROWS_PER_LOAD * (c.wave * SH::LOADS + g) + lane / SH::CHUNKS;
      const int chunk = swz_b<W>(r, lane % SH::CHUNKS);  // the swizzle is an involution in the chunk
      c.offB[g] = (uint32_t)(r * p.ldb * 2) + (uint32_t)chunk * 16u;
    }
  }
  c.nk = (int)(K / BK);  // the host guarantees K is a positive multiple of BK

  f32x4 acc[MB][SH::CB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int cb = 0; cb < SH::CB; ++cb) acc[mb][cb] = f32x4{};

  prologue<MB, W, BCOL, 0>(c);
  // whole rounds; the slices past K in the last one are zero
  for (int j = 0; j < c.nk; j += SH::NS) round_from<BF16, MB, W, BCOL, 0>(c, j, acc);
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the loads issued past the end

  // ---- epilogue: lane holds C[r0 + 16 mb + lane % 16][n .. n+3]; a K-split
  // pass stores raw float32 sums into slab z * splits + s (its ldc is N)
  const Epilogue ep = epilogue_of(p);
  const int64_t zc = p.splits ? z * p.splits + s : z;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) {
    const int64_t m = mb * 16 + (lane & 15);
    if (m >= M) continue;
#pragma unroll
    for (int cb = 0; cb < SH::CB; ++cb) {
      const int64_t n = n0 + c.wave * SH::CPW + cb * 16 + 4 * (lane >> 4);
      const int64_t at = zc * p.sC + (r0 + m) * p.ldc + n;
      store4<OUT16>(OUT16 ? (void *)((uint16_t *)p.C + at) : (void *)((float *)p.C + at), ep, acc[mb][cb][0],
                    acc[mb][cb][1], acc[mb][cb][2], acc[mb][cb][3]);
    }
  }
}

template <bool BF16, bool OUT16, int MB, int W, bool BCOL>
hipError_t launch_t(const KernelArgs &base, int64_t batch, hipStream_t stream) {
  for (int64_t z0 = 0; z0 < batch; z0 += kMaxGridY) {
    KernelArgs a = base;
    a.z0 = (int32_t)z0;
    const int64_t nz = batch - z0 < kMaxGridY ? batch - z0 : kMaxGridY;
    hipLaunchKernelGGL((gemm_skinny_kernel<BF16, OUT16, MB, W, BCOL>), dim3((unsigned)(base.N / W), (unsigned)nz),
                       dim3(256), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int MB, int W, bool BCOL>
hipError_t launch_layout(const Problem &p, const KernelArgs &a, hipStream_t stream) {
  if (p.in_bf16)
    return p.out16 ? launch_t<true, true, MB, W, BCOL>(a, p.batch, stream)
                   : launch_t<true, false, MB, W, BCOL>(a, p.batch, stream);
  return p.out16 ? launch_t<false, true, MB, W, BCOL>(a, p.batch, stream)
                 : launch_t<false, false, MB, W, BCOL>(a, p.batch, stream);
}

template <int MB, int W>
hipError_t launch_shape(const Problem &p, const KernelArgs &a, hipStream_t stream) {
  return p.b_col ? launch_layout<MB, W, true>(p, a, stream) : launch_layout<MB, W, false>(p, a, stream);
}

}  // namespace

SkinnyPlan skinny_plan(const Problem &p) {
  SkinnyPlan pl{};
  if (p.a_col) return pl;  // row-major A; B either way
  if (p.M < 1 || p.M > 128) return pl;
  pl.mb = p.M <= 16 ? 1 : p.M <= 32 ? 2 : p.M <= 64 ? 4 : 8;
  // The widest panel whose grid fills the chip (one workgroup per CU): wider
  // panels re-read A fewer times.  W = 256 up to 64 rows; W = 128 with
  // row-major B, or with 65-128 rows (with K-contiguous B and fewer rows it
  // measured slower than W = 64: 16 x 16384 x 8192, batch 2, 119 us against
  // 105); else W = 64, whose grid is four times that of W = 256 (a single
  // decode product: 49.5 us against 56.1 for W = 128 at 16 rows, 70.5 against
  // 82.3 at 128 rows).  A forced width must fit the problem.
  const bool fills256 = (p.N / 256) * p.batch >= 256, fills128 = (p.N / 128) * p.batch >= 256;
  int w = 64;
  if (p.N % 256 == 0 && pl.mb <= 4 && fills256)
    w = 256;
  else if (p.N % 128 == 0 && fills128 && (!p.b_col || pl.mb == 8))
    w = 128;
  pl.w = p.skinny_w ? p.skinny_w : w;
  if (pl.w != 64 && pl.w != 128 && pl.w != 256) return SkinnyPlan{};
  if (pl.w == 256 && pl.mb > 4) return SkinnyPlan{};
  if (p.N % pl.w) return SkinnyPlan{};
  if ((p.N / pl.w) * 256 > 0xffffffffLL) return SkinnyPlan{};  // a launch's work-items stay below 2^32
  if (p.K % BK || p.K == 0) return SkinnyPlan{};
  if (((uintptr_t)p.A & 15) || ((uintptr_t)p.B & 15) || ((uintptr_t)p.C & 15)) return SkinnyPlan{};
  if (p.lda % 8 || p.ldb % 8 || p.ldc % 4) return SkinnyPlan{};
  if (p.batch > 1 && (p.sA % 8 || p.sB % 8 || p.sC % 4)) return SkinnyPlan{};
  // 32-bit buffer offsets: one B panel (K rows of W, or W rows of K) and A's M rows below 1 GiB
  if ((p.b_col ? (pl.w - 1) * p.ldb + p.K : (p.K - 1) * p.ldb + pl.w) >= ((int64_t)1 << 29)) return SkinnyPlan{};
  if ((p.M - 1) * p.lda + p.K >= ((int64_t)1 << 29)) return SkinnyPlan{};
  return pl;
}

bool skinny_supports(const Problem &p) { return skinny_plan(p).mb != 0; }

int skinny_ring_slices(const SkinnyPlan &pl) {
  if (pl.w == 256) return Shape<1, 256>::NS;
  if (pl.w == 128) return pl.mb == 8 ? Shape<8, 128>::NS : Shape<1, 128>::NS;
  return pl.mb == 8 ? Shape<8, 64>::NS : Shape<1, 64>::NS;
}

hipError_t launch_skinny(const Problem &p, hipStream_t stream) {
  const SkinnyPlan pl = skinny_plan(p);
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
  a.tiles_n = (int32_t)(p.N / pl.w);
  if (pl.w == 256) {
    if (pl.mb == 1) return launch_shape<1, 256>(p, a, stream);
    if (pl.mb == 2) return launch_shape<2, 256>(p, a, stream);
    return launch_shape<4, 256>(p, a, stream);
  }
  if (pl.w == 128) {
    if (pl.mb == 1) return launch_shape<1, 128>(p, a, stream);
    if (pl.mb == 2) return launch_shape<2, 128>(p, a, stream);
    if (pl.mb == 4) return launch_shape<4, 128>(p, a, stream);
    return launch_shape<8, 128>(p, a, stream);
  }
  if (pl.mb == 1) return launch_shape<1, 64>(p, a, stream);
  if (pl.mb == 2) return launch_shape<2, 64>(p, a, stream);
  if (pl.mb == 4) return launch_shape<4, 64>(p, a, stream);
  return launch_shape<8, 64>(p, a, stream);
}

namespace {
// The split with row blocks of 16 * mb rows (splits 0: none).
KSplit ksplit_for(int64_t M, int64_t N, int64_t K, int64_t batch, bool wide, int mb) {
  KSplit ks;
  const int64_t row_blocks = (M + 16 * mb - 1) / (16 * mb);
  // every row block reads all of B again: beyond 512 rows the 256 x 256
  // kernels' split (tsplit_shape) reads less
  if (row_blocks > 8) return ks;
  // workgroups without a split: 64-column panels, or (wide: row-major B)
  // 256-column panels when there are enough of them for a split of at most 8
  // (each workgroup then streams 512-byte row segments of B, which HBM serves
  // faster than the 128-byte segments of 64-column panels; a K-contiguous B
  // is read in 128-byte row segments at either width, and the wider split
  // measured slower there)
  int w = 64;
  int64_t base = batch * (N / 64) * row_blocks;
  if (wide && N % 256 == 0) {
    const int64_t base256 = batch * (N / 256) * row_blocks;
    if (base256 >= 32 && base256 < 128) {
      w = 256;
      base = base256;
    }
  }
  if (base >= 128) return ks;                          // enough to keep most CUs busy
  int64_t splits = 256 / base;                         // about one workgroup per CU
  if (splits > K / 256) splits = K / 256;              // chunks at least 256 deep
  if (splits > 64) splits = 64;
  if (splits < 2) return ks;
  const int64_t kchunk = ((K + splits - 1) / splits + BK - 1) / BK * BK;
  splits = (K + kchunk - 1) / kchunk;
  if (splits < 2 || batch * splits * row_blocks > 0x7fffffffLL) return ks;
  ks.splits = (int)splits;
  ks.kchunk = kchunk;
  ks.mb = mb;
  ks.row_blocks = (int)row_blocks;
  ks.w = w;
  return ks;
}
}  // namespace

KSplit ksplit_shape(int64_t M, int64_t N, int64_t K, int64_t batch, bool wide) {
  if (M < 1 || N < 64 || N % 64 || K % BK || K < 512 || batch < 1) return KSplit{};
  // over 128 rows the general kernel's 64 x 64 tiles run short K faster than
  // the split's two launches (512 x 512 x 1024: 7.3 us against 9.7; 256 x 256
  // x 1024: 7.2 against 8.8; at K = 2048 the split wins, 10.0 against 11.5)
  if (M > 128 && K < 2048) return KSplit{};
  const int mb = M <= 16 ? 1 : M <= 32 ? 2 : 4;
  KSplit ks = ksplit_for(M, N, K, batch, wide, mb);
  // 64-row blocks whose chunks would not fill two rounds of the 64-column
  // kernel's ring: 32-row blocks reach about as many workgroups with deeper
  // chunks (and fewer partial slabs), which the ring then pipelines
  // (256 x 256 x 8192: 32-row blocks in 8 chunks 8.5 us, 64-row blocks in 16
  // chunks 10.2; 256 x 256 x 4096 7.8 against 9.7; 128 x 256 x 8192 8.3
  // against 10.4).  Where 64-row chunks are deep enough the extra re-reads of
  // B lose (256 x 512 x 8192: 11.6 against 10.7).
  if (mb == 4 && ks.splits && ks.w == 64 && ks.kchunk < 2 * Shape<4, 64>::NS * BK) {
    const KSplit k2 = ksplit_for(M, N, K, batch, wide, 2);
    if (k2.splits && k2.w == 64 && k2.kchunk > ks.kchunk) ks = k2;
  }
  return ks;
}

KSplit ksplit_plan(const Problem &p) {
  const KSplit ks = ksplit_shape(p.M, p.N, p.K, p.batch, !p.b_col);
  if (!ks.splits || p.a_col || p.rows) return KSplit{};
  if (((uintptr_t)p.A & 15) || ((uintptr_t)p.B & 15) || ((uintptr_t)p.C & 15)) return KSplit{};
  if (p.lda % 8 || p.ldb % 8 || p.ldc % 4) return KSplit{};
  if (p.batch > 1 && (p.sA % 8 || p.sB % 8 || p.sC % 4)) return KSplit{};
  // 32-bit buffer offsets within one chunk: B's panel, A's row block
  if ((p.b_col ? (ks.w - 1) * p.ldb + ks.kchunk : (ks.kchunk - 1) * p.ldb + ks.w) >= ((int64_t)1 << 29))
    return KSplit{};
  if ((16 * ks.mb - 1) * p.lda + ks.kchunk >= ((int64_t)1 << 29)) return KSplit{};
  return ks;
}

template <int MB, int W, bool BCOL>
hipError_t launch_split_mb(const Problem &p, const KernelArgs &a, int64_t launches, hipStream_t stream) {
  return p.in_bf16 ? launch_t<true, false, MB, W, BCOL>(a, launches, stream)
                   : launch_t<false, false, MB, W, BCOL>(a, launches, stream);
}

template <int W, bool BCOL>
hipError_t launch_split_layout(const Problem &p, const KSplit &ks, const KernelArgs &a, int64_t launches,
                               hipStream_t stream) {
  if (ks.mb == 1) return launch_split_mb<1, W, BCOL>(p, a, launches, stream);
  if (ks.mb == 2) return launch_split_mb<2, W, BCOL>(p, a, launches, stream);
  return launch_split_mb<4, W, BCOL>(p, a, launches, stream);
}

template <int W>
hipError_t launch_split_w(const Problem &p, const KSplit &ks, const KernelArgs &a, int64_t launches,
                          hipStream_t stream) {
  return p.b_col ? launch_split_layout<W, true>(p, ks, a, launches, stream)
                 : launch_split_layout<W, false>(p, ks, a, launches, stream);
}

hipError_t launch_ksplit_pass1(const Problem &p, const KSplit &ks, float *ws, hipStream_t stream) {
  KernelArgs a{};
  a.A = p.A;
  a.B = p.B;
  a.C = ws;
  a.M = p.M;
  a.N = p.N;
  a.K = p.K;
  a.lda = p.lda;
  a.ldb = p.ldb;
  a.ldc = p.N;
  a.sA = p.sA;
  a.sB = p.sB;
  a.sC = p.M * p.N;
  a.splits = ks.splits;
  a.row_blocks = ks.row_blocks;
  a.kchunk = ks.kchunk;
  a.tiles_m = 1;
  a.tiles_n = (int32_t)(p.N / ks.w);
  const int64_t launches = p.batch * ks.row_blocks * ks.splits;  // grid.y entries
  return ks.w == 256 ? launch_split_w<256>(p, ks, a, launches, stream) : launch_split_w<64>(p, ks, a, launches, stream);
}

const char *ksplit_name(const KSplit &ks, bool b_col) {
  if (ks.dp_tiles) {
    switch (ks.dp_variant) {
      case 8:
        return "hybrid_tile_256x256x64_mi16_st+reduce";
      case 2:
        return "hybrid_tile_256x256x32_mi16_nn+reduce";
      case 5:
        return "hybrid_tile_256x256x32_mi16_tn+reduce";
      default:
        return "hybrid_tile_256x256x32_mi16_tt+reduce";
    }
  }
  if (ks.sk_runs) {
    switch (ks.tile_variant) {
      case 1:
        return "streamk_tile_256x256x32_mi16+reduce";
      case 2:
        return "streamk_tile_256x256x32_mi16_nn+reduce";
      case 5:
        return "streamk_tile_256x256x32_mi16_tn+reduce";
      default:
        return "streamk_tile_256x256x32_mi16_tt+reduce";
    }
  }
  if (ks.splits && ks.tile_variant == 3) return "ksplit_tile_256x256x64_mi16+reduce";
  if (ks.splits && ks.tile_variant == 2) return "ksplit_tile_256x256x32_mi16_nn+reduce";
  if (ks.splits && ks.tile_variant == 5) return "ksplit_tile_256x256x32_mi16_tn+reduce";
  if (ks.splits && ks.tile_variant == 6) return "ksplit_tile_256x256x32_mi16_tt+reduce";
  static const char *const names[2][2][3] = {
      {{"ksplit_skinny_m16_n64_k64+reduce", "ksplit_skinny_m32_n64_k64+reduce", "ksplit_skinny_m64_n64_k64+reduce"},
       {"ksplit_skinny_m16_n256_k64+reduce", "ksplit_skinny_m32_n256_k64+reduce",
        "ksplit_skinny_m64_n256_k64+reduce"}},
      {{"ksplit_skinny_m16_n64_k64_t+reduce", "ksplit_skinny_m32_n64_k64_t+reduce",
        "ksplit_skinny_m64_n64_k64_t+reduce"},
       {"ksplit_skinny_m16_n256_k64_t+reduce", "ksplit_skinny_m32_n256_k64_t+reduce",
        "ksplit_skinny_m64_n256_k64_t+reduce"}}};
  if (!ks.splits) return nullptr;
  return names[b_col][ks.w == 256][ks.mb == 1 ? 0 : ks.mb == 2 ? 1 : 2];
}

const char *skinny_name(const Problem &p) {
  // suffix _t: B stored transposed (column-major, K-contiguous)
  static const char *const names[2][3][4] = {
      {{"skinny_m16_n64_k64", "skinny_m32_n64_k64", "skinny_m64_n64_k64", "skinny_m128_n64_k64"},
       {"skinny_m16_n128_k64", "skinny_m32_n128_k64", "skinny_m64_n128_k64", "skinny_m128_n128_k64"},
       {"skinny_m16_n256_k64", "skinny_m32_n256_k64", "skinny_m64_n256_k64", nullptr}},
      {{"skinny_m16_n64_k64_t", "skinny_m32_n64_k64_t", "skinny_m64_n64_k64_t", "skinny_m128_n64_k64_t"},
       {"skinny_m16_n128_k64_t", "skinny_m32_n128_k64_t", "skinny_m64_n128_k64_t", "skinny_m128_n128_k64_t"},
       {"skinny_m16_n256_k64_t", "skinny_m32_n256_k64_t", "skinny_m64_n256_k64_t", nullptr}}};
  const SkinnyPlan pl = skinny_plan(p);
  if (!pl.mb) return nullptr;
  const int i = pl.mb == 1 ? 0 : pl.mb == 2 ? 1 : pl.mb == 4 ? 2 : 3;
  return names[p.b_col][pl.w == 64 ? 0 : pl.w == 128 ? 1 : 2][i];
}

}  // namespace tsm
