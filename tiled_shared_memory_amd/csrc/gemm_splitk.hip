// Split-K GEMM for gfx950: small M x N, deep K, row-major A and B.
//
// When M x N holds too few large tiles to occupy 256 CUs (for example
// 256 x 256 x 8192: four 128 x 128 tiles), the parallelism has to come from K.
// Each 1024-thread workgroup owns a 16 x 16 tile of C and splits K across its
// 16 waves; every wave walks its K range in 32-deep steps ("The PTSS Cliff",
// section "The Idea: Stage in SLM, Tile K": one slice live at a time, a float32
// accumulator carried across the loop), and the 16 partial tiles are then
// summed through LDS in a fixed order and stored once.  The reduction stays
// inside the workgroup ("A Dumb Triton Runtime Error", section "The Takeaway
// and the Final Fix": reduce within the block and store, rather than
// accumulate across blocks with atomics), so the result is deterministic, C is
// overwritten, and no workspace is needed.
//
// Per wave and step: the 16 x 32 A slice and the 32 x 16 B slice (1 KiB each)
// go global -> LDS with buffer loads that write LDS directly, into the wave's
// own region of a 4-stage ring, three steps ahead.  No other wave reads that
// region, so the loop has no barrier: each wave waits only for its own loads.
// B is row-major (contiguous along n); ds_read_b64_tr_b16 turns two 4 x 16
// blocks into the 8-consecutive-k operand of v_mfma_f32_16x16x32.
//
// Tiles are ordered so the 32 workgroups resident on one XCD cover 4 tile rows
// x 8 tile columns (A and B panels of 64 and 128 lines share that XCD's L2).
#include "gemm_internal.hpp"
#include "mfma.hpp"

namespace tsm {
namespace {

constexpr int WAVES = SplitKInfo::WAVES;      // 16: K is split 16 ways
constexpr int NS = 4;                         // ring stages per wave
constexpr int STEP_BYTES = 2048;              // A (1 KiB) + B (1 KiB) per wave and step
constexpr int STAGE_BYTES = WAVES * STEP_BYTES;
constexpr int GROUP_M = 4;

typedef __attribute__((address_space(3))) void lds_void;
typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) char lds_char;

__shared__ __attribute__((aligned(1024))) char g_k0[STAGE_BYTES];
__shared__ __attribute__((aligned(1024))) char g_k1[STAGE_BYTES];
__shared__ __attribute__((aligned(1024))) char g_k2[STAGE_BYTES];
__shared__ __attribute__((aligned(1024))) char g_k3[STAGE_BYTES];

template <int S> __device__ __forceinline__ char *stage();
template <> __device__ __forceinline__ char *stage<0>() { return g_k0; }
template <> __device__ __forceinline__ char *stage<1>() { return g_k1; }
template <> __device__ __forceinline__ char *stage<2>() { return g_k2; }
template <> __device__ __forceinline__ char *stage<3>() { return g_k3; }

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}

struct Ctx {
  __amdgpu_buffer_rsrc_t ra, rb;
  uint32_t offA, offB;  // per-lane byte offsets of the wave's first step
  uint32_t kstepB;      // bytes between consecutive 32-deep steps of B (32 rows)
  int nsteps, wave, lane;
};

// Issue step `t` of this wave into its region of stage s: A rows m0 .. m0+15,
// k 32t .. 32t+31 (lane l: row l/4, 8 k at 8*(l%4)) and B rows k 32t .. +31,
// columns n0 .. n0+15 (lane l: row l/2, 8 columns at 8*(l%2)).
__device__ __forceinline__ void issue(const Ctx &c, int t, char *s) {
  char *w = s + c.wave * STEP_BYTES;
  __builtin_amdgcn_raw_ptr_buffer_load_lds(c.ra, (lds_void *)w, 16, c.offA + (uint32_t)t * 64u, 0, 0, 0);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(c.rb, (lds_void *)(w + 1024), 16, c.offB + (uint32_t)t * c.kstepB, 0, 0,
                                           0);
}

template <bool BF16, bool BCOL, int S>
__device__ __forceinline__ void step(Ctx &c, int t, f32x4 &acc) {
  // step t has landed once only the two younger steps' loads (2 each) are
  // pending; the previous step's LDS reads are complete before its stage is
  // refilled below
  asm volatile("s_waitcnt vmcnt(4) lgkmcnt(0)" ::: "memory");
  const int next = min(t + NS - 1, c.nsteps - 1);  // the last step again near the end keeps counts uniform
  const char *w = stage<S>() + c.wave * STEP_BYTES;
  const int lane = c.lane;
  // A operand: row lane % 16 (64 bytes), k 8*(lane/16) .. +7
  const u32x4 af = *reinterpret_cast<const u32x4 *>(w + (lane & 15) * 64 + (lane >> 4) * 16);
  u32x4 bf;
  if constexpr (BCOL) {
    // K-contiguous B: staged like A, column lane % 16 (64 bytes), k 8*(lane/16) .. +7
    bf = *reinterpret_cast<const u32x4 *>(w + 1024 + (lane & 15) * 64 + (lane >> 4) * 16);
  } else {
    // row-major B: two transpose reads of rows 8*(lane/16) + 4h + (lane%16)/4, columns 4*(lane%4)
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int row = 8 * (lane >> 4) + 4 * h + ((lane & 15) >> 2);
      const v4s v =
          __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)((lds_char *)(w + 1024) + row * 32 + (lane & 3) * 8));
      const u32x2 d = __builtin_bit_cast(u32x2, v);
      bf[2 * h] = d[0];
      bf[2 * h + 1] = d[1];
    }
  }
  issue(c, next, stage<(S + NS - 1) % NS>());  // stage S-1 was read in step t-1
  acc = mfma_16x16x32<BF16>(bf, af, acc);
}

// BCOL: B is K-contiguous (column-major); its 16 x 32 slice per step is staged
// and read like A's.
template <bool BF16, bool OUT16, bool BCOL>
__global__ __launch_bounds__(WAVES * 64, 1) void gemm_splitk_kernel(KernelArgs p) {
  Ctx c;
  const int tid = threadIdx.x;
  c.lane = tid & 63;
  c.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = c.lane;

  // ---- tile order: per-XCD regrouping, then GROUP_M tile rows column by column
  int tm, tn;
  tile_order(xcd_remap(blockIdx.x, p.tiles_m * p.tiles_n), p.tiles_m, p.tiles_n, GROUP_M, tm, tn);
  const int64_t m0 = (int64_t)tm * 16;
  const int64_t n0 = (int64_t)tn * 16;
  const int64_t z = (int64_t)p.z0 + blockIdx.y;

  // this wave's K range: nsteps steps of 32 starting at k0
  c.nsteps = (int)(p.K / (32 * WAVES));
  const int64_t k0 = (int64_t)c.wave * c.nsteps * 32;
  const uint16_t *A = p.A + z * p.sA + m0 * p.lda + k0;
  const uint16_t *B = p.B + z * p.sB + (BCOL ? n0 * p.ldb + k0 : k0 * p.ldb + n0);
  c.ra = make_rsrc(A, (uint32_t)((15 * p.lda + (int64_t)c.nsteps * 32) * 2));
  c.offA = (uint32_t)((lane >> 2) * p.lda + 8 * (lane & 3)) * 2u;
  if constexpr (BCOL) {
    c.rb = make_rsrc(B, (uint32_t)((15 * p.ldb + (int64_t)c.nsteps * 32) * 2));
    c.offB = (uint32_t)((lane >> 2) * p.ldb + 8 * (lane & 3)) * 2u;
    c.kstepB = 64;
  } else {
    c.rb = make_rsrc(B, (uint32_t)((((int64_t)c.nsteps * 32 - 1) * p.ldb + 16) * 2));
    c.offB = (uint32_t)((lane >> 1) * p.ldb + 8 * (lane & 1)) * 2u;
    c.kstepB = (uint32_t)(32 * p.ldb * 2);
  }

  f32x4 acc = f32x4{};
  issue(c, 0, stage<0>());
  issue(c, min(1, c.nsteps - 1), stage<1>());
  issue(c, min(2, c.nsteps - 1), stage<2>());
  for (int t = 0; t < c.nsteps; t += NS) {
    step<BF16, BCOL, 0>(c, t + 0, acc);
    step<BF16, BCOL, 1>(c, t + 1, acc);
    step<BF16, BCOL, 2>(c, t + 2, acc);
    step<BF16, BCOL, 3>(c, t + 3, acc);
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");  // the duplicate tail loads

  // ---- fixed-order reduction of the 16 partial tiles through LDS
  __syncthreads();  // every wave is done with the ring
  f32x4 *part = reinterpret_cast<f32x4 *>(g_k0);  // 16 waves x 64 lanes x 16 bytes = 16 KiB
  part[c.wave * 64 + lane] = acc;
  __syncthreads();
  if (c.wave == 0) {
    f32x4 sum = part[lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) sum += part[w * 64 + lane];
    // lane holds C[m0 + lane % 16][n0 + 4 * (lane / 16) .. +3]
    const int64_t m = m0 + (lane & 15);
    const int64_t n = n0 + 4 * (lane >> 4);
    const int64_t at = z * p.sC + m * p.ldc + n;
    store4<OUT16>(OUT16 ? (void *)((uint16_t *)p.C + at) : (void *)((float *)p.C + at), epilogue_of(p), sum[0], sum[1],
                  sum[2], sum[3]);
  }
}

template <bool BF16, bool OUT16, bool BCOL>
hipError_t launch_t(const KernelArgs &base, int64_t batch, hipStream_t stream) {
  const int64_t tiles = (int64_t)base.tiles_m * base.tiles_n;
  for (int64_t z0 = 0; z0 < batch; z0 += kMaxGridY) {
    KernelArgs a = base;
    a.z0 = (int32_t)z0;
    const int64_t nz = batch - z0 < kMaxGridY ? batch - z0 : kMaxGridY;
    hipLaunchKernelGGL((gemm_splitk_kernel<BF16, OUT16, BCOL>), dim3((unsigned)tiles, (unsigned)nz), dim3(WAVES * 64), 0,
                       stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

bool splitk_supports(const Problem &p) {
  if (p.a_col) return false;  // row-major A; B either way
  if (p.rows) return false;  // stores whole 16 x 16 tiles: no per-problem row counts
  if (p.M % 16 || p.N % 16 || p.K % (32 * WAVES * NS) || p.K == 0) return false;
  if (((uintptr_t)p.A & 15) || ((uintptr_t)p.B & 15) || ((uintptr_t)p.C & 15)) return false;
  if (p.lda % 8 || p.ldb % 8 || p.ldc % 4) return false;
  if (p.batch > 1 && (p.sA % 8 || p.sB % 8 || p.sC % 4)) return false;
  // a wave's B range (K / 16 rows, or 16 columns) and A rows must span less than 2 GiB
  if ((p.b_col ? 16 * p.ldb : (p.K / WAVES) * p.ldb) >= ((int64_t)1 << 30) || 16 * p.lda >= ((int64_t)1 << 30))
    return false;
  // a launch's work-items (tiles x 1024 threads) stay below 2^32
  if ((p.M / 16) * (p.N / 16) * (WAVES * 64) > 0xffffffffLL) return false;
  return true;
}

hipError_t launch_splitk(const Problem &p, hipStream_t stream) {
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
  a.tiles_m = (int32_t)(p.M / 16);
  a.tiles_n = (int32_t)(p.N / 16);
  if (p.b_col) {
    if (p.in_bf16)
      return p.out16 ? launch_t<true, true, true>(a, p.batch, stream) : launch_t<true, false, true>(a, p.batch, stream);
    return p.out16 ? launch_t<false, true, true>(a, p.batch, stream) : launch_t<false, false, true>(a, p.batch, stream);
  }
  if (p.in_bf16)
    return p.out16 ? launch_t<true, true, false>(a, p.batch, stream) : launch_t<true, false, false>(a, p.batch, stream);
  return p.out16 ? launch_t<false, true, false>(a, p.batch, stream) : launch_t<false, false, false>(a, p.batch, stream);
}

const char *splitk_name(bool b_col) { return b_col ? "splitk_16x16_w16_t" : "splitk_16x16_w16"; }

}  // namespace tsm
