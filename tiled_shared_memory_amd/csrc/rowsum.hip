// Tiled row-sum reduction for gfx950: out[r] = sum_c X[r*row_stride + c*col_stride].
//
// The kernel of "A Dumb Triton Runtime Error" (sections "The kernel itself",
// "Step 2: Sliding Tile Window, Boundary Masking, and Vector Accumulation",
// "Step 3: Cross-Lane Tree Reduction (tl.sum) and Scalar Store"):
//  * a row is walked in fixed-width tiles, so the register footprint does not
//    depend on the row length;
//  * each element is converted to float32 before it is added, into lane-local
//    float32 accumulators (no communication inside the loop);
//  * out-of-range lanes contribute the additive identity 0, never -inf;
//  * after the loop, one cross-lane tree reduction per row and one plain store:
//    the output is overwritten, so whatever it held before does not matter
//    ("Making It Compile, and Why I'd Still Use the Original").
//
// MI355X mapping.  The row sum is HBM-bound (one add per element loaded), so
// the design is about bytes in flight:
//  * contiguous rows (col_stride 1) with 16-byte aligned starts load 16 bytes
//    per lane (4 float32 or 8 16-bit values), eight loads in flight per lane;
//  * every load is non-temporal: each byte is read once, and streaming it past
//    the caches measured 6.7 TB/s against 5.7 TB/s for cached loads (1 GiB of
//    float32 rows);
//  * otherwise each lane loads single elements (coalesced when col_stride is
//    1, a gather when it is not);
//  * many rows: one 64-lane wave per row, 4 rows per workgroup, no barrier;
//    few long rows: one 256-thread workgroup per row, the 4 wave sums combined
//    through LDS in a fixed order.
// The reduction order is fixed, so results are bitwise reproducible.
#include "gemm_internal.hpp"
#include "mfma.hpp"

namespace tsm {
namespace {

// Element -> float32 (exact for every format).
template <int FMT>
__device__ __forceinline__ float to_f32(uint32_t bits) {
  if constexpr (FMT == RowsumInfo::F32) {
    return __builtin_bit_cast(float, bits);
  } else if constexpr (FMT == RowsumInfo::F16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
  } else {
    return __builtin_bit_cast(float, bits << 16);
  }
}

template <int FMT>
__device__ __forceinline__ float load_one(const char *X, int64_t idx) {
  if constexpr (FMT == RowsumInfo::F32) return to_f32<FMT>(__builtin_nontemporal_load((const uint32_t *)X + idx));
  return to_f32<FMT>(__builtin_nontemporal_load((const uint16_t *)X + idx));
}

// Sum of one 16-byte chunk: 4 float32 or 8 16-bit values, in a fixed order.
template <int FMT>
__device__ __forceinline__ float chunk_sum(const u32x4 &v) {
  if constexpr (FMT == RowsumInfo::F32) {
    return (to_f32<FMT>(v[0]) + to_f32<FMT>(v[1])) + (to_f32<FMT>(v[2]) + to_f32<FMT>(v[3]));
  } else {
    float s[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = to_f32<FMT>(v[i] & 0xffffu) + to_f32<FMT>(v[i] >> 16);
    return (s[0] + s[1]) + (s[2] + s[3]);
  }
}

// Lane-local partial sum of row `row` over the lanes [lane0, lane0 + width)
// of the row's tile window: VEC reads 16-byte chunks, else single elements.
template <int FMT, bool VEC>
__device__ __forceinline__ float partial(const RowsumArgs &p, int64_t row, int lane, int width) {
  constexpr int ES = FMT == RowsumInfo::F32 ? 4 : 2;  // element bytes
  const char *X = (const char *)p.X + row * p.row_stride * ES;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
  if constexpr (VEC) {
    constexpr int VW = 16 / ES;  // elements per chunk
    const int64_t nchunks = p.C / VW;
    const u32x4 *Xv = (const u32x4 *)X;
    int64_t c = lane;
    // eight chunks in flight per lane
    constexpr int U = 8;
    for (; c + (U - 1) * width < nchunks; c += U * width) {
      u32x4 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) v[u] = __builtin_nontemporal_load(&Xv[c + u * width]);
#pragma unroll
      for (int u = 0; u < U; ++u) acc[u & 3] += chunk_sum<FMT>(v[u]);
    }
    for (; c < nchunks; c += width) acc[0] += chunk_sum<FMT>(__builtin_nontemporal_load(&Xv[c]));
    // the tail (fewer than VW elements): masked single loads
    const int64_t t = nchunks * VW + lane;
    if (lane < VW && t < p.C) acc[1] += load_one<FMT>(X, t);
  } else {
    int64_t c = lane;
    for (; c + 3 * width < p.C; c += 4 * width) {
      const float v0 = load_one<FMT>(X, c * p.col_stride), v1 = load_one<FMT>(X, (c + width) * p.col_stride);
      const float v2 = load_one<FMT>(X, (c + 2 * width) * p.col_stride);
      const float v3 = load_one<FMT>(X, (c + 3 * width) * p.col_stride);
      acc[0] += v0;
      acc[1] += v1;
      acc[2] += v2;
      acc[3] += v3;
    }
    for (; c < p.C; c += width) acc[0] += load_one<FMT>(X, c * p.col_stride);
  }
  return (acc[0] + acc[1]) + (acc[2] + acc[3]);
}

// Tree reduction over the 64 lanes of a wave (butterfly: every lane ends with the sum).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
  return v;
}

// One wave per row, 4 rows per workgroup.
template <int FMT, bool VEC>
__global__ __launch_bounds__(256) void rowsum_wave_kernel(RowsumArgs p) {
  const int lane = threadIdx.x & 63;
  const int64_t row = p.r0 + (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= p.R) return;  // uniform per wave; no barrier in this kernel
  const float s = wave_sum(partial<FMT, VEC>(p, row, lane, 64));
  if (lane == 0) p.out[row] = s;
}

// One 256-thread workgroup per row.
template <int FMT, bool VEC>
__global__ __launch_bounds__(256) void rowsum_block_kernel(RowsumArgs p) {
  __shared__ float wsum[4];
  const int tid = threadIdx.x;
  const int64_t row = p.r0 + blockIdx.x;
  const float s = wave_sum(partial<FMT, VEC>(p, row, tid, 256));
  if ((tid & 63) == 0) wsum[tid >> 6] = s;
  __syncthreads();
  if (tid == 0) p.out[row] = (wsum[0] + wsum[1]) + (wsum[2] + wsum[3]);
}

// Rows per launch: a launch's work-items (blocks x 256) stay below 2^32.
constexpr int64_t kBlocksPerLaunch = 0xffffffffLL / 256;

template <int FMT, bool VEC>
hipError_t launch_t(const RowsumArgs &args, bool block_per_row, hipStream_t stream) {
  const int64_t per = block_per_row ? kBlocksPerLaunch : 4 * kBlocksPerLaunch;
  for (int64_t r0 = 0; r0 < args.R; r0 += per) {
    RowsumArgs a = args;
    a.r0 = r0;
    const int64_t rows = args.R - r0 < per ? args.R - r0 : per;
    if (block_per_row)
      hipLaunchKernelGGL((rowsum_block_kernel<FMT, VEC>), dim3((unsigned)rows), dim3(256), 0, stream, a);
    else
      hipLaunchKernelGGL((rowsum_wave_kernel<FMT, VEC>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, stream, a);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int FMT>
hipError_t launch_fmt(const RowsumArgs &a, bool vec, bool block, hipStream_t stream) {
  return vec ? launch_t<FMT, true>(a, block, stream) : launch_t<FMT, false>(a, block, stream);
}

}  // namespace

RowsumPlan rowsum_plan(const RowsumArgs &a) {
  const int es = a.fmt == RowsumInfo::F32 ? 4 : 2;
  RowsumPlan pl;
  pl.vec = a.col_stride == 1 && ((uintptr_t)a.X % 16) == 0 && (a.R <= 1 || (a.row_stride * es) % 16 == 0);
  // few long rows: a workgroup per row keeps more bytes in flight per row
  pl.block = a.R < 2048 && a.C >= 2048;
  return pl;
}

hipError_t launch_rowsum(const RowsumArgs &a, hipStream_t stream) {
  const RowsumPlan pl = rowsum_plan(a);
  switch (a.fmt) {
    case RowsumInfo::F32:
      return launch_fmt<RowsumInfo::F32>(a, pl.vec, pl.block, stream);
    case RowsumInfo::F16:
      return launch_fmt<RowsumInfo::F16>(a, pl.vec, pl.block, stream);
    default:
      return launch_fmt<RowsumInfo::BF16>(a, pl.vec, pl.block, stream);
  }
}

const char *rowsum_name(const RowsumArgs &a) {
  const RowsumPlan pl = rowsum_plan(a);
  if (pl.block) return pl.vec ? "rowsum_block_vec16" : "rowsum_block_elem";
  return pl.vec ? "rowsum_wave_vec16" : "rowsum_wave_elem";
}

}  // namespace tsm
