// K split through a caller's workspace: the split of the 256 x 256 kernels
// and the fixed-order reduction (pass 2).
//
// Problems with few output tiles and deep K (256 x 256 x 8192 has sixteen
// 64 x 64 tiles) cannot occupy 256 CUs by tiling M and N.  Pass 1 gives each
// workgroup one output tile and one K chunk and writes float32 partial sums,
// one M x N slab per (problem, chunk): the skinny kernel in its K-split mode
// (a 64- or 256-column panel and a row block of up to 64 rows), or, for 8-127
// tiles of 256 x 256, the large-tile kernel run over the chunks as a strided
// batch.  Pass 2 adds the slabs of each problem in chunk order and applies
// the epilogue, so C is overwritten with a deterministic result and no atomics
// or zeroed memory are involved ("A Dumb Triton Runtime Error", section "The
// Takeaway and the Final Fix": reduce, then store once, rather than
// accumulate across blocks with atomics).
//
// Memory-bound: each thread owns 4 consecutive columns of one row, loads the
// 16-byte partials of sixteen chunks at a time (all issued before the first
// add) and stores 16 bytes of float32 or 8 bytes of 16-bit output.
#include "gemm_internal.hpp"
#include "mfma.hpp"

namespace tsm {
namespace {

struct ReduceArgs {
  const float *ws;  // slabs [batch][splits][M][N]
  void *C;
  int64_t M, N, ldc, sC;
  int64_t groups;  // batch * M * N / 4
  int32_t splits;
  int32_t act;
  float slope;
  int32_t out_bf16;
};

template <bool OUT16>
__global__ __launch_bounds__(256) void ksplit_reduce_kernel(ReduceArgs r) {
  const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // group of 4 columns
  if (g >= r.groups) return;
  const int64_t q = r.N / 4;
  const int64_t per_problem = r.M * q;
  const int64_t z = g / per_problem;
  const int64_t rem = g - z * per_problem;
  const int64_t m = rem / q;
  const int64_t n = (rem - m * q) * 4;
  const int64_t slab = r.M * r.N;
  const f32x4 *w = reinterpret_cast<const f32x4 *>(r.ws + (z * r.splits * r.M + m) * r.N + n);
  const int64_t step = slab / 4;
  // sixteen chunks in flight, added in chunk order (missing ones add +0)
  f32x4 acc = f32x4{};
  for (int s0 = 0; s0 < r.splits; s0 += 16) {
    f32x4 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) v[u] = s0 + u < r.splits ? __builtin_nontemporal_load(&w[(s0 + u) * step]) : f32x4{};
#pragma unroll
    for (int u = 0; u < 16; ++u) acc += v[u];
  }
  const Epilogue ep{r.act, r.slope, r.out_bf16 != 0};
  const int64_t at = z * r.sC + m * r.ldc + n;
  store4<OUT16>(OUT16 ? (void *)((uint16_t *)r.C + at) : (void *)((float *)r.C + at), ep, acc[0], acc[1], acc[2],
                acc[3]);
}

}  // namespace

// Stream-K (on request only): runs at most 256 (the workspace holds 2
// partial tiles per run), and tiles from 32 up.
constexpr int64_t kSkMaxRuns = 256;
constexpr int64_t kSkMinTiles = 32;

KSplit tsplit_shape(int64_t M, int64_t N, int64_t K, int64_t batch) {
  KSplit ks;
  // up to 128 rows the skinny kernel's split fits better than 256-row tiles
  if (batch != 1 || M <= 128 || N < 8 || K % 128 || K < 1024) return ks;
  const int64_t tiles = ((M + TileInfo::BM - 1) / TileInfo::BM) * ((N + TileInfo::BN - 1) / TileInfo::BN);
  if (tiles < 8 || tiles > 128) return ks;
  // The plain route wins below K = 4096, and below K = 8192 under 64 tiles:
  // pass 1's tile kernel carries a fixed cost of several microseconds per
  // tile (its first slabs and its epilogue) that a short chunk does not
  // amortize, and the general kernel's 64 x 64 tiles run such shapes fast
  // (bf16, plain against split, us: 1024^2 x 4096 23.5 against 29.1, x 8192
  // 41.6 against 37.3; 2048 x 1024 x 4096 30.8 against 37.8; 1536^2 x 4096
  // 40.1 against 37.2; 2048^2 x 2048 27.3 against 37.1, x 4096 49.9 against
  // 46.4)
  if (K < 4096 || (tiles < 64 && K < 8192)) return ks;
  // about one workgroup per CU, chunks of 512 or more that divide K into
  // equal multiples of 128 (the chunks run as one strided batch).  At 128
  // tiles two chunks fill the chip (4096 x 2048 x 8192: 111 us against 135 on
  // the plain kernel); from 129 tiles two chunks need a second round and lose
  // (3072 x 3072 x 8192: 182 against 133)
  int64_t splits = 256 / tiles;
  if (splits > K / 512) splits = K / 512;
  while (splits >= 2 && (K / 128) % splits) --splits;
  if (splits < 2) return ks;
  ks.splits = (int)splits;
  ks.kchunk = K / splits;
  ks.tile_variant = 0;  // chosen by tsplit_plan from B's layout
  return ks;
}

namespace {
// Pass 1 of the tile split: the K chunks as a strided batch of products whose
// float32 results are the workspace slabs.
Problem tsplit_pass1_problem(const Problem &p, const KSplit &ks, float *ws) {
  Problem q = p;
  q.C = ws;
  q.ldc = p.N;
  q.sC = p.M * p.N;
  q.out16 = false;
  q.out_bf16 = false;
  q.act = 0;
  q.slope = 0.f;
  q.rows = nullptr;
  q.K = ks.kchunk;
  q.batch = ks.splits;
  q.sA = p.a_col ? ks.kchunk * p.lda : ks.kchunk;  // A: the next chunk starts kchunk columns (rows) on
  q.sB = p.b_col ? ks.kchunk : ks.kchunk * p.ldb;  // B: kchunk columns (K-contiguous) or rows on
  return q;
}
}  // namespace

KSplit tsplit_plan(const Problem &p) {
  KSplit ks = tsplit_shape(p.M, p.N, p.K, p.batch);
  if (!ks.splits || p.rows) return KSplit{};
  // pass 2 stores 4 consecutive columns of C at once
  if (((uintptr_t)p.C & 15) || p.ldc % 4) return KSplit{};
  const Problem q = tsplit_pass1_problem(p, ks, (float *)p.C);  // alignment of the workspace is checked apart
  if (!tile_supports(q, p.a_col, !p.b_col)) return KSplit{};
  // the default large-tile kernel for the operands' layouts
  ks.tile_variant = p.a_col ? (p.b_col ? 6 : 5) : (p.b_col ? 3 : 2);
  return ks;
}

KSplit sk_shape(int64_t M, int64_t N, int64_t K, int64_t batch, int cus) {
  KSplit ks;
  // up to 128 rows the skinny kernel's split fits better than 256-row tiles
  if (M <= 128 || K % 128 || K < 2048 || N < 8) return ks;
  const int64_t T = ((M + TileInfo::BM - 1) / TileInfo::BM) * ((N + TileInfo::BN - 1) / TileInfo::BN) * batch;
  const int64_t U = K / 128;
  const int64_t P = cus < kSkMaxRuns ? cus : kSkMaxRuns;
  // one run per tile at most (every run then meets at most two tiles), and
  // worth it while the tiles leave an eighth of the CUs or more idle
  if (T < kSkMinTiles || 8 * T > 7 * P || T * U > 0x7fffffffLL) return ks;
  ks.splits = 2;
  ks.sk_runs = (int)P;
  return ks;
}

KSplit sk_plan(const Problem &p, int cus) {
  KSplit ks = sk_shape(p.M, p.N, p.K, p.batch, cus);
  if (!ks.splits || p.rows) return KSplit{};
  if (!tile_supports(p, p.a_col, !p.b_col)) return KSplit{};
  // the 32-deep kernels: two segments of the 64-deep ones in one workgroup spill
  ks.tile_variant = p.a_col ? (p.b_col ? 6 : 5) : (p.b_col ? 1 : 2);
  return ks;
}

KSplit hybrid_shape(int64_t M, int64_t N, int64_t K, int64_t batch, int cus) {
  KSplit ks;
  // one problem of more than 128 rows (fewer belong to the streaming kernel's split)
  if (batch != 1 || M <= 128 || N < 8 || K % 128 || K < 2048) return ks;
  const int64_t T = ((M + TileInfo::BM - 1) / TileInfo::BM) * ((N + TileInfo::BN - 1) / TileInfo::BN);
  const int64_t P = cus < kSkMaxRuns ? cus : kSkMaxRuns;
  if (T <= P || T > 0x7fffffffLL / 2) return ks;
  const int64_t rem = T % P;
  if (rem == 0) return ks;
  // the last round's rem tiles in s equal chunks of K, one run each: s rem <= P runs,
  // chunks a whole number of 128-deep units
  // (at most 8: deeper runs and half the partials of 16 measured 1-2% faster
  // at 272 and 528 tiles, K = 8192: 224.7 against 227.0 us, 403.7 against 412.9)
  const int64_t U = K / 128;
  int64_t s = P / rem;
  if (s > 8) s = 8;
  while (s >= 2 && U % s) --s;
  if (s < 2) return ks;
  ks.splits = (int)s;
  ks.dp_tiles = (int)(T - rem);
  ks.sk_runs = (int)(rem * s);
  return ks;
}

KSplit hybrid_plan(const Problem &p, int cus, int dp_variant) {
  KSplit ks = hybrid_shape(p.M, p.N, p.K, p.batch, cus);
  if (!ks.splits || p.rows) return KSplit{};
  if (!tile_supports(p, p.a_col, !p.b_col)) return KSplit{};
  ks.dp_variant = dp_variant;
  ks.tile_variant = dp_variant;  // the leftover tiles' runs on the same kernel (one segment each)
  return ks;
}

hipError_t launch_ksplit(const Problem &p, const KSplit &ks, float *ws, hipStream_t stream) {
  if (ks.dp_tiles)
    return launch_tile_hybrid(p, ks.dp_variant, ks.tile_variant, ks.dp_tiles, ks.splits, ws, stream);
  if (ks.sk_runs) return launch_tile_sk(p, ks.tile_variant, ws, ks.sk_runs, stream);
  hipError_t e = ks.tile_variant >= 0 ? launch_tile(tsplit_pass1_problem(p, ks, ws), ks.tile_variant, stream)
                                      : launch_ksplit_pass1(p, ks, ws, stream);
  if (e != hipSuccess) return e;
  ReduceArgs r;
  r.ws = ws;
  r.C = p.C;
  r.M = p.M;
  r.N = p.N;
  r.ldc = p.ldc;
  r.sC = p.sC;
  r.groups = p.batch * p.M * (p.N / 4);
  r.splits = ks.splits;
  r.act = p.act;
  r.slope = p.slope;
  r.out_bf16 = p.out_bf16;
  // one wave per workgroup while 256-thread workgroups would leave CUs idle:
  // each thread's loads are all issued at once, so the reduction takes about
  // one memory latency wherever the threads run, and spreading them over more
  // CUs adds request slots
  const int threads = r.groups >= 256 * 256 ? 256 : 64;
  const int64_t blocks = (r.groups + threads - 1) / threads;
  if (p.out16)
    hipLaunchKernelGGL((ksplit_reduce_kernel<true>), dim3((unsigned)blocks), dim3(threads), 0, stream, r);
  else
    hipLaunchKernelGGL((ksplit_reduce_kernel<false>), dim3((unsigned)blocks), dim3(threads), 0, stream, r);
  return hipGetLastError();
}

}  // namespace tsm
