// Host side of the C ABI declared in include/tsm_gemm.h: argument checks,
// kernel selection and launch on the caller's stream.
//
// Every check runs on the host before any HIP call, so a rejected call enqueues
// nothing.  Offsets and extents are computed in 64 bits with explicit overflow
// checks (Intel XPU Triton README, "Avoid int32 Overflow": a stride product that
// wraps silently addresses the wrong memory).
#include <stdarg.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <set>
#include <string>

#include "gemm_internal.hpp"
#include "tsm_gemm.h"

namespace tsm {
namespace {

thread_local char g_detail[256];

int fail(int code, const char *fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_detail, sizeof g_detail, fmt, ap);
  va_end(ap);
  return code;
}

bool mul_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_mul_overflow(a, b, out); }
bool add_ok(int64_t a, int64_t b, int64_t *out) { return !__builtin_add_overflow(a, b, out); }

// Number of elements spanned by `batch` matrices of rows x cols with leading
// dimension ld and batch stride s: (batch-1)*s + (rows-1)*ld + cols.
bool extent(int64_t batch, int64_t s, int64_t rows, int64_t ld, int64_t cols, int64_t *out) {
  int64_t a, b, c;
  if (!mul_ok(batch - 1, s, &a) || !mul_ok(rows - 1, ld, &b)) return false;
  if (!add_ok(a, b, &c) || !add_ok(c, cols, out)) return false;
  return true;
}

bool ranges_overlap(const void *p, int64_t pbytes, const void *q, int64_t qbytes) {
  const uintptr_t a = (uintptr_t)p, b = (uintptr_t)q;
  return a < b + (uintptr_t)qbytes && b < a + (uintptr_t)pbytes;
}

enum class Kernel {
  None, Masked8, MaskedU, Small8, SmallU, Tile32, Tile16, Tile16NN, TileW, TileWNN, Tile16TN, Tile16TT, TileWTT, Skinny,
  SplitK, TileST
};

const char *kernel_name(Kernel k, const Problem &p) {
  switch (k) {
    case Kernel::Masked8:
      return masked_name(8, 128);
    case Kernel::MaskedU:
      return masked_name(0, 128);
    case Kernel::Small8:
      return masked_name(8, 64);
    case Kernel::SmallU:
      return masked_name(0, 64);
    case Kernel::Tile32:
      return tile_name(0);
    case Kernel::Tile16:
      return tile_name(1);
    case Kernel::Tile16NN:
      return tile_name(2);
    case Kernel::TileW:
      return tile_name(3);
    case Kernel::TileWNN:
      return tile_name(4);
    case Kernel::Tile16TN:
      return tile_name(5);
    case Kernel::Tile16TT:
      return tile_name(6);
    case Kernel::TileWTT:
      return tile_name(7);
    case Kernel::TileST:
      return tile_name(8);
    case Kernel::Skinny:
      return skinny_name(p);
    case Kernel::SplitK:
      return splitk_name(p.b_col);
    default:
      return nullptr;
  }
}

struct Plan {
  Problem p;
  Kernel kernel = Kernel::None;
  bool forced = false;                      // TSM_GEMM_KERNEL named the kernel
  int64_t a_bytes = 0, b_bytes = 0, c_bytes = 0;  // operand extents (A and B only when K > 0)
  // Row bands (band_rows > 0): rows [0, band_rows) run on `kernel`, rows
  // [band_rows, M) as a problem of their own, `low` on `low_kernel`.
  int64_t band_rows = 0;
  Problem low;
  Kernel low_kernel = Kernel::None;
};

// Can an operand be read with 16-byte vectors along its contiguous dimension?
// Needs the base 16-byte aligned and the contiguous extent, the leading
// dimension and the batch stride all multiples of 8 elements.
bool vec8_ok(const void *X, int64_t contiguous_extent, int64_t ld, int64_t stride, int64_t batch) {
  if (((uintptr_t)X & 15) != 0) return false;
  if (contiguous_extent % 8 != 0 || ld % 8 != 0) return false;
  if (batch > 1 && stride % 8 != 0) return false;
  return true;
}

// rows: null for plain (batched) products; for grouped products the device
// array of per-problem row counts (each clamped to [0, M] by the kernels).
// act, slope: the epilogue activation (TSM_ACT_*) and the leaky-ReLU slope.
// One kernel for the whole problem; plan() below may then cut it in row bands.
int plan_one(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a, int64_t strideA, const void *B,
         int64_t ldb, int layout_b, int64_t strideB, void *C, int64_t ldc, int64_t strideC, int64_t batch, int dtype,
         const int32_t *rows, bool grouped, int act, float slope, Plan *out) {
  g_detail[0] = '\0';
  if (dtype < TSM_F16_F32 || dtype > TSM_BF16_BF16) return fail(TSM_ERROR_INVALID_VALUE, "unknown dtype %d", dtype);
  if (act != TSM_ACT_NONE && act != TSM_ACT_RELU && act != TSM_ACT_LEAKY_RELU)
    return fail(TSM_ERROR_INVALID_VALUE, "unknown activation %d", act);
  if (act == TSM_ACT_LEAKY_RELU && !__builtin_isfinite(slope))
    return fail(TSM_ERROR_INVALID_VALUE, "leaky ReLU slope is not finite");
  if (layout_a != TSM_ROW && layout_a != TSM_COL)
    return fail(TSM_ERROR_INVALID_VALUE, "unknown layout_a %d", layout_a);
  if (layout_b != TSM_ROW && layout_b != TSM_COL)
    return fail(TSM_ERROR_INVALID_VALUE, "unknown layout_b %d", layout_b);
  if (M < 0 || N < 0 || K < 0) return fail(TSM_ERROR_INVALID_VALUE, "negative size M=%lld N=%lld K=%lld",
                                           (long long)M, (long long)N, (long long)K);
  if (batch < 0) return fail(TSM_ERROR_INVALID_VALUE, "negative batch %lld", (long long)batch);

  *out = Plan{};
  Problem &p = out->p;
  p.A = (const uint16_t *)A;
  p.B = (const uint16_t *)B;
  p.C = C;
  p.M = M;
  p.N = N;
  p.K = K;
  p.lda = lda;
  p.ldb = ldb;
  p.ldc = ldc;
  p.sA = strideA;
  p.sB = strideB;
  p.sC = strideC;
  p.batch = batch;
  p.a_col = layout_a == TSM_COL;
  p.b_col = layout_b == TSM_COL;
  p.in_bf16 = dtype == TSM_BF16_F32 || dtype == TSM_BF16_F16 || dtype == TSM_BF16_BF16;
  p.out16 = dtype != TSM_F16_F32 && dtype != TSM_BF16_F32;
  p.out_bf16 = dtype == TSM_F16_BF16 || dtype == TSM_BF16_BF16;
  p.act = act;
  p.slope = act == TSM_ACT_LEAKY_RELU ? slope : 0.f;
  p.rows = rows;
  out->kernel = Kernel::None;

  if (M == 0 || N == 0 || batch == 0) return TSM_SUCCESS;  // nothing to compute
  if (grouped) {
    if (!rows) return fail(TSM_ERROR_INVALID_VALUE, "rows is NULL");
    if ((uintptr_t)rows % 4) return fail(TSM_ERROR_INVALID_VALUE, "rows not 4-byte aligned");
  }

  // ---- launch limits (tile indices and in-kernel loop counts stay in 32 bits)
  const int64_t kMaxDim = 0x7fffffffLL;
  if (M > kMaxDim || N > kMaxDim || K > kMaxDim)
    return fail(TSM_ERROR_NOT_SUPPORTED, "a dimension exceeds 2^31-1");

  // ---- C
  const int64_t csize = p.out16 ? 2 : 4;
  if (!C) return fail(TSM_ERROR_INVALID_VALUE, "C is NULL");
  if (((uintptr_t)C % (uintptr_t)csize) != 0)
    return fail(TSM_ERROR_INVALID_VALUE, "C not %lld-byte aligned", (long long)csize);
  if (ldc < (N > 1 ? N : 1)) return fail(TSM_ERROR_INVALID_VALUE, "ldc=%lld < N=%lld", (long long)ldc, (long long)N);
  if (batch > 1) {
    if (strideC < 0) return fail(TSM_ERROR_INVALID_VALUE, "negative strideC");
    int64_t span;
    if (!extent(1, 0, M, ldc, N, &span)) return fail(TSM_ERROR_NOT_SUPPORTED, "C extent overflows int64");
    if (strideC < span)
      return fail(TSM_ERROR_INVALID_VALUE, "strideC=%lld makes the outputs overlap (needs >= %lld)",
                  (long long)strideC, (long long)span);
  }
  int64_t c_elems, c_bytes;
  if (!extent(batch, strideC, M, ldc, N, &c_elems) || !mul_ok(c_elems, csize, &c_bytes))
    return fail(TSM_ERROR_NOT_SUPPORTED, "C extent overflows int64");
  out->c_bytes = c_bytes;

  // ---- A and B (only read when K > 0)
  if (K > 0) {
    if (!A) return fail(TSM_ERROR_INVALID_VALUE, "A is NULL");
    if (!B) return fail(TSM_ERROR_INVALID_VALUE, "B is NULL");
    if (((uintptr_t)A & 1) || ((uintptr_t)B & 1)) return fail(TSM_ERROR_INVALID_VALUE, "A or B not 2-byte aligned");
    const int64_t a_rows = p.a_col ? K : M, a_cols = p.a_col ? M : K;
    const int64_t b_rows = p.b_col ? N : K, b_cols = p.b_col ? K : N;
    if (lda < a_cols)
      return fail(TSM_ERROR_INVALID_VALUE, "lda=%lld < %lld", (long long)lda, (long long)a_cols);
    if (ldb < b_cols)
      return fail(TSM_ERROR_INVALID_VALUE, "ldb=%lld < %lld", (long long)ldb, (long long)b_cols);
    if (batch > 1 && (strideA < 0 || strideB < 0))
      return fail(TSM_ERROR_INVALID_VALUE, "negative strideA or strideB");
    int64_t a_elems, b_elems, a_bytes, b_bytes;
    if (!extent(batch, batch > 1 ? strideA : 0, a_rows, lda, a_cols, &a_elems) || !mul_ok(a_elems, 2, &a_bytes) ||
        !extent(batch, batch > 1 ? strideB : 0, b_rows, ldb, b_cols, &b_elems) || !mul_ok(b_elems, 2, &b_bytes))
      return fail(TSM_ERROR_NOT_SUPPORTED, "operand extent overflows int64");
    if (ranges_overlap(C, c_bytes, A, a_bytes)) return fail(TSM_ERROR_INVALID_VALUE, "C overlaps A");
    if (ranges_overlap(C, c_bytes, B, b_bytes)) return fail(TSM_ERROR_INVALID_VALUE, "C overlaps B");
    out->a_bytes = a_bytes;
    out->b_bytes = b_bytes;
  }
  if (batch == 1) {
    p.sA = p.sB = p.sC = 0;
  }

  // ---- kernel selection
  const int64_t tiles = ((M + MaskedInfo::BM - 1) / MaskedInfo::BM) * ((N + MaskedInfo::BN - 1) / MaskedInfo::BN);
  if (tiles * MaskedInfo::THREADS > 0xffffffffLL)
    return fail(TSM_ERROR_NOT_SUPPORTED, "tile grid too large (%lld tiles)", (long long)tiles);
  const bool a8 = K == 0 || vec8_ok(A, p.a_col ? M : K, lda, p.sA, batch);
  const bool b8 = K == 0 || vec8_ok(B, p.b_col ? K : N, ldb, p.sB, batch);
  out->kernel = (a8 && b8) ? Kernel::Masked8 : Kernel::MaskedU;
  const int64_t masked_tiles = tiles * batch;
  // fewer than 180 tiles of 128 x 128: 64 x 64 tiles, four times the
  // workgroups (1664 x 1664 x 2048, 169 tiles: 24.4 us against 28.3; 1792 x
  // 1792, 196 tiles: 29.2 against 28.4 at K = 2048, 100.9 against 92.8 at
  // K = 8192)
  if (masked_tiles < 180) out->kernel = (a8 && b8) ? Kernel::Small8 : Kernel::SmallU;
  // few output tiles and deep K: take the parallelism from K.  The 64 x 64
  // masked tiles walk K at a fixed pace per workgroup for any grid below the
  // CU count (about 36 us for K = 8192 with K-contiguous B, 40 us with
  // row-major B); split-K beats that up to 9 such tiles with K-contiguous B
  // (384 x 384 x 8192: 27 us against 36) and up to 4 with row-major B, whose
  // 16-column slices it reads as 32-byte rows (256 x 256 x 8192: 16 us
  // against 41; 384 x 384: 47 against 40)
  const bool splitk_ok = K > 0 && splitk_supports(p);
  if (splitk_ok && masked_tiles <= (p.b_col ? 9 : 4)) out->kernel = Kernel::SplitK;
  // The 256 x 256 kernels take about the same time per round of up to 256
  // tiles (one workgroup per CU) whatever the tile count.  They overtake the
  // masked kernels from 72 tiles (2560 x 2560, 100 tiles: 13.7 us against
  // 16.1 at K = 512; 2304 x 2304, 81 tiles: 22.1 against 24.4 at K = 1024,
  // 124.6 against 140.4 at K = 8192; 2048 x 2304, 72 tiles: 13.5 against
  // 15.4 for 128 x 128 tiles at K = 512, 124.9 against 132.1 at K = 8192); at
  // 64 tiles the masked kernels stay ahead (2048 x 2048 x 8192: 92.9 against
  // 124.7).
  const int64_t tiles256 =
      ((M + TileInfo::BM - 1) / TileInfo::BM) * ((N + TileInfo::BN - 1) / TileInfo::BN) * batch;
  const bool tile_ok = K > 0 && tiles256 >= 72;
  if (tile_ok && tile_supports(p, false, false)) out->kernel = Kernel::TileST;
  if (tile_ok && tile_supports(p, false, true)) out->kernel = Kernel::Tile16NN;
  if (tile_ok && tile_supports(p, true, true)) out->kernel = Kernel::Tile16TN;
  if (tile_ok && tile_supports(p, true, false)) out->kernel = Kernel::Tile16TT;
  // up to 128 rows: the streaming kernel reads B once, where split-K reads
  // it once per 16-row tile and the 256-row tiles waste most of their MFMA
  // work.  Its rate grows with its grid (about 6.7 TB/s at 256 workgroups,
  // one per CU); split-K's falls with the row tiles (about 3 TB/s over one).
  // Split-K keeps the problem while grid x row tiles < 128.
  // The streaming kernel runs whole rounds of its ring: with 33-128 rows and
  // fewer K slices than one round, the 64 x 64 masked tiles win (64 x 128 x
  // 128: 3.7 us against 4.2; 128 x 8192 x 256: 5.6 against 6.6); with up to
  // 32 rows it keeps them (16 x 16384 x 448: 4.2 against 6.2).
  if (K > 0) {
    const SkinnyPlan sp = skinny_plan(p);
    const bool narrow = sp.mb && (N / sp.w) * batch * ((M + 15) / 16) < 128;
    const bool short_k = sp.mb > 2 && K < 64 * (int64_t)skinny_ring_slices(sp);
    if (sp.mb && !short_k) out->kernel = narrow && splitk_ok && masked_tiles < 256 ? Kernel::SplitK : Kernel::Skinny;
  }

  // TSM_GEMM_KERNEL=<name> forces a kernel variant (tests and tuning); a
  // variant that cannot run this problem is an error, never a silent fallback.
  const char *force = getenv("TSM_GEMM_KERNEL");
  if (force && *force) {
    const Kernel all[] = {Kernel::Masked8,  Kernel::MaskedU,  Kernel::Small8,   Kernel::SmallU,  Kernel::Tile32,
                          Kernel::Tile16,   Kernel::Tile16NN, Kernel::TileW,    Kernel::TileWNN, Kernel::Tile16TN,
                          Kernel::Tile16TT, Kernel::TileWTT,  Kernel::Skinny,   Kernel::SplitK,  Kernel::TileST};
    Kernel want = Kernel::None;
    for (Kernel k : all)
      if (k != Kernel::Skinny && strcmp(force, kernel_name(k, p)) == 0) want = k;
    // a skinny name fixes the workgroup width (its row blocks follow from M)
    if (strncmp(force, "skinny_", 7) == 0) {
      want = Kernel::Skinny;
      const char *w = strstr(force, "_n");
      p.skinny_w = w ? atoi(w + 2) : -1;
      const char *nm = skinny_name(p);
      if (!nm || strcmp(nm, force) != 0)
        return fail(TSM_ERROR_NOT_SUPPORTED, "TSM_GEMM_KERNEL=%s cannot run this problem", force);
    }
    if (want == Kernel::None) return fail(TSM_ERROR_INVALID_VALUE, "TSM_GEMM_KERNEL=%s names no kernel", force);
    const bool ok = want == Kernel::MaskedU || want == Kernel::SmallU ||
                    ((want == Kernel::Masked8 || want == Kernel::Small8) && a8 && b8) ||
                    ((want == Kernel::Tile32 || want == Kernel::Tile16 || want == Kernel::TileW || want == Kernel::TileST) && K > 0 &&
                     tile_supports(p, false, false)) ||
                    ((want == Kernel::Tile16NN || want == Kernel::TileWNN) && K > 0 && tile_supports(p, false, true)) ||
                    (want == Kernel::Tile16TN && K > 0 && tile_supports(p, true, true)) ||
                    ((want == Kernel::Tile16TT || want == Kernel::TileWTT) && K > 0 && tile_supports(p, true, false)) ||
                    (want == Kernel::Skinny && K > 0 && skinny_supports(p)) ||
                    (want == Kernel::SplitK && K > 0 && splitk_supports(p));
    if (!ok) return fail(TSM_ERROR_NOT_SUPPORTED, "TSM_GEMM_KERNEL=%s cannot run this problem", force);
    out->kernel = want;
    out->forced = true;
  }
  // the masked kernels address each operand slice (32 or 64 deep) with
  // 32-bit offsets from its corner: up to 127 rows of a leading dimension
  const bool masked = out->kernel == Kernel::Masked8 || out->kernel == Kernel::MaskedU ||
                      out->kernel == Kernel::Small8 || out->kernel == Kernel::SmallU;
  if (masked && K > 0 && (lda >= MaskedInfo::kMaxLd || ldb >= MaskedInfo::kMaxLd))
    return fail(TSM_ERROR_NOT_SUPPORTED, "lda=%lld or ldb=%lld >= %lld on the general kernel", (long long)lda,
                (long long)ldb, (long long)MaskedInfo::kMaxLd);
  return TSM_SUCCESS;
}

// CUs of the current device (looked up once per device).
int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n > 0) return n;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) n = 256;
  cache[dev].store(n, std::memory_order_relaxed);
  return n;
}

bool is_tile256(Kernel k) {
  return k == Kernel::TileST || k == Kernel::Tile16NN || k == Kernel::Tile16TN || k == Kernel::Tile16TT;
}

// Row bands for one plain product a little over whole rounds of 256 x 256
// tiles (a round: one tile per CU).  The large-tile kernel takes about as long
// over a last round of 16 tiles as over a full one, each workgroup's time being
// one tile's K loop.  The rows past the whole rounds run better as a problem
// of their own, after the whole rounds, when its kernel spreads them over every
// CU in smaller tiles.  Measured with bf16 operands (K = 2048-8192; N = 4096
// with 4096 rows plus 64-1792, N = 3072, 8192 and 16384): bottom rows that go
// to the streaming kernel, to 64 x 64 tiles or to one round of 128 x 128 tiles
// gain 4-32% (4352 x 4096 x 8192: 235 us against 308; 5120 x 4096 x 8192: 295
// against 311); a bottom that needs a second round of 128 x 128 tiles or the
// large-tile kernel loses 1-9%, so those keep one kernel.  The bands are
// disjoint rows of C, each computed by its kernel alone.
int plan(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a, int64_t strideA, const void *B,
         int64_t ldb, int layout_b, int64_t strideB, void *C, int64_t ldc, int64_t strideC, int64_t batch, int dtype,
         const int32_t *rows, bool grouped, int act, float slope, Plan *out) {
  const int st = plan_one(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC, batch,
                          dtype, rows, grouped, act, slope, out);
  if (st != TSM_SUCCESS || out->forced || !is_tile256(out->kernel) || batch != 1 || grouped) return st;
  const Problem &p = out->p;
  const int64_t tn = (N + TileInfo::BN - 1) / TileInfo::BN;
  const int64_t T = ((M + TileInfo::BM - 1) / TileInfo::BM) * tn;
  const int64_t P = device_cus();
  if (T <= P || T % P == 0) return st;
  // the tile rows that fill the whole rounds (up to a row's tiles short of
  // them when N's tile count does not divide the CU count)
  const int64_t top = T / P * P / tn * TileInfo::BM;
  if (top <= 0 || top >= M) return st;
  Plan low;
  const int64_t es = p.out16 ? 2 : 4;
  const int ls = plan_one(M - top, N, K, p.A + top * (p.a_col ? 1 : lda), lda, layout_a, 0, B, ldb, layout_b, 0,
                          (char *)C + top * ldc * es, ldc, 0, 1, dtype, nullptr, false, act, slope, &low);
  g_detail[0] = '\0';
  if (ls != TSM_SUCCESS) return st;
  const Kernel k = low.kernel;
  bool ok = k == Kernel::Skinny || k == Kernel::SplitK || k == Kernel::Small8 || k == Kernel::SmallU;
  if (k == Kernel::Masked8 || k == Kernel::MaskedU)
    ok = ((M - top + MaskedInfo::BM - 1) / MaskedInfo::BM) * ((N + MaskedInfo::BN - 1) / MaskedInfo::BN) <= P;
  if (!ok) return st;
  out->band_rows = top;
  out->low = low.p;
  out->low_kernel = k;
  return st;
}

hipError_t launch(Kernel k, const Problem &p, hipStream_t s) {
  switch (k) {
    case Kernel::None:
      return hipSuccess;
    case Kernel::Masked8:
      return launch_masked(p, 8, 128, s);
    case Kernel::MaskedU:
      return launch_masked(p, 0, 128, s);
    case Kernel::Small8:
      return launch_masked(p, 8, 64, s);
    case Kernel::SmallU:
      return launch_masked(p, 0, 64, s);
    case Kernel::Tile32:
      return launch_tile(p, 0, s);
    case Kernel::Tile16:
      return launch_tile(p, 1, s);
    case Kernel::Tile16NN:
      return launch_tile(p, 2, s);
    case Kernel::TileW:
      return launch_tile(p, 3, s);
    case Kernel::TileWNN:
      return launch_tile(p, 4, s);
    case Kernel::Tile16TN:
      return launch_tile(p, 5, s);
    case Kernel::Tile16TT:
      return launch_tile(p, 6, s);
    case Kernel::TileWTT:
      return launch_tile(p, 7, s);
    case Kernel::TileST:
      return launch_tile(p, 8, s);
    case Kernel::Skinny:
      return launch_skinny(p, s);
    case Kernel::SplitK:
      return launch_splitk(p, s);
  }
  return hipSuccess;
}

int run(const Plan &pl, void *stream) {
  const hipStream_t s = (hipStream_t)stream;
  hipError_t e;
  if (pl.band_rows) {
    Problem top = pl.p;
    top.M = pl.band_rows;
    e = launch(pl.kernel, top, s);
    if (e == hipSuccess) e = launch(pl.low_kernel, pl.low, s);
  } else {
    e = launch(pl.kernel, pl.p, s);
  }
  if (e != hipSuccess) return fail(TSM_ERROR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return TSM_SUCCESS;
}

// What a plan launches: one kernel's name, or "band_<top>+<bottom>" for row
// bands (composed names are kept until the process ends, so every returned
// string stays valid).
const char *plan_name(const Plan &pl) {
  const char *top = kernel_name(pl.kernel, pl.p);
  if (!pl.band_rows || !top) return top;
  const char *low = kernel_name(pl.low_kernel, pl.low);
  if (!low) return nullptr;
  static std::mutex mu;
  static std::set<std::string> names;
  std::lock_guard<std::mutex> lock(mu);
  return names.insert(std::string("band_") + top + "+" + low).first->c_str();
}

// Is stream-K requested (TSM_GEMM_SPLIT=streamk)?  Measured on MI355X it
// loses to the plain kernel for 144-224 tiles of 256 x 256 and to the tile
// split below (its runs meet the tiles at staggered K, which defeats the L2
// sharing of operand panels, and its partial tiles cost a float32 round trip
// through HBM), so it runs only on request.
bool streamk_requested() {
  const char *force = getenv("TSM_GEMM_SPLIT");
  return force && strcmp(force, "streamk") == 0;
}

// The K split a planned problem takes given enough workspace (none: splits == 0).
// TSM_GEMM_SPLIT=none keeps the kernel that needs no workspace, =streamk
// takes stream-K wherever the problem allows it, =hybrid the hybrid over row
// bands (tests and tuning).
KSplit split_of(const Plan &pl) {
  if (pl.kernel == Kernel::None || pl.forced) return KSplit{};
  // The in-workgroup split with a K-contiguous B over at most 4 tiles of
  // 128 x 128 beats the workspace split at every K measured (256 x 256 x 2048:
  // 5.4 us against 8.8; x 8192: 8.4 against 9.2); from 9 tiles the workspace
  // split wins (384 x 384 x 4096: 12.1 against 13.8).
  const int64_t tiles128 =
      ((pl.p.M + MaskedInfo::BM - 1) / MaskedInfo::BM) * ((pl.p.N + MaskedInfo::BN - 1) / MaskedInfo::BN) * pl.p.batch;
  if (pl.kernel == Kernel::SplitK && pl.p.b_col && tiles128 <= 4) return KSplit{};
  KSplit k = ksplit_plan(pl.p);
  if (k.splits) return k;
  const char *force = getenv("TSM_GEMM_SPLIT");
  if (force && strcmp(force, "none") == 0) return KSplit{};
  if (streamk_requested()) return sk_plan(pl.p, device_cus());
  k = tsplit_plan(pl.p);
  if (k.splits) return k;
  // Row bands (no workspace) beat the hybrid up to K = 4096, and while at most
  // 64 rows lie past the whole rounds (4096 columns, bf16: 4352 x 4096 x 2048
  // 69 us against 78; x 4096: 121 against 124; 4160 x 4096 x 8192: 208 against
  // 218).  From K = 6144 the hybrid wins for more rows (4352 x 4096 x 8192: 219
  // against 230; 5120 x 4096 x 6144: 192 against 217).  TSM_GEMM_SPLIT=hybrid
  // takes the hybrid wherever it applies (tests and tuning).
  const bool want_hybrid = force && strcmp(force, "hybrid") == 0;
  if (pl.band_rows && !want_hybrid && (pl.p.K <= 4096 || pl.p.M - pl.band_rows <= 64)) return KSplit{};
  // a little over whole rounds of 256 x 256 tiles: the hybrid, on the large-tile
  // kernel the plan chose for the whole rounds
  const int dp_variant = pl.kernel == Kernel::TileST     ? 8
                         : pl.kernel == Kernel::Tile16NN ? 2
                         : pl.kernel == Kernel::Tile16TN ? 5
                         : pl.kernel == Kernel::Tile16TT ? 6
                                                         : -1;
  return dp_variant >= 0 ? hybrid_plan(pl.p, device_cus(), dp_variant) : KSplit{};
}
int64_t split_bytes(const Plan &pl, const KSplit &k) {
  if (k.dp_tiles) return hybrid_workspace_bytes(k);
  return k.sk_runs ? sk_workspace_bytes(k.sk_runs) : pl.p.batch * k.splits * pl.p.M * pl.p.N * 4;
}

// ---- static scratch (gemm_strided_batched_noalloc) -----------------------------
// The partial sums of a K split, for callers that cannot allocate: one array
// per GPU, held from the library's load until the process ends.  Calls on one
// GPU share it, so calls that overlap on one GPU (two streams, or two host
// threads) race on it.  The split needs no zeroed memory: pass 1 writes every
// partial it reads back in pass 2.
constexpr int64_t kScratchBytes = (int64_t)64 << 20;
static __device__ __align__(256) char scratch[kScratchBytes];

// Device address of `scratch` on device `dev`, looked up once per device with
// that device current (the name `scratch` on the host is a stand-in, not a
// device address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

int scratch_of(hipStream_t stream, void **out) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return fail(TSM_ERROR_LAUNCH, "cannot tell the stream's device: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return fail(TSM_ERROR_NOT_SUPPORTED, "device %d beyond the scratch table", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e == hipSuccess && cur != dev) e = hipSetDevice(dev);
    void *p = nullptr;
    if (e == hipSuccess) e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess || !p)
      return fail(TSM_ERROR_LAUNCH, "no address for the static scratch on device %d: %s", dev, hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return TSM_SUCCESS;
}

// Workspace of a K-split call: validated on the host; `ks` gets the split to
// run (none when the problem does not split, the workspace is too small, or
// a kernel is forced).
int ws_check(const Plan &pl, const void *ws, int64_t ws_bytes, KSplit *ks) {
  *ks = KSplit{};
  if (ws_bytes < 0) return fail(TSM_ERROR_INVALID_VALUE, "negative workspace_bytes");
  if (!ws && ws_bytes > 0) return fail(TSM_ERROR_INVALID_VALUE, "workspace is NULL with workspace_bytes > 0");
  if (!ws || pl.kernel == Kernel::None || pl.forced) return TSM_SUCCESS;
  if ((uintptr_t)ws & 15) return fail(TSM_ERROR_INVALID_VALUE, "workspace not 16-byte aligned");
  if (ranges_overlap(ws, ws_bytes, pl.p.C, pl.c_bytes)) return fail(TSM_ERROR_INVALID_VALUE, "workspace overlaps C");
  if (ranges_overlap(ws, ws_bytes, pl.p.A, pl.a_bytes)) return fail(TSM_ERROR_INVALID_VALUE, "workspace overlaps A");
  if (ranges_overlap(ws, ws_bytes, pl.p.B, pl.b_bytes)) return fail(TSM_ERROR_INVALID_VALUE, "workspace overlaps B");
  const KSplit k = split_of(pl);
  if (!k.splits || split_bytes(pl, k) > ws_bytes) return TSM_SUCCESS;
  *ks = k;
  return TSM_SUCCESS;
}

int run_ws(const Plan &pl, const KSplit &ks, void *ws, void *stream) {
  if (!ks.splits) return run(pl, stream);
  const hipError_t e = launch_ksplit(pl.p, ks, (float *)ws, (hipStream_t)stream);
  if (e != hipSuccess) return fail(TSM_ERROR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return TSM_SUCCESS;
}

// Host checks of a row-sum call; on success `a` is filled (a.R == 0: nothing to do).
int rowsum_check(int64_t R, int64_t C, const void *X, int64_t row_stride, int64_t col_stride, int xdtype,
                 const float *out, RowsumArgs *a) {
  g_detail[0] = '\0';
  if (xdtype != TSM_ROWSUM_F32 && xdtype != TSM_ROWSUM_F16 && xdtype != TSM_ROWSUM_BF16)
    return fail(TSM_ERROR_INVALID_VALUE, "unknown xdtype %d", xdtype);
  if (R < 0 || C < 0) return fail(TSM_ERROR_INVALID_VALUE, "negative size R=%lld C=%lld", (long long)R, (long long)C);
  if (row_stride < 0 || col_stride < 0) return fail(TSM_ERROR_INVALID_VALUE, "negative stride");
  *a = RowsumArgs{X, (float *)out, R, C, 0, row_stride, col_stride,
                  xdtype == TSM_ROWSUM_F32 ? (int)RowsumInfo::F32
                                           : xdtype == TSM_ROWSUM_F16 ? (int)RowsumInfo::F16 : (int)RowsumInfo::BF16};
  if (R == 0) return TSM_SUCCESS;
  if (R > 0x7fffffffLL) return fail(TSM_ERROR_NOT_SUPPORTED, "R exceeds 2^31-1");
  if (!out) return fail(TSM_ERROR_INVALID_VALUE, "out is NULL");
  if ((uintptr_t)out % 4) return fail(TSM_ERROR_INVALID_VALUE, "out not 4-byte aligned");
  if (C == 0) return TSM_SUCCESS;  // empty sums: out := 0
  const int64_t es = xdtype == TSM_ROWSUM_F32 ? 4 : 2;
  if (!X) return fail(TSM_ERROR_INVALID_VALUE, "X is NULL");
  if ((uintptr_t)X % (uintptr_t)es) return fail(TSM_ERROR_INVALID_VALUE, "X not %lld-byte aligned", (long long)es);
  int64_t a1, a2, span, bytes;
  if (!mul_ok(R - 1, row_stride, &a1) || !mul_ok(C - 1, col_stride, &a2) || !add_ok(a1, a2, &span) ||
      !add_ok(span, 1, &span) || !mul_ok(span, es, &bytes))
    return fail(TSM_ERROR_NOT_SUPPORTED, "X extent overflows int64");
  if (ranges_overlap(out, R * 4, X, bytes)) return fail(TSM_ERROR_INVALID_VALUE, "out overlaps X");
  return TSM_SUCCESS;
}

}  // namespace
}  // namespace tsm

extern "C" {

int rowsum(int64_t R, int64_t C, const void *X, int64_t row_stride, int64_t col_stride, int xdtype, float *out,
           void *stream) {
  tsm::RowsumArgs a;
  const int st = tsm::rowsum_check(R, C, X, row_stride, col_stride, xdtype, out, &a);
  if (st != TSM_SUCCESS || R == 0) return st;
  const hipError_t e = tsm::launch_rowsum(a, (hipStream_t)stream);
  if (e != hipSuccess) return tsm::fail(TSM_ERROR_LAUNCH, "launch failed: %s", hipGetErrorString(e));
  return TSM_SUCCESS;
}

const char *tsm_rowsum_kernel_name(int64_t R, int64_t C, const void *X, int64_t row_stride, int64_t col_stride,
                                   int xdtype, const float *out) {
  tsm::RowsumArgs a;
  if (tsm::rowsum_check(R, C, X, row_stride, col_stride, xdtype, out, &a) != TSM_SUCCESS || R == 0) return nullptr;
  return tsm::rowsum_name(a);
}

int gemm_strided_batched_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a,
                            int64_t strideA, const void *B, int64_t ldb, int layout_b, int64_t strideB, void *C,
                            int64_t ldc, int64_t strideC, int64_t batch, int dtype, void *stream) {
  tsm::Plan pl;
  int st = tsm::plan(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC, batch, dtype,
                     nullptr, false, TSM_ACT_NONE, 0.f, &pl);
  if (st != TSM_SUCCESS) return st;
  return tsm::run(pl, stream);
}

int gemm_strided_batched_act(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a,
                             int64_t strideA, const void *B, int64_t ldb, int layout_b, int64_t strideB, void *C,
                             int64_t ldc, int64_t strideC, int64_t batch, int dtype, int activation, float slope,
                             void *stream) {
  tsm::Plan pl;
  int st = tsm::plan(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC, batch, dtype,
                     nullptr, false, activation, slope, &pl);
  if (st != TSM_SUCCESS) return st;
  return tsm::run(pl, stream);
}

int64_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int64_t batch) {
  // the largest need over the splits a problem of this shape may take
  int64_t most = 0;
  const tsm::KSplit cand[3] = {tsm::ksplit_shape(M, N, K, batch, true), tsm::ksplit_shape(M, N, K, batch, false),
                               tsm::tsplit_shape(M, N, K, batch)};
  for (const tsm::KSplit &ks : cand)
    if (ks.splits && batch * ks.splits * M * N * 4 > most) most = batch * ks.splits * M * N * 4;
  const tsm::KSplit hy = tsm::hybrid_shape(M, N, K, batch, tsm::device_cus());
  if (hy.splits && tsm::hybrid_workspace_bytes(hy) > most) most = tsm::hybrid_workspace_bytes(hy);
  if (tsm::streamk_requested()) {
    const tsm::KSplit sk = tsm::sk_shape(M, N, K, batch, tsm::device_cus());
    if (sk.sk_runs && tsm::sk_workspace_bytes(sk.sk_runs) > most) most = tsm::sk_workspace_bytes(sk.sk_runs);
  }
  return most;
}

int gemm_strided_batched_ws(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a,
                            int64_t strideA, const void *B, int64_t ldb, int layout_b, int64_t strideB, void *C,
                            int64_t ldc, int64_t strideC, int64_t batch, int dtype, int activation, float slope,
                            void *workspace, int64_t workspace_bytes, void *stream) {
  tsm::Plan pl;
  int st = tsm::plan(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC, batch, dtype,
                     nullptr, false, activation, slope, &pl);
  if (st != TSM_SUCCESS) return st;
  tsm::KSplit ks;
  st = tsm::ws_check(pl, workspace, workspace_bytes, &ks);
  if (st != TSM_SUCCESS) return st;
  return tsm::run_ws(pl, ks, workspace, stream);
}

const char *tsm_gemm_ws_kernel_name(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a,
                                    int64_t strideA, const void *B, int64_t ldb, int layout_b, int64_t strideB,
                                    void *C, int64_t ldc, int64_t strideC, int64_t batch, int dtype,
                                    const void *workspace, int64_t workspace_bytes) {
  tsm::Plan pl;
  if (tsm::plan(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC, batch, dtype, nullptr,
                false, TSM_ACT_NONE, 0.f, &pl) != TSM_SUCCESS)
    return nullptr;
  tsm::KSplit ks;
  if (tsm::ws_check(pl, workspace, workspace_bytes, &ks) != TSM_SUCCESS) return nullptr;
  return ks.splits ? tsm::ksplit_name(ks, pl.p.b_col) : tsm::plan_name(pl);
}

int gemm_strided_batched_noalloc(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a,
                                 int64_t strideA, const void *B, int64_t ldb, int layout_b, int64_t strideB, void *C,
                                 int64_t ldc, int64_t strideC, int64_t batch, int dtype, int activation, float slope,
                                 void *stream) {
  tsm::Plan pl;
  int st = tsm::plan(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC, batch, dtype,
                     nullptr, false, activation, slope, &pl);
  if (st != TSM_SUCCESS) return st;
  const tsm::KSplit ks = tsm::split_of(pl);
  if (!ks.splits) return tsm::run(pl, stream);
  const int64_t need = tsm::split_bytes(pl, ks);
  if (need > tsm::kScratchBytes)
    return tsm::fail(TSM_ERROR_NOT_SUPPORTED,
                     "the K split needs %lld bytes of scratch, the static scratch holds %lld (call "
                     "gemm_strided_batched_ws with a workspace)",
                     (long long)need, (long long)tsm::kScratchBytes);
  void *ws = nullptr;
  st = tsm::scratch_of((hipStream_t)stream, &ws);
  if (st != TSM_SUCCESS) return st;
  return tsm::run_ws(pl, ks, ws, stream);
}

int64_t gemm_noalloc_scratch_bytes(void) { return tsm::kScratchBytes; }

int gemm_grouped(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a, int64_t strideA,
                 const void *B, int64_t ldb, int layout_b, int64_t strideB, void *C, int64_t ldc, int64_t strideC,
                 const int32_t *rows, int64_t groups, int dtype, void *stream) {
  tsm::Plan pl;
  int st = tsm::plan(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC, groups, dtype,
                     rows, true, TSM_ACT_NONE, 0.f, &pl);
  if (st != TSM_SUCCESS) return st;
  return tsm::run(pl, stream);
}

int gemm_strided_batched(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int64_t strideA,
                         const void *B, int64_t ldb, int64_t strideB, void *C, int64_t ldc, int64_t strideC,
                         int64_t batch, int dtype, void *stream) {
  return gemm_strided_batched_ex(M, N, K, A, lda, TSM_ROW, strideA, B, ldb, TSM_ROW, strideB, C, ldc, strideC, batch,
                                 dtype, stream);
}

int gemm_ex(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a, const void *B, int64_t ldb,
            int layout_b, void *C, int64_t ldc, int dtype, void *stream) {
  return gemm_strided_batched_ex(M, N, K, A, lda, layout_a, 0, B, ldb, layout_b, 0, C, ldc, 0, 1, dtype, stream);
}

int gemm(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, const void *B, int64_t ldb, void *C,
         int64_t ldc, int dtype, void *stream) {
  return gemm_strided_batched_ex(M, N, K, A, lda, TSM_ROW, 0, B, ldb, TSM_ROW, 0, C, ldc, 0, 1, dtype, stream);
}

const char *tsm_status_string(int status) {
  switch (status) {
    case TSM_SUCCESS:
      return "success";
    case TSM_ERROR_INVALID_VALUE:
      return "invalid value";
    case TSM_ERROR_NOT_SUPPORTED:
      return "not supported";
    case TSM_ERROR_LAUNCH:
      return "launch failure";
    default:
      return "unknown status";
  }
}

const char *tsm_last_error_detail(void) { return tsm::g_detail; }

const char *tsm_gemm_kernel_name(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a,
                                 int64_t strideA, const void *B, int64_t ldb, int layout_b, int64_t strideB, void *C,
                                 int64_t ldc, int64_t strideC, int64_t batch, int dtype) {
  tsm::Plan pl;
  if (tsm::plan(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC, batch, dtype, nullptr,
                false, TSM_ACT_NONE, 0.f, &pl) != TSM_SUCCESS)
    return nullptr;
  return tsm::plan_name(pl);
}

const char *tsm_gemm_grouped_kernel_name(int64_t M, int64_t N, int64_t K, const void *A, int64_t lda, int layout_a,
                                         int64_t strideA, const void *B, int64_t ldb, int layout_b, int64_t strideB,
                                         void *C, int64_t ldc, int64_t strideC, const int32_t *rows, int64_t groups,
                                         int dtype) {
  tsm::Plan pl;
  if (tsm::plan(M, N, K, A, lda, layout_a, strideA, B, ldb, layout_b, strideB, C, ldc, strideC, groups, dtype, rows,
                true, TSM_ACT_NONE, 0.f, &pl) != TSM_SUCCESS)
    return nullptr;
  return tsm::kernel_name(pl.kernel, pl.p);
}

}  // extern "C"
