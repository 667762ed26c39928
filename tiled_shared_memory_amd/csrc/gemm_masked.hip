// Masked, register-staged LDS GEMM kernel for gfx950: the general path.
//
// It handles every layout, every alignment and ragged M, N and K.  Each
// 256-thread workgroup owns a T x T tile of C (T = 128, or 64 when the
// 128-tile grid is too small to occupy the chip) and walks K in slices of
// BK = 32 (T = 128) or 64 (T = 64) ("The PTSS Cliff", section "The Idea:
// Stage in SLM, Tile K": only a bounded K slice is live, the float32
// accumulator is carried across the loop).  Unlike the page's pass, which
// stages whole operands once, the slices are streamed: at large K a whole
// operand panel cannot fit LDS, so registers hold the next slices in flight
// while the current one, in LDS, feeds the matrix cores (double-buffered LDS,
// one barrier per slice).  Tiles are regrouped per XCD and walked in groups of
// 8 tile rows; a strided batch or grouped call is one 1-D grid.
//
// Loads: each thread fetches vectors of 8 contiguous 16-bit elements of an
// operand along its contiguous dimension.  VEC = 8: one 16-byte load, when the
// base, the leading dimension, the batch stride and the contiguous extent
// allow it.  Otherwise (any 2-byte alignment, e.g. rows of 777 elements) one
// dword-aligned 16-byte load and one 4-byte load cover the vector; one byte
// permute per dword realigns it and, in K's last slice, clears the elements
// past K; an operand whose vectors all start on a dword skips the 4-byte load
// (and, contiguous along M or N, the permute).  Elements outside M, N or K read
// as zero in both
// operands: "A Dumb Triton Runtime Error", Step 2 on masked loads, where the
// padding must be the additive identity (a -inf or garbage pad would poison the
// sum); the masked K loop of the Intel XPU Triton README ("Use Tensor
// Descriptors ...", the pointer-based loop) zero-fills the same way.
//
// LDS layout: an operand contiguous along K is stored as it comes, [outer][BK
// + 8] 16-bit elements (row pitch 80 or 144 bytes, so every 16-byte fragment
// read stays aligned and the rows one 16-lane group reads fall on distinct
// banks).  An operand
// contiguous along M or N (row-major B, column-major A) is also stored as it
// comes, [BK][T] with its 16-byte chunks XOR-swizzled by the k row, and
// ds_read_b64_tr_b16 transposes it on the way out of LDS into the
// 8-consecutive-k fragments of v_mfma_f32_32x32x16.
//
// Compute: 4 waves in a 2 x 2 grid, each owning (T/2) x (T/2) of the tile as
// blocks of v_mfma_f32_32x32x16 (2 x 2 blocks, 64 accumulator registers per
// lane, for T = 128; one block for T = 64): fixed by the tile, never by K.
//
// Epilogue: masked stores of rows < M and columns < N, float32 or f16 (round to
// nearest even); C's padding beyond N is never touched.
#include "gemm_internal.hpp"
#include "mfma.hpp"

namespace tsm {
namespace {

constexpr uint32_t kOutside = 0x80000000u;  // a per-lane offset past every buffer resource
constexpr int THREADS = MaskedInfo::THREADS;
// K slice depth: 32 for 128-tiles, 64 for 64-tiles (whose waves have one
// 32 x 32 block each: a deeper slice gives them twice the matrix-core work per
// barrier).
template <int T>
constexpr int bk() {
  return T == 64 ? 64 : 32;
}
// LDS row pitch of a K-contiguous tile, in 16-bit elements (80 or 144 bytes:
// 16-byte aligned, and the 16 rows one 16-lane group reads fall on distinct
// banks)
template <int T>
constexpr int pitch() {
  return bk<T>() + 8;
}

typedef short v4s __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4s lds_v4s;
typedef __attribute__((address_space(3))) char lds_char;

// Byte offset of element (k, o) in a [BK][T] tile contiguous along o.  The
// 16-byte chunk index is XORed with the row: the transposing reads of one
// half-wave cover 4 rows x 64 bytes, which then fall on 64 distinct banks
// (rows of 128 bytes sit 32 banks apart, rows of 256 bytes on the same ones).
template <int T>
__device__ __forceinline__ int omaj_off(int k, int o) {
  constexpr int SW = T == 64 ? 2 : 4;
  return k * (T * 2) + (((o >> 3) ^ (SW * (k & 3))) << 4) + (o & 7) * 2;
}

// ds_read_b64_tr_b16: within each 16-lane group, lane j gives the address of
// 4 elements (row j / 4 of a 4 x 16 block) and receives column j of the block.
__device__ __forceinline__ u32x2 read_tr(const char *p) {
  return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s *)(lds_char *)p));
}

// The 32x32x16 operand of block column cb from a [BK][T] tile: lane holds
// k = 16 ks + 8 (lane / 32) .. +7 of column cb + lane % 32, read as two 4-row
// transposes.
template <int T>
__device__ __forceinline__ u32x4 read_omaj(const uint16_t *s, int cb, int ks, int lane) {
  const int o = cb + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const int k = ks * 16 + 8 * (lane >> 5) + ((lane & 15) >> 2);
  const u32x2 lo = read_tr(reinterpret_cast<const char *>(s) + omaj_off<T>(k, o));
  const u32x2 hi = read_tr(reinterpret_cast<const char *>(s) + omaj_off<T>(k + 4, o));
  return u32x4{lo[0], lo[1], hi[0], hi[1]};
}

// Load modes (VEC): 8 = 16-byte loads of both operands; 0-3 = realigning
// loads, where bit 0 (A) and bit 1 (B) mark an even operand: its leading
// dimension and batch stride are even and its base lies on a dword, so every
// vector starts on a dword and needs no fifth dword; one contiguous along M or
// N then needs no byte permute either.
template <int VEC>
constexpr bool realigning() {
  return VEC != 8;
}

// Slices in flight in registers (even: the LDS buffers alternate): 4 x 32 k
// on 128-tiles, 2 x 64 k on 64-tiles (the same k distance ahead).
template <int T, int VEC>
constexpr int depth() {
  return T == 64 ? 2 : 4;
}

// Staging registers for one operand tile (T x BK elements): 8-element vectors,
// and with realigning loads the dword after each 16-byte load.
template <int T, int VEC>
struct Stage {
  static constexpr int kLoads = (T * bk<T>()) / (THREADS * 8);  // vectors per thread
  u32x4 v[kLoads];
  uint32_t tail[realigning<VEC>() ? kLoads : 1];
};

// One operand of one tile, fixed for the whole K loop.
struct Src {
  const uint16_t *base;  // element (o0, k = 0) of the tile, one element lower when that sits at 2 mod 4 bytes
  int64_t ld;
  int64_t rest;          // elements from base to the operand's last element + 1 (realigning loads)
  int o_left;            // rows (outer) of the tile inside the matrix, at most T
  uint32_t delta;        // 1 when base was moved down one element
};

// Slice k0 of a tile starts k0 (KMAJ) or k0 * ld (outer contiguous) elements
// after the tile's corner: an even count (k0 is a multiple of BK), so the
// corner's alignment, and delta, hold for every slice.
template <int T, bool KMAJ, int VEC>
__device__ __forceinline__ Src make_src(const uint16_t *X, int64_t ld, int64_t outer_total, int64_t K, int64_t o0) {
  const int64_t at = KMAJ ? o0 * ld : o0;
  const uint16_t *p = X + at;
  const uint32_t delta = realigning<VEC>() ? (uint32_t)(((uintptr_t)p >> 1) & 1) : 0u;
  // the operand's storage ends after row outer_total - 1 (K contiguous) or k row K - 1
  const int64_t end = KMAJ ? (outer_total - 1) * ld + K : (K - 1) * ld + outer_total;
  return Src{p - delta, ld, end - at + delta, (int)(outer_total - o0 < T ? outer_total - o0 : T), delta};
}

// Thread tid's first vector of a slice: (o_t, k_t .. +7) when K is the
// contiguous dimension, (o_t .. +7, k_t) otherwise.  Its offset from the
// slice's corner advances by an even number of elements per vector.
template <int T, bool KMAJ>
__device__ __forceinline__ void first_vector(int tid, int &o_t, int &k_t) {
  constexpr int PER_ROW = KMAJ ? bk<T>() / 8 : T / 8;  // vectors per row of the contiguous dimension
  const int row_t = tid / PER_ROW, col_t = (tid % PER_ROW) * 8;
  o_t = KMAJ ? row_t : col_t;
  k_t = KMAJ ? col_t : row_t;
}

// Realigning loads: byte selectors of v_perm_b32 that turn a thread's five loaded
// dwords into its 8 elements.  The realignment (by 0 or 2 bytes) is the
// element offset's parity, the same for all of the thread's vectors and
// slices.  Elements past K would multiply real sums (they are the next row's
// first elements), so in K's last slice a K-contiguous operand's selectors
// also zero them (selector byte 0x0c reads as zero).  Elements past M or N need
// no clearing: they only reach rows or columns of the tile that are never
// stored.  One v_perm_b32 per dword replaces the funnel shift, the mask and
// the mask's selects.
struct Realign {
  uint32_t sel;      // every slice but K's last
  uint32_t last[4];  // K's last slice, per dword of the vector
};

template <int T, bool KMAJ>
__device__ __forceinline__ Realign make_realign(const Src &src, int64_t K, int tid) {
  int o_t, k_t;
  first_vector<T, KMAJ>(tid, o_t, k_t);
  const uint32_t ld = (uint32_t)src.ld;
  const uint32_t off = (KMAJ ? (uint32_t)o_t * ld + (uint32_t)k_t : (uint32_t)k_t * ld + (uint32_t)o_t) + src.delta;
  Realign r;
  // bytes 2..5 of {hi, lo} when the vector starts 2 bytes into its first dword
  r.sel = (off & 1u) ? 0x05040302u : 0x03020100u;
#pragma unroll
  for (int j = 0; j < 4; ++j) r.last[j] = r.sel;
  if constexpr (KMAJ) {
    constexpr int BK = bk<T>();
    const int64_t nk = (K + BK - 1) / BK;
    const int valid = (int)(K - (nk - 1) * BK) - k_t;  // the vector's elements below K in the last slice
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t keep = valid >= 2 * j + 2 ? 0xffffffffu : (valid == 2 * j + 1 ? 0x0000ffffu : 0u);
      r.last[j] = (r.sel & keep) | (0x0c0c0c0cu & ~keep);
    }
  }
  return r;
}

// Fetch the OUTER x BK slice starting at (o0, k0) of an operand.
//   KMAJ: element (o, k) at X[o*ld + k]   (K contiguous)
//  !KMAJ: element (o, k) at X[k*ld + o]   (outer contiguous)
// Buffer loads relative to the slice's corner, with 32-bit offsets (the host
// keeps a slice's span below 2^31 bytes): elements outside the matrix get an
// offset with bit 31 set, past the buffer resource, and load as zero without a
// branch.
template <int T, bool KMAJ, int VEC, bool EVEN>
__device__ __forceinline__ void fetch(Stage<T, VEC> &st, const Src &src, int64_t K, int64_t k0, int tid) {
  constexpr int BK = bk<T>();
  const int64_t koff = KMAJ ? k0 : k0 * src.ld;
  // Realigning loads: the resource starts at the dword holding the slice's corner and
  // ends at the dword holding the operand's last element, so the dwords a
  // vector's cover reads past that end load as zero instead of touching
  // memory (the range check is per dword).  Every dword inside lies in a page
  // the operand uses.
  int64_t records = 0x7fffffff;
  if constexpr (realigning<VEC>()) {
    const int64_t bytes = ((src.rest - koff) * 2 + 3) & ~(int64_t)3;
    records = bytes < 0 ? 0 : (bytes > 0x7fffffff ? 0x7fffffff : bytes);
  }
  const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t *>(src.base + koff),
                                                                        (short)0, (int)records, 0x00020000);
  const int o_left = src.o_left;
  const int k_left = (int)(K - k0 < BK ? K - k0 : BK);  // k still inside the matrix (clamped to the slice)
  // vector r of a thread covers (o, k) = (o_t + r * o_step, k_t .. +7) (KMAJ)
  // or (o_t .. +7, k_t + r * k_step): its offset advances by a fixed stride,
  // kept in a vector register (hoisting one scalar product per load would run
  // the 128-tile kernels out of scalar registers)
  constexpr int PER_ROW = KMAJ ? BK / 8 : T / 8;  // vectors per row of the contiguous dimension
  constexpr int STEP = THREADS / PER_ROW;         // rows advanced per vector (even)
  int o_t, k_t;
  first_vector<T, KMAJ>(tid, o_t, k_t);
  const uint32_t ld = (uint32_t)src.ld;
  uint32_t stride;
  asm("v_mov_b32 %0, %1" : "=v"(stride) : "s"(STEP * ld * 2u));
  uint32_t off = (KMAJ ? (uint32_t)o_t * ld + (uint32_t)k_t : (uint32_t)k_t * ld + (uint32_t)o_t);
  off = (off + src.delta) * 2u;
  // realigning loads start at the dword holding the vector's first element;
  // the fifth dword only matters when that element is its upper half
  uint32_t unshifted = 0;
  if constexpr (realigning<VEC>()) {
    unshifted = (off & 2u) ? 0u : kOutside;
    off &= ~3u;
  }
#pragma unroll
  for (int r = 0; r < Stage<T, VEC>::kLoads; ++r, off += stride) {
    // A vector wholly outside the matrix (past the other dimension, or
    // starting past the contiguous extent) sets bit 31 of its offsets (past the
    // resource), in arithmetic rather than with a per-load lane mask.  With
    // VEC = 8 the host guarantees the contiguous extent is a multiple of 8, so
    // no vector is partly outside.
    const int o = KMAJ ? o_t + r * STEP : o_t, k = KMAJ ? k_t : k_t + r * STEP;
    const uint32_t outside = ((uint32_t)(o_left - 1 - o) | (uint32_t)(k_left - 1 - k)) & kOutside;
    const uint32_t voff = off | outside;
    st.v[r] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rsrc, voff, 0, 0));
    if constexpr (realigning<VEC>() && !EVEN)
      st.tail[r] = __builtin_amdgcn_raw_buffer_load_b32(rsrc, (voff | unshifted) + 16u, 0, 0);
  }
}

// Vector r of a stage as 8 elements: as loaded (16-byte loads, or an even
// operand contiguous along M or N), or dword j taken from dwords j and j + 1 by
// selector sel[j] (an even operand's selectors never take the fifth dword).
template <int T, int VEC, bool KMAJ, bool EVEN>
__device__ __forceinline__ u32x4 vector_of(const Stage<T, VEC> &st, int r, const uint32_t (&sel)[4]) {
  if constexpr (!realigning<VEC>() || (EVEN && !KMAJ)) {
    return st.v[r];
  } else {
    const u32x4 w = st.v[r];
    const uint32_t fifth = EVEN ? 0u : st.tail[r];
    return u32x4{__builtin_amdgcn_perm(w[1], w[0], sel[0]), __builtin_amdgcn_perm(w[2], w[1], sel[1]),
                 __builtin_amdgcn_perm(w[3], w[2], sel[2]), __builtin_amdgcn_perm(fifth, w[3], sel[3])};
  }
}

// Write the staged slice into its LDS tile: [outer][PITCH] when K is the
// contiguous dimension, [BK][T] (swizzled) otherwise.
// last: the slice is K's last (uniform; selects the K-clearing selectors).
template <int T, bool KMAJ, int VEC, bool EVEN>
__device__ __forceinline__ void commit(const Stage<T, VEC> &st, uint16_t *s, int tid, const Realign &rl, bool last) {
  constexpr int BK = bk<T>(), PITCH = pitch<T>();
  uint32_t sel[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) sel[j] = KMAJ && last ? rl.last[j] : rl.sel;
#pragma unroll
  for (int r = 0; r < Stage<T, VEC>::kLoads; ++r) {
    const int v = tid + r * THREADS;
    const u32x4 e = vector_of<T, VEC, KMAJ, EVEN>(st, r, sel);
    if constexpr (KMAJ) {
      constexpr int PER_ROW = BK / 8;
      const int o = v / PER_ROW, k = (v % PER_ROW) * 8;
      *reinterpret_cast<u32x4 *>(s + o * PITCH + k) = e;
    } else {
      constexpr int PER_ROW = T / 8;
      const int k = v / PER_ROW, o = (v % PER_ROW) * 8;
      *reinterpret_cast<u32x4 *>(reinterpret_cast<char *>(s) + omaj_off<T>(k, o)) = e;
    }
  }
}

template <int T, bool BF16, bool OUT16, bool A_KMAJ, bool B_KMAJ, int VEC>
__global__ __launch_bounds__(THREADS) void gemm_masked_kernel(KernelArgs p) {
  constexpr int W = T / 2;    // wave tile
  constexpr int NB = W / 32;  // 32 x 32 MFMA blocks per wave and dimension
  constexpr int BK = bk<T>(), PITCH = pitch<T>();
  static_assert(BK * T <= T * PITCH, "a [BK][T] tile fits the buffer of a [T][PITCH] one");
  __shared__ __attribute__((aligned(16))) uint16_t sA[2][T * PITCH];
  __shared__ __attribute__((aligned(16))) uint16_t sB[2][T * PITCH];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // tile order: per-XCD regrouping, then groups of 8 tile rows column by
  // column, so the tiles resident on one XCD share A and B panels in its L2;
  // a strided batch runs as one 1-D grid over every problem's tiles
  const int ntiles = p.tiles_m * p.tiles_n;
  int pid;
  int64_t z;
  if (p.flat_batch) {
    pid = xcd_remap(blockIdx.x, ntiles * p.flat_batch);
    z = pid / ntiles;
    pid -= (int)z * ntiles;
  } else {
    pid = xcd_remap(blockIdx.x, ntiles);
    z = (int64_t)p.z0 + blockIdx.y;
  }
  int tm, tn;
  tile_order(pid, p.tiles_m, p.tiles_n, 8, tm, tn);
  const int64_t m0 = (int64_t)tm * T;
  const int64_t n0 = (int64_t)tn * T;
  const int64_t M = rows_of(p, z);  // this problem's rows
  if (m0 >= M) return;              // the whole tile lies past them (uniform)
  const Epilogue ep = epilogue_in_vgprs(p);  // kept out of the scalar registers the loop needs
  const uint16_t *A = p.A + z * p.sA;
  const uint16_t *B = p.B + z * p.sB;
  const Src src_a = make_src<T, A_KMAJ, VEC>(A, p.lda, M, p.K, m0);
  const Src src_b = make_src<T, B_KMAJ, VEC>(B, p.ldb, p.N, p.K, n0);
  constexpr bool EA = realigning<VEC>() && (VEC & 1), EB = realigning<VEC>() && (VEC & 2);
  Realign rl_a{}, rl_b{};
  if constexpr (realigning<VEC>()) {
    rl_a = make_realign<T, A_KMAJ>(src_a, p.K, tid);
    rl_b = make_realign<T, B_KMAJ>(src_b, p.K, tid);
  }

  f32x16 acc[NB][NB];
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = f32x16{};

  // Software pipeline: registers hold the next D slices in flight while LDS
  // holds the current one (double-buffered), so a slice's loads have D slices
  // of work to land behind instead of one.  Slices past K load as zeros (no
  // memory access).
  constexpr int D = depth<T, VEC>();
  constexpr int STEPS = BK / 16;  // 16-deep MFMA steps per slice
  const int nk = (int)((p.K + BK - 1) / BK);  // K <= 2^31 - 1 (host check)
  Stage<T, VEC> ra[D], rb[D];
  if (nk > 0) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      fetch<T, A_KMAJ, VEC, EA>(ra[u], src_a, p.K, u * BK, tid);
      fetch<T, B_KMAJ, VEC, EB>(rb[u], src_b, p.K, u * BK, tid);
    }
    commit<T, A_KMAJ, VEC, EA>(ra[0], sA[0], tid, rl_a, nk == 1);
    commit<T, B_KMAJ, VEC, EB>(rb[0], sB[0], tid, rl_b, nk == 1);
    // registers then hold slices 1 .. D: slice D goes where slice 0 was
    fetch<T, A_KMAJ, VEC, EA>(ra[0], src_a, p.K, D * BK, tid);
    fetch<T, B_KMAJ, VEC, EB>(rb[0], src_b, p.K, D * BK, tid);
  }
  __syncthreads();

  // The fragments of step ks of the slice in LDS buffers a_s, b_s.
  auto step_fragments = [&](const uint16_t *a_s, const uint16_t *b_s, int ks, u32x4(&af)[NB], u32x4(&bf)[NB]) {
    const int kk = ks * 16 + (lane >> 5) * 8;
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      if constexpr (A_KMAJ)
        af[i] = *reinterpret_cast<const u32x4 *>(a_s + (wm * W + i * 32 + (lane & 31)) * PITCH + kk);
      else
        af[i] = read_omaj<T>(a_s, wm * W + i * 32, ks, lane);
      if constexpr (B_KMAJ)
        bf[i] = *reinterpret_cast<const u32x4 *>(b_s + (wn * W + i * 32 + (lane & 31)) * PITCH + kk);
      else
        bf[i] = read_omaj<T>(b_s, wn * W + i * 32, ks, lane);
    }
  };
  auto step_mma = [&](const u32x4(&af)[NB], const u32x4(&bf)[NB]) {
#pragma unroll
    for (int i = 0; i < NB; ++i)
#pragma unroll
      for (int j = 0; j < NB; ++j) acc[i][j] = mfma_32x32x16<BF16>(af[i], bf[j], acc[i][j]);
  };

  // At slice t: LDS buffer t % 2 holds slice t, registers slices t+1 .. t+D.
  // Every slice before K's last is whole, and runs without a branch: its
  // fragment reads, its MFMAs, the next slice's commit and the refill form one
  // block, so the reads' latencies overlap and the commit's VALU work and
  // loads interleave with the MFMAs.
  for (int kt = 0; kt < nk - 1; kt += D) {
#pragma unroll
    for (int u = 0; u < D; ++u) {        // slice kt + u (D is even, so its buffer is u % 2)
      if (kt + u >= nk - 1) break;       // uniform: K's last slice runs after the loop
      u32x4 af[STEPS][NB], bf[STEPS][NB];
#pragma unroll
      for (int ks = 0; ks < STEPS; ++ks) step_fragments(sA[u & 1], sB[u & 1], ks, af[ks], bf[ks]);
#pragma unroll
      for (int ks = 0; ks < STEPS; ++ks) step_mma(af[ks], bf[ks]);
      // slice kt+u+1 (fetched D slices ago) into the other LDS buffer, whose
      // last readers passed the previous barrier; then refill its registers
      // with slice kt+u+1+D
      const int nx = (u + 1) % D;          // a constant once the loop is unrolled
      const bool last = kt + u + 2 == nk;  // the slice committed is K's last
      commit<T, A_KMAJ, VEC, EA>(ra[nx], sA[(u + 1) & 1], tid, rl_a, last);
      commit<T, B_KMAJ, VEC, EB>(rb[nx], sB[(u + 1) & 1], tid, rl_b, last);
      const int64_t kf = (int64_t)(kt + u + 1 + D) * BK;
      fetch<T, A_KMAJ, VEC, EA>(ra[nx], src_a, p.K, kf, tid);
      fetch<T, B_KMAJ, VEC, EB>(rb[nx], src_b, p.K, kf, tid);
      __syncthreads();
    }
  }
  // K's last slice, in buffer (nk - 1) % 2: it stops after its last 16-deep
  // step that holds K (the steps past K would add only zeros).
  if (nk > 0) {
    const int lb = (nk - 1) & 1;
    const int krest = (int)(p.K - (int64_t)(nk - 1) * BK);  // K in this slice
#pragma unroll
    for (int ks = 0; ks < STEPS; ++ks) {
      if (ks > 0 && ks * 16 >= krest) break;  // uniform
      u32x4 af[NB], bf[NB];
      step_fragments(sA[lb], sB[lb], ks, af, bf);
      step_mma(af, bf);
    }
  }

  void *C = OUT16 ? (void *)((uint16_t *)p.C + z * p.sC) : (void *)((float *)p.C + z * p.sC);
  // Epilogue: buffer stores relative to the tile's corner, through a resource
  // that ends after the tile's last element inside M x N.  A lane whose column
  // lies past N gets an offset past the resource; rows past M lie past its end
  // (ldc >= N), so no store needs a branch, and the offsets are one scalar
  // multiple of ldc apart.  The activation is a uniform branch around the
  // stores.  When T rows of C span 2^31 bytes or more (an offset could then
  // wrap), the stores take 64-bit addresses instead, and so do the 128-tile
  // realigning kernels with both operands contiguous along M or N, where the
  // buffer form spilled two scalar registers.
  constexpr int ES = OUT16 ? 2 : 4;
  constexpr bool kBufferStores = !(T == 128 && realigning<VEC>() && !A_KMAJ && !B_KMAJ);
  const int mvalid = (int)(M - m0 < T ? M - m0 : T), nvalid = (int)(p.N - n0 < T ? p.N - n0 : T);
  const int64_t span = ((int64_t)(mvalid - 1) * p.ldc + nvalid) * ES;
  if (kBufferStores && (int64_t)T * p.ldc * ES < 0x7fffffff) {
    const __amdgpu_buffer_rsrc_t rc = __builtin_amdgcn_make_buffer_rsrc(
        static_cast<char *>(C) + (m0 * p.ldc + n0) * ES, (short)0, (int)span, 0x00020000);
    const uint32_t row_bytes = (uint32_t)p.ldc * ES;
    const int act = __builtin_amdgcn_readfirstlane(ep.act);
    auto stores = [&](auto with_act) {
#pragma unroll
      for (int i = 0; i < NB; ++i)
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int lcol = wn * W + j * 32 + (lane & 31);
          const uint32_t coff = lcol < nvalid ? (uint32_t)lcol * ES : kOutside;
          const uint32_t lane_off = (uint32_t)(wm * W + i * 32 + 4 * (lane >> 5)) * row_bytes + coff;
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t off = lane_off + (uint32_t)(8 * (r >> 2) + (r & 3)) * row_bytes;
            const float v = decltype(with_act)::value ? ep.apply(acc[i][j][r]) : acc[i][j][r];
            if constexpr (OUT16)
              __builtin_amdgcn_raw_buffer_store_b16(ep.to16(v), rc, off, 0, 0);
            else
              __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, v), rc, off, 0, 0);
          }
        }
    };
    if (act == 0)
      stores(std::false_type{});
    else
      stores(std::true_type{});
    return;
  }
#pragma unroll
  for (int i = 0; i < NB; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t row = m0 + wm * W + i * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        const int64_t col = n0 + wn * W + j * 32 + (lane & 31);
        store_masked<OUT16>(C, p.ldc, M, p.N, row, col, acc[i][j][r], ep);
      }
}

template <int T, bool BF16, bool OUT16, bool A_KMAJ, bool B_KMAJ, int VEC>
hipError_t launch_t(const KernelArgs &base, int64_t batch, hipStream_t stream) {
  const int64_t tiles = (int64_t)base.tiles_m * base.tiles_n;
  // one 1-D grid while its work-items stay below 2^32, else a 2-D grid
  if (batch > 1 && tiles * batch * THREADS <= 0xffffffffLL) {
    KernelArgs a = base;
    a.z0 = 0;
    a.flat_batch = (int32_t)batch;
    hipLaunchKernelGGL((gemm_masked_kernel<T, BF16, OUT16, A_KMAJ, B_KMAJ, VEC>), dim3((unsigned)(tiles * batch)),
                       dim3(THREADS), 0, stream, a);
    return hipGetLastError();
  }
  for (int64_t z0 = 0; z0 < batch; z0 += kMaxGridY) {
    KernelArgs a = base;
    a.z0 = (int32_t)z0;
    const int64_t nz = batch - z0 < kMaxGridY ? batch - z0 : kMaxGridY;
    hipLaunchKernelGGL((gemm_masked_kernel<T, BF16, OUT16, A_KMAJ, B_KMAJ, VEC>), dim3((unsigned)tiles, (unsigned)nz),
                       dim3(THREADS), 0, stream, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

template <int T, bool BF16, bool OUT16, int VEC>
hipError_t dispatch_layout(const Problem &p, const KernelArgs &a, hipStream_t s) {
  const bool a_kmaj = !p.a_col, b_kmaj = p.b_col;
  if (a_kmaj && b_kmaj) return launch_t<T, BF16, OUT16, true, true, VEC>(a, p.batch, s);
  if (a_kmaj && !b_kmaj) return launch_t<T, BF16, OUT16, true, false, VEC>(a, p.batch, s);
  if (!a_kmaj && b_kmaj) return launch_t<T, BF16, OUT16, false, true, VEC>(a, p.batch, s);
  return launch_t<T, BF16, OUT16, false, false, VEC>(a, p.batch, s);
}

template <int T, int VEC>
hipError_t dispatch_types(const Problem &p, const KernelArgs &a, hipStream_t s) {
  if (p.in_bf16)
    return p.out16 ? dispatch_layout<T, true, true, VEC>(p, a, s) : dispatch_layout<T, true, false, VEC>(p, a, s);
  return p.out16 ? dispatch_layout<T, false, true, VEC>(p, a, s) : dispatch_layout<T, false, false, VEC>(p, a, s);
}

}  // namespace

hipError_t launch_masked(const Problem &p, int vec, int tile, hipStream_t stream) {
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
  a.tiles_m = (int32_t)((p.M + tile - 1) / tile);
  a.tiles_n = (int32_t)((p.N + tile - 1) / tile);
  // realigning loads: the even operands (see the load modes above)
  auto even = [&](const void *X, int64_t ld, int64_t stride) {
    return ((uintptr_t)X & 3) == 0 && ld % 2 == 0 && (p.batch == 1 || stride % 2 == 0);
  };
  const int mode = vec == 8 ? 8 : (even(p.A, p.lda, p.sA) ? 1 : 0) | (even(p.B, p.ldb, p.sB) ? 2 : 0);
  switch (tile * 16 + mode) {
    case 64 * 16 + 8: return dispatch_types<64, 8>(p, a, stream);
    case 64 * 16 + 0: return dispatch_types<64, 0>(p, a, stream);
    case 64 * 16 + 1: return dispatch_types<64, 1>(p, a, stream);
    case 64 * 16 + 2: return dispatch_types<64, 2>(p, a, stream);
    case 64 * 16 + 3: return dispatch_types<64, 3>(p, a, stream);
    case 128 * 16 + 8: return dispatch_types<128, 8>(p, a, stream);
    case 128 * 16 + 0: return dispatch_types<128, 0>(p, a, stream);
    case 128 * 16 + 1: return dispatch_types<128, 1>(p, a, stream);
    case 128 * 16 + 2: return dispatch_types<128, 2>(p, a, stream);
    default: return dispatch_types<128, 3>(p, a, stream);
  }
}

const char *masked_name(int vec, int tile) {
  if (tile == 64) return vec == 8 ? "masked_64x64x64_vec8" : "masked_64x64x64_vecu";
  return vec == 8 ? "masked_128x128x32_vec8" : "masked_128x128x32_vecu";
}

}  // namespace tsm
