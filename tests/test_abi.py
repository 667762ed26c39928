"""C-ABI library: loads, exports every declared symbol, and validates arguments on the host.

CPU only: every call here is rejected by the host-side checks (or has nothing
to compute) before the library makes any HIP call, so no GPU is needed.
"""

import ctypes
import os
import re

import pytest

import tiled_shared_memory_amd as tsm
from tiled_shared_memory_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include")) if f.endswith(".h")]

# fake, suitably aligned device addresses: never dereferenced by these calls
A0, B0, C0 = 0x7F0000000000, 0x7F1000000000, 0x7F2000000000


def declared_functions():
    names = []
    for h in HEADERS:
        text = open(h).read()
        text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
        for m in re.finditer(r"^[A-Za-z_][\w \t\*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M):
            if not m.group(0).lstrip().startswith("#"):
                names.append(m.group(1))
    return names


def test_header_declares_the_entry_points():
    names = declared_functions()
    for n in ("gemm", "gemm_ex", "gemm_strided_batched", "gemm_strided_batched_ex", "gemm_grouped", "rowsum",
              "tsm_status_string", "tsm_last_error_detail", "tsm_gemm_kernel_name", "tsm_gemm_grouped_kernel_name",
              "tsm_rowsum_kernel_name"):
        assert n in names


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIBRARY)
    for n in declared_functions():
        assert hasattr(lib, n), f"{n} declared in include/ but not exported"
    assert set(declared_functions()) == set(_lib.SIGNATURES), "binding and header disagree"


def test_header_compiles_as_c():
    import subprocess
    import tempfile

    with tempfile.TemporaryDirectory() as d:
        src = os.path.join(d, "t.c")
        open(src, "w").write('#include "tsm_gemm.h"\nint main(void){return TSM_SUCCESS;}\n')
        subprocess.run(["gcc", "-std=c99", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), src, "-o",
                        os.path.join(d, "t")], check=True)


def _call(**kw):
    args = dict(M=64, N=128, K=128, A=A0, lda=128, la=0, sA=0, B=B0, ldb=128, lb=0, sB=0, C=C0, ldc=128, sC=0,
                batch=1, dtype=0)
    args.update(kw)
    return tsm.gemm_strided_batched_ex(args["M"], args["N"], args["K"], args["A"], args["lda"], args["la"],
                                       args["sA"], args["B"], args["ldb"], args["lb"], args["sB"], args["C"],
                                       args["ldc"], args["sC"], args["batch"], args["dtype"], 0)


@pytest.mark.parametrize("kw,status,needle", [
    (dict(M=-1), 1, "negative size"),
    (dict(K=-5), 1, "negative size"),
    (dict(batch=-1), 1, "negative batch"),
    (dict(dtype=6), 1, "dtype"),
    (dict(dtype=-1), 1, "dtype"),
    (dict(la=2), 1, "layout_a"),
    (dict(lb=7), 1, "layout_b"),
    (dict(C=0), 1, "C is NULL"),
    (dict(A=0), 1, "A is NULL"),
    (dict(B=0), 1, "B is NULL"),
    (dict(lda=127), 1, "lda"),
    (dict(la=1, lda=63), 1, "lda"),
    (dict(ldb=127), 1, "ldb"),
    (dict(lb=1, ldb=127), 1, "ldb"),
    (dict(ldc=127), 1, "ldc"),
    (dict(A=A0 + 1), 1, "aligned"),
    (dict(B=B0 + 3), 1, "aligned"),
    (dict(C=C0 + 2), 1, "aligned"),           # float32 C needs 4-byte alignment
    (dict(C=A0 + 4096), 1, "C overlaps A"),
    (dict(C=B0), 1, "C overlaps B"),
    (dict(batch=2, sC=64 * 128 - 1), 1, "strideC"),
    (dict(batch=2, sA=-1), 1, "stride"),
    (dict(M=1 << 31, lda=128), 2, "2^31"),
    (dict(batch=1 << 40, sA=1 << 40, sB=1 << 40, sC=1 << 40), 2, "overflows"),
])
def test_invalid_arguments_are_rejected(kw, status, needle):
    with pytest.raises(tsm.TsmError) as ei:
        _call(**kw)
    assert ei.value.status == status
    assert needle in ei.value.detail


def test_f16_output_needs_only_2_byte_alignment():
    # dtype 1 = f16 -> f16 output: C + 2 is fine; C + 1 is not
    assert tsm.tsm_gemm_kernel_name(4, 4, 4, A0, 4, 0, 0, B0, 4, 0, 0, C0 + 2, 4, 0, 1, 1) is not None
    assert tsm.tsm_gemm_kernel_name(4, 4, 4, A0, 4, 0, 0, B0, 4, 0, 0, C0 + 1, 4, 0, 1, 1) is None


@pytest.mark.parametrize("kw", [dict(M=0), dict(N=0), dict(batch=0), dict(M=0, A=0, B=0, C=0)])
def test_empty_problems_succeed_without_launch(kw):
    assert _call(**kw) == 0
    assert tsm.tsm_last_error_detail() == ""


def test_k_zero_needs_no_operands():
    # K = 0 writes zeros into C; A and B are never read, so NULL is accepted
    name = tsm.tsm_gemm_kernel_name(8, 8, 0, 0, 1, 0, 0, 0, 8, 0, 0, C0, 8, 0, 1, 0)
    assert name is not None


def test_status_strings():
    assert tsm.tsm_status_string(0) == "success"
    assert tsm.tsm_status_string(1) == "invalid value"
    assert tsm.tsm_status_string(2) == "not supported"
    assert tsm.tsm_status_string(3) == "launch failure"
    assert tsm.tsm_status_string(99) == "unknown status"


def test_kernel_selection_for_the_workloads():
    from workloads import WORKLOADS

    picks = {}
    for name, w in WORKLOADS.items():
        lda, ldb, ldc = w.lds()
        sA, sB, sC = w.strides()
        code = {("f16", "f32"): 0, ("f16", "f16"): 1, ("bf16", "f32"): 2, ("bf16", "f16"): 3}[(w.in_fmt, w.out_fmt)]
        picks[name] = tsm.tsm_gemm_kernel_name(w.M, w.N, w.K, A0, lda, int(w.a_layout == "col"), sA,
                                               0x7E0000000000, ldb, int(w.b_layout == "col"), sB, C0, ldc, sC,
                                               w.batch, code)
        assert picks[name] is not None, name
    # the ragged workload has K = 777, so rows of A are only 2-byte aligned
    assert picks["ragged_f16_1000x1500x777"].endswith("vecu")


def test_kernel_selection_by_layout_and_shape():
    """Aligned 256-multiples with at least 256 tiles go to the large-tile kernel for both B layouts (K-contiguous
    B on the 64-deep variant, row-major B on the transpose-read variant); fewer tiles, a misaligned ldb or K not a
    multiple of 128 go elsewhere."""
    B0 = 0x7E0000000000
    n = 4096
    col = tsm.tsm_gemm_kernel_name(n, n, n, A0, n, 0, 0, B0, n, 1, 0, C0, n, 0, 1, 2)
    row = tsm.tsm_gemm_kernel_name(n, n, n, A0, n, 0, 0, B0, n, 0, 0, C0, n, 0, 1, 2)
    assert col == "tile_256x256x64_mi16_st"
    assert row == "tile_256x256x32_mi16_nn"
    # 16 tiles of 256 x 256 but a batch of 16: 256 workgroups
    assert tsm.tsm_gemm_kernel_name(1024, 1024, 1024, A0, 1024, 0, 1 << 20, B0, 1024, 1, 1 << 20, C0, 1024, 1 << 20,
                                    16, 2) == "tile_256x256x64_mi16_st"
    # 16 tiles, one problem: the 128 x 128 kernel spreads over more CUs
    assert tsm.tsm_gemm_kernel_name(1024, 1024, 1024, A0, 1024, 0, 0, B0, 1024, 1, 0, C0, 1024, 0, 1,
                                    2).startswith("masked_")
    odd = tsm.tsm_gemm_kernel_name(n, n, n, A0, n, 0, 0, B0, n + 4, 0, 0, C0, n, 0, 1, 2)
    assert odd.startswith("masked_")
    assert tsm.tsm_gemm_kernel_name(n, n, n + 64, A0, n + 64, 0, 0, B0, n, 0, 0, C0, n, 0, 1, 2).startswith("masked_")
    # few output tiles and deep K: split-K
    assert tsm.tsm_gemm_kernel_name(256, 256, 8192, A0, 8192, 0, 0, B0, 256, 0, 0, C0, 256, 0, 1, 0).startswith("splitk_")


def test_mid_size_selection():
    """The 256 x 256 kernels from 72 tiles, whatever the layouts; below that the masked
    kernels (64 x 64 tiles under 180 tiles of 128 x 128), and split-K up to 9 such tiles with K-contiguous B, 4
    with row-major B."""
    B0 = 0x7E0000000000

    def pick(n, K, lb, m=None):
        m = m or n
        return tsm.tsm_gemm_kernel_name(m, n, K, A0, K, 0, 0, B0, K if lb else n, lb, 0, C0, n, 0, 1, 3)

    assert pick(3072, 1024, 1) == "tile_256x256x64_mi16_st"  # 144 tiles
    assert pick(3072, 1024, 0) == "tile_256x256x32_mi16_nn"
    assert pick(2560, 8192, 0) == "tile_256x256x32_mi16_nn"  # 100 tiles, deep K
    assert pick(2560, 2048, 0) == "tile_256x256x32_mi16_nn"  # 100 tiles
    assert pick(2304, 1024, 1) == "tile_256x256x64_mi16_st"  # 81 tiles
    assert pick(2304, 1024, 1, m=2048) == "tile_256x256x64_mi16_st"  # 72 tiles
    assert pick(2560, 512, 0) == "tile_256x256x32_mi16_nn"  # 100 tiles, short K
    assert pick(2304, 512, 1, m=2048) == "tile_256x256x64_mi16_st"  # 72 tiles, short K
    assert pick(2048, 2048, 1) == "masked_128x128x32_vec8"  # 64 tiles
    assert pick(2048, 8192, 1) == "masked_128x128x32_vec8"  # 64 tiles, 256 of 128 x 128
    assert pick(2048, 8192, 0) == "masked_128x128x32_vec8"
    assert pick(1792, 8192, 1) == "masked_128x128x32_vec8"  # 196 of 128 x 128
    assert pick(1664, 8192, 1) == "masked_64x64x64_vec8"  # 169 of 128 x 128
    assert pick(1536, 8192, 1) == "masked_64x64x64_vec8"  # 144 of 128 x 128
    assert pick(1024, 8192, 0) == "masked_64x64x64_vec8"
    assert pick(384, 8192, 1) == "splitk_16x16_w16_t"  # 9 of 128 x 128
    assert pick(512, 8192, 1) == "masked_64x64x64_vec8"  # 16
    assert pick(256, 8192, 0) == "splitk_16x16_w16"  # 4
    assert pick(384, 8192, 0) == "masked_64x64x64_vec8"  # 9
    # column-major A (M-contiguous): the transposing variants
    n, K = 3072, 8192
    for lb, name in ((0, "tile_256x256x32_mi16_tn"), (1, "tile_256x256x32_mi16_tt")):
        assert tsm.tsm_gemm_kernel_name(n, n, K, A0, n, 1, 0, B0, K if lb else n, lb, 0, C0, n, 0, 1, 3) == name
    # M not a multiple of 8: the general kernel
    assert tsm.tsm_gemm_kernel_name(n - 4, n, K, A0, n, 1, 0, B0, n, 0, 0, C0, n, 0, 1, 3).startswith("masked_")


def test_skinny_selection():
    """Up to 128 rows of row-major A go to the streaming kernel: the widest panel whose grid fills the 256 CUs
    (256 columns up to 64 rows; 128 columns with row-major B or 65-128 rows), 64 columns otherwise; row blocks
    follow M; B either way.  K not a multiple of 64 or N not a multiple of 64 go elsewhere."""
    B0 = 0x7E0000000000
    N, K = 16384, 8192

    def pick(M, N=N, K=K, batch=1, lb=0, ldb=None):
        ldb = ldb if ldb is not None else (K if lb else N)
        return tsm.tsm_gemm_kernel_name(M, N, K, A0, K, 0, M * K, B0, ldb, lb, K * N, C0, N, M * N, batch, 0)

    assert pick(16, batch=8) == "skinny_m16_n256_k64"  # 64 x 8 = 512 workgroups of 256 columns
    assert pick(16) == "skinny_m16_n64_k64"  # 64 workgroups of 256 columns would leave most CUs idle
    assert pick(1) == "skinny_m16_n64_k64"
    assert pick(17) == "skinny_m32_n64_k64"
    assert pick(32, batch=4) == "skinny_m32_n256_k64"
    assert pick(48) == "skinny_m64_n64_k64"
    assert pick(64, batch=4) == "skinny_m64_n256_k64"
    assert pick(16, N=16448) == "skinny_m16_n64_k64"  # N % 256 != 0
    assert pick(65) == "skinny_m128_n64_k64"
    assert pick(128) == "skinny_m128_n64_k64"
    assert not pick(129).startswith("skinny_")
    # few streaming workgroups times few 16-row tiles: split-K spreads the passes over B wider
    assert pick(16, N=4096, K=4096).startswith("splitk_")
    assert pick(32, N=4096, K=4096) == "skinny_m32_n64_k64"
    assert pick(48, N=128, K=4096).startswith("splitk_")
    assert not pick(16, K=8200).startswith("skinny_")
    assert not pick(16, N=16400).startswith("skinny_")
    # K-contiguous B (a weight stored output feature by output feature): the same kernel, B staged like A
    assert pick(16, lb=1) == "skinny_m16_n64_k64_t"
    assert pick(16, batch=8, lb=1) == "skinny_m16_n256_k64_t"
    # 128-column panels: 256 of them over a batch of 2, or 128 rows (no 256-column variant)
    assert pick(16, batch=2) == "skinny_m16_n128_k64"
    assert pick(128, batch=2) == "skinny_m128_n128_k64"
    assert pick(128, batch=8) == "skinny_m128_n128_k64"
    assert pick(128, batch=8, lb=1) == "skinny_m128_n128_k64_t"
    assert pick(16, batch=2, lb=1) == "skinny_m16_n64_k64_t"
    assert pick(16, N=16448, batch=2) == "skinny_m16_n64_k64"  # N % 128 != 0
    # 33-128 rows with fewer K slices than one round of the ring: the 64 x 64 masked tiles
    assert pick(64, N=128, K=128) == "masked_64x64x64_vec8"
    assert pick(128, N=8192, K=256) == "masked_64x64x64_vec8"
    assert pick(128, N=8192, K=384) == "skinny_m128_n64_k64"  # 6 slices: one round of its ring
    assert pick(16, N=4096, K=128) == "skinny_m16_n64_k64"  # up to 32 rows the streaming kernel keeps them


def test_skinny_forced_width(monkeypatch):
    B0 = 0x7E0000000000
    args = (100, 512, 512, A0, 512, 0, 0, B0, 512, 0, 0, C0, 512, 0, 1, 0)
    for good in ("skinny_m128_n64_k64", "skinny_m128_n128_k64"):
        monkeypatch.setenv("TSM_GEMM_KERNEL", good)
        assert tsm.tsm_gemm_kernel_name(*args) == good
    # a name whose row blocks do not match M, or 256 columns with 128 rows, cannot run the problem
    for bad in ("skinny_m64_n64_k64", "skinny_m128_n256_k64", "skinny_m16_n128_k64"):
        monkeypatch.setenv("TSM_GEMM_KERNEL", bad)
        assert tsm.tsm_gemm_kernel_name(*args) is None
        with pytest.raises(tsm.TsmError) as ei:
            tsm.gemm(100, 512, 512, A0, 512, B0, 512, C0, 512, 0, 0)
        assert ei.value.status == 2


W0 = 0x7F4000000000  # fake device address of a workspace


def test_general_kernel_leading_dimension_limit():
    """The general kernel addresses operand slices with 32-bit offsets: a leading dimension of 2^23 elements or
    more is reported, not truncated."""
    B0 = 0x7E0000000000
    big = 1 << 23
    with pytest.raises(tsm.TsmError) as ei:
        tsm.gemm_ex(100, 100, 100, A0, big, 0, B0, 100, 0, C0, 100, 0, 0)
    assert ei.value.status == 2 and "general kernel" in ei.value.detail
    assert tsm.tsm_gemm_kernel_name(100, 100, 100, A0, big - 8, 0, 0, B0, 100, 0, 0, C0, 100, 0, 1, 0) is not None


def test_workspace_bytes():
    """The K split's workspace depends on the shape only: batch * chunks * M * N * 4 bytes, or 0."""
    # 32-row blocks in eight 1024-deep chunks (64-row blocks would need sixteen chunks of 512, one ring round)
    assert tsm.gemm_workspace_bytes(256, 256, 8192, 1) == 8 * 256 * 256 * 4
    assert tsm.gemm_workspace_bytes(16, 4096, 4096, 1) == 4 * 16 * 4096 * 4
    assert tsm.gemm_workspace_bytes(100, 192, 1344, 1) == 5 * 100 * 192 * 4  # chunks of 320, the last 64 deep
    assert tsm.gemm_workspace_bytes(8192, 8192, 8192, 1) == 0  # enough output tiles
    assert tsm.gemm_workspace_bytes(16, 16384, 8192, 1) == 4 * 16 * 16384 * 4  # 64 panels of 256 columns, 4 chunks
    assert tsm.gemm_workspace_bytes(16, 16384, 8192, 8) == 0  # 512 panels of 256 columns already
    assert tsm.gemm_workspace_bytes(256, 256, 8200, 1) == 0  # K % 64
    assert tsm.gemm_workspace_bytes(256, 250, 8192, 1) == 0  # N % 64
    assert tsm.gemm_workspace_bytes(256, 256, 448, 1) == 0  # K below 512
    assert tsm.gemm_workspace_bytes(-1, 256, 8192, 1) == 0


def test_launch_limits_planned_on_the_host():
    """Calls whose one-launch grid would reach 2^32 work-items still plan (the kernels then launch as 2-D grids
    of at most 65535 problems, or row sums in chunks of rows); the GPU tests run the first and the last."""
    big = (1 << 24) + 3  # 64 x 64 masked tiles of 256 threads: 2^32 + 768 work-items in one 1-D grid
    assert tsm.tsm_gemm_kernel_name(16, 16, 16, A0, 16, 0, 0, B0, 16, 0, 0, C0, 16, 256, big, 0).startswith("masked_")
    # 256 x 256 tiles: a 1-D grid over 2^24 + 3 of them would need 2^32 + 768 work-items too
    assert tsm.tsm_gemm_kernel_name(256, 256, 128, A0, 128, 0, 0, B0, 128, 1, 0, C0, 256, 65536, big,
                                    3) == "tile_256x256x64_mi16_st"
    assert tsm.tsm_rowsum_kernel_name((1 << 26) + 5, 16, A0, 16, 1, tsm.TSM_ROWSUM_F32, C0).startswith("rowsum_wave")


def test_hybrid_routing(monkeypatch):
    """A little over whole rounds of 256 x 256 tiles: whole rounds data-parallel, the last round's tiles cut into
    s equal chunks of K (s * leftover <= 256 runs, s <= 8, s dividing K / 128), one float32 partial tile per run."""
    monkeypatch.delenv("TSM_GEMM_SPLIT", raising=False)

    def route(M, N, K, la=0, lb=1, nbytes=None):
        need = tsm.gemm_workspace_bytes(M, N, K, 1) if nbytes is None else nbytes
        return tsm.tsm_gemm_ws_kernel_name(M, N, K, A0, M if la else K, la, 0, B0, K if lb else N, lb, 0, C0, N, 0, 1,
                                           3, W0, need)

    tile = 256 * 256 * 4
    for M, leftover, chunks in ((4352, 16, 8), (4608, 32, 8), (5120, 64, 4), (6144, 128, 2)):
        assert tsm.gemm_workspace_bytes(M, 4096, 8192, 1) == leftover * chunks * tile
        assert route(M, 4096, 8192) == "hybrid_tile_256x256x64_mi16_st+reduce"
    # 289 tiles: 33 left over; 7 chunks do not divide K / 128 = 16, so 4
    assert tsm.gemm_workspace_bytes(4352, 4104, 2048, 1) == 33 * 4 * tile
    assert route(4352, 4096, 8192, la=0, lb=0) == "hybrid_tile_256x256x32_mi16_nn+reduce"
    assert route(4352, 4096, 8192, la=1, lb=0) == "hybrid_tile_256x256x32_mi16_tn+reduce"
    assert route(4352, 4096, 8192, la=1, lb=1) == "hybrid_tile_256x256x32_mi16_tt+reduce"
    # whole rounds, or more than half a round left over: no split; one byte short: no split
    for M, N in ((4096, 4096), (7168, 4096), (5120, 5120)):
        assert tsm.gemm_workspace_bytes(M, N, 8192, 1) == 0
        assert route(M, N, 8192, nbytes=1 << 30) == "tile_256x256x64_mi16_st"
    # one byte short: the row bands, which need no workspace
    assert route(4352, 4096, 8192, nbytes=16 * 8 * tile - 1) == "band_tile_256x256x64_mi16_st+masked_64x64x64_vec8"
    # the row bands, not the hybrid, up to K = 4096 or with at most 64 rows past the whole rounds ...
    assert route(4352, 4096, 4096) == "band_tile_256x256x64_mi16_st+masked_64x64x64_vec8"
    assert route(4160, 4096, 8192) == "band_tile_256x256x64_mi16_st+skinny_m64_n64_k64_t"
    assert route(4352, 4104, 2048) == "band_tile_256x256x64_mi16_st+masked_64x64x64_vec8"
    # ... where the bands would lose, the hybrid at any depth (80 tiles left: 2 chunks)
    assert route(5376, 4096, 2048) == "hybrid_tile_256x256x64_mi16_st+reduce"
    # ... and wherever it applies when asked for
    monkeypatch.setenv("TSM_GEMM_SPLIT", "hybrid")
    for M, N, K in ((4352, 4096, 4096), (4160, 4096, 8192), (4352, 4104, 2048)):
        assert route(M, N, K) == "hybrid_tile_256x256x64_mi16_st+reduce"
    # its workspace fits the allocation-free entry point's scratch
    assert 256 * tile <= tsm.gemm_noalloc_scratch_bytes()


def test_band_routing(monkeypatch):
    """Plain calls a little over whole rounds of 256 x 256 tiles: the rows of the whole rounds on the large-tile
    kernel, the rest as a problem of their own, when that problem goes to the streaming kernel, to 64 x 64 tiles or
    to one round of 128 x 128 tiles; otherwise one kernel."""
    monkeypatch.delenv("TSM_GEMM_KERNEL", raising=False)

    def route(M, N, K, la=0, lb=1, batch=1):
        return tsm.tsm_gemm_kernel_name(M, N, K, A0, M if la else K, la, M * K, B0, K if lb else N, lb, N * K, C0, N,
                                        M * N, batch, 3)

    st = "band_tile_256x256x64_mi16_st+"
    assert route(4160, 4096, 8192) == st + "skinny_m64_n64_k64_t"
    assert route(4224, 4096, 8192) == st + "skinny_m128_n64_k64_t"
    assert route(4352, 4096, 8192) == st + "masked_64x64x64_vec8"
    assert route(4864, 4096, 8192) == st + "masked_128x128x32_vec8"  # 768 rows left: 192 tiles of 128 x 128
    assert route(5120, 4096, 8192) == st + "masked_128x128x32_vec8"  # 256 tiles of 128 x 128: one round
    assert route(8448, 4096, 8192) == st + "masked_64x64x64_vec8"  # two whole rounds, then 256 rows
    # 12 tiles a row: 21 rows (252 tiles) fill the round, 256 rows are left
    assert route(5632, 3072, 8192) == st + "masked_64x64x64_vec8"
    assert route(4352, 4096, 8192, la=0, lb=0) == "band_tile_256x256x32_mi16_nn+masked_64x64x64_vec8"
    assert route(4352, 4096, 8192, la=1, lb=0) == "band_tile_256x256x32_mi16_tn+masked_64x64x64_vec8"
    assert route(4352, 4096, 8192, la=1, lb=1) == "band_tile_256x256x32_mi16_tt+masked_64x64x64_vec8"
    assert route(4224, 4096, 8192, la=0, lb=0) == "band_tile_256x256x32_mi16_nn+skinny_m128_n64_k64"
    # more than one round of 128 x 128 tiles left, or enough for the large-tile kernel: one kernel
    for M in (5376, 5632, 5888):
        assert route(M, 4096, 8192) == "tile_256x256x64_mi16_st"
    # whole rounds; a batch; a forced kernel: one kernel
    assert route(8192, 8192, 8192) == "tile_256x256x64_mi16_st"
    assert route(4352, 4096, 8192, batch=2) == "tile_256x256x64_mi16_st"
    monkeypatch.setenv("TSM_GEMM_KERNEL", "tile_256x256x64_mi16_st")
    assert route(4352, 4096, 8192) == "tile_256x256x64_mi16_st"


def test_streamk_on_request_only(monkeypatch):
    """Stream-K's workspace (two 256 x 256 float32 partial tiles for each of 256 runs) and route appear only with
    TSM_GEMM_SPLIT=streamk; by default 144 tiles run unsplit and 128 take the two-chunk tile split."""
    args = (3072, 3072, 8192, A0, 8192, 0, 0, B0, 8192, 1, 0, C0, 3072, 0, 1, 3)
    monkeypatch.delenv("TSM_GEMM_SPLIT", raising=False)
    assert tsm.gemm_workspace_bytes(3072, 3072, 8192, 1) == 0
    assert tsm.tsm_gemm_ws_kernel_name(*args, W0, 1 << 30) == "tile_256x256x64_mi16_st"
    assert tsm.gemm_workspace_bytes(4096, 2048, 8192, 1) == 2 * 4096 * 2048 * 4
    monkeypatch.setenv("TSM_GEMM_SPLIT", "streamk")
    need = tsm.gemm_workspace_bytes(3072, 3072, 8192, 1)
    assert need == 2 * 256 * 256 * 256 * 4
    assert tsm.tsm_gemm_ws_kernel_name(*args, W0, need) == "streamk_tile_256x256x32_mi16+reduce"
    assert tsm.tsm_gemm_ws_kernel_name(*args, W0, need - 1) == "tile_256x256x64_mi16_st"
    lay = {(0, 0): "_nn", (1, 0): "_tn", (1, 1): "_tt"}
    for (la, lb), suffix in lay.items():
        a2 = (3072, 3072, 8192, A0, 3072 if la else 8192, la, 0, B0, 8192 if lb else 3072, lb, 0, C0, 3072, 0, 1, 3)
        assert tsm.tsm_gemm_ws_kernel_name(*a2, W0, need) == f"streamk_tile_256x256x32_mi16{suffix}+reduce"
    # 225 tiles fill 7/8 of the CUs, and up to 128 rows belong to the streaming kernel: stream-K declines both
    assert tsm.gemm_workspace_bytes(3840, 3840, 8192, 1) == 0
    for M in (16, 128):
        assert tsm.tsm_gemm_ws_kernel_name(M, 16384, 8192, A0, 8192, 0, 0, B0, 8192, 1, 0, C0, 16384, 0, 1, 3, W0,
                                           1 << 30).startswith("skinny_")
    monkeypatch.setenv("TSM_GEMM_SPLIT", "none")
    assert tsm.tsm_gemm_ws_kernel_name(4096, 2048, 8192, A0, 8192, 0, 0, B0, 8192, 1, 0, C0, 2048, 0, 1, 3, W0,
                                       1 << 30) == "tile_256x256x64_mi16_st"


def _ws_args(M=256, N=256, K=8192, ws=W0, nbytes=None, lb=0):
    nbytes = tsm.gemm_workspace_bytes(M, N, K, 1) if nbytes is None else nbytes
    ldb = K if lb else N
    return (M, N, K, A0, K, 0, 0, 0x7E0000000000, ldb, lb, 0, C0, N, 0, 1, 0, ws, nbytes)


def test_workspace_routing(monkeypatch):
    assert tsm.tsm_gemm_ws_kernel_name(*_ws_args()) == "ksplit_skinny_m32_n64_k64+reduce"
    # chunks deep enough with 64-row blocks keep them (256 x 512 x 8192: eight 1024-deep chunks)
    assert tsm.tsm_gemm_ws_kernel_name(*_ws_args(N=512)) == "ksplit_skinny_m64_n64_k64+reduce"
    assert tsm.tsm_gemm_ws_kernel_name(*_ws_args(M=16, N=4096, K=4096)) == "ksplit_skinny_m16_n64_k64+reduce"
    assert tsm.tsm_gemm_ws_kernel_name(*_ws_args(M=24, N=4096, K=4096)) == "ksplit_skinny_m32_n64_k64+reduce"
    # 32 to 127 panels of 256 columns: split those (512-byte row segments of B)
    assert tsm.tsm_gemm_ws_kernel_name(*_ws_args(M=16, N=16384, K=8192)) == "ksplit_skinny_m16_n256_k64+reduce"
    assert tsm.tsm_gemm_ws_kernel_name(*_ws_args(M=64, N=8192, K=8192)) == "ksplit_skinny_m64_n256_k64+reduce"
    # C rows that are not 16-byte multiples: the reduction's 4-column stores would not be aligned
    args = list(_ws_args(M=1024, N=1024, K=8192, nbytes=1 << 30))
    assert tsm.tsm_gemm_ws_kernel_name(*args).startswith("ksplit_tile_")
    args[12] = 1026  # ldc
    assert not tsm.tsm_gemm_ws_kernel_name(*args).startswith("ksplit_")
    # a K-contiguous B splits the same way from 9 tiles of 128 x 128; up to 4 the split inside the workgroup stays
    assert tsm.tsm_gemm_ws_kernel_name(*_ws_args(M=384, N=384, lb=1, nbytes=1 << 30)).startswith("ksplit_skinny_")
    assert tsm.tsm_gemm_ws_kernel_name(*_ws_args(lb=1, nbytes=1 << 30)) == "splitk_16x16_w16_t"
    # over 128 rows and K below 2048: no split
    assert not tsm.tsm_gemm_ws_kernel_name(*_ws_args(M=512, N=512, K=1024, nbytes=1 << 30)).startswith("ksplit_")
    # too little workspace, none or a forced kernel: the kernel that needs none
    assert tsm.tsm_gemm_ws_kernel_name(*_ws_args(nbytes=8 * 256 * 256 * 4 - 4)).startswith("splitk_")
    assert tsm.tsm_gemm_ws_kernel_name(*_ws_args(ws=0, nbytes=0)).startswith("splitk_")
    monkeypatch.setenv("TSM_GEMM_KERNEL", "masked_64x64x64_vec8")
    assert tsm.tsm_gemm_ws_kernel_name(*_ws_args()) == "masked_64x64x64_vec8"


@pytest.mark.parametrize("kw,needle", [
    (dict(nbytes=-1), "negative workspace_bytes"),
    (dict(ws=0, nbytes=64), "workspace is NULL"),
    (dict(ws=W0 + 8), "not 16-byte aligned"),
    (dict(ws=C0 + 1024), "workspace overlaps C"),
    (dict(ws=A0 + 4096), "workspace overlaps A"),
])
def test_workspace_errors(kw, needle):
    args = list(_ws_args(**kw))
    with pytest.raises(tsm.TsmError) as ei:
        tsm.gemm_strided_batched_ws(*args[:16], 0, 0.0, args[16], args[17], 0)
    assert ei.value.status == 1
    assert needle in ei.value.detail
    assert tsm.tsm_gemm_ws_kernel_name(*args) is None


R0 = 0x7F3000000000  # fake device address of the row counts


def _grouped(**kw):
    args = dict(M=64, N=128, K=128, A=A0, lda=128, la=0, sA=64 * 128, B=B0, ldb=128, lb=0, sB=128 * 128, C=C0,
                ldc=128, sC=64 * 128, rows=R0, groups=4, dtype=0)
    args.update(kw)
    return [args[k] for k in ("M", "N", "K", "A", "lda", "la", "sA", "B", "ldb", "lb", "sB", "C", "ldc", "sC",
                              "rows", "groups", "dtype")]


@pytest.mark.parametrize("kw,status,needle", [
    (dict(rows=0), 1, "rows is NULL"),
    (dict(rows=R0 + 2), 1, "rows not 4-byte aligned"),
    (dict(groups=-1), 1, "negative batch"),
    (dict(sC=64 * 128 - 1), 1, "strideC"),
    (dict(dtype=9), 1, "dtype"),
])
def test_grouped_invalid_arguments_are_rejected(kw, status, needle):
    with pytest.raises(tsm.TsmError) as ei:
        tsm.gemm_grouped(*_grouped(**kw), 0)
    assert ei.value.status == status
    assert needle in ei.value.detail


@pytest.mark.parametrize("kw", [dict(groups=0), dict(M=0), dict(N=0, rows=0)])
def test_grouped_empty_succeeds_without_launch(kw):
    assert tsm.gemm_grouped(*_grouped(**kw), 0) == 0


def test_grouped_kernel_selection():
    """Grouped products route like batched ones (any M on the large-tile kernel, M <= 16 on the skinny kernel),
    except that split-K, which stores whole 16 x 16 tiles, is never used."""
    # MoE-like: 8 experts, up to 2048 tokens, 1024 x 1024 weights stored K-contiguous
    big = _grouped(M=2048, N=1024, K=1024, lda=1024, sA=2048 * 1024, ldb=1024, lb=1, sB=1024 * 1024, ldc=1024,
                   sC=2048 * 1024, groups=8, dtype=3)
    assert tsm.tsm_gemm_grouped_kernel_name(*big) == "tile_256x256x64_mi16_st"
    big[9] = 0  # row-major weights
    assert tsm.tsm_gemm_grouped_kernel_name(*big) == "tile_256x256x32_mi16_nn"
    # up to 16 rows per group: the skinny kernel
    sk = _grouped(M=16, N=1024, K=1024, lda=1024, sA=16 * 1024, ldb=1024, sB=1024 * 1024, ldc=1024, sC=16 * 1024)
    assert tsm.tsm_gemm_grouped_kernel_name(*sk).startswith("skinny_")
    # deep K, few tiles: a batched call would take split-K, a grouped one must not
    dk = _grouped(M=256, N=256, K=8192, lda=8192, sA=256 * 8192, ldb=256, sB=8192 * 256, ldc=256, sC=256 * 256,
                  groups=1)
    assert tsm.tsm_gemm_kernel_name(256, 256, 8192, A0, 8192, 0, 0, B0, 256, 0, 0, C0, 256, 0, 1, 0).startswith("splitk")
    assert tsm.tsm_gemm_grouped_kernel_name(*dk).startswith("masked_")


def test_plain_products_with_ragged_m_use_the_tile_kernel():
    """M need not be a multiple of 256 for the large-tile kernels: rows past M load as zero and are not stored."""
    assert tsm.tsm_gemm_kernel_name(8000, 8192, 8192, A0, 8192, 0, 0, B0, 8192, 1, 0, C0, 8192, 0, 1,
                                    3) == "tile_256x256x64_mi16_st"


X0, O0 = 0x7F4000000000, 0x7F5000000000


@pytest.mark.parametrize("args,status,needle", [
    ((-1, 3, X0, 3, 1, 0, O0), 1, "negative size"),
    ((2, 3, X0, -3, 1, 0, O0), 1, "negative stride"),
    ((2, 3, X0, 3, 1, 7, O0), 1, "xdtype"),
    ((2, 3, 0, 3, 1, 0, O0), 1, "X is NULL"),
    ((2, 3, X0, 3, 1, 0, 0), 1, "out is NULL"),
    ((2, 3, X0 + 2, 3, 1, 0, O0), 1, "X not 4-byte aligned"),
    ((2, 3, X0 + 1, 3, 1, 1, O0), 1, "X not 2-byte aligned"),
    ((2, 3, X0, 3, 1, 0, O0 + 2), 1, "out not 4-byte aligned"),
    ((2, 3, X0, 3, 1, 0, X0 + 8), 1, "out overlaps X"),
    ((1 << 31, 3, X0, 3, 1, 0, O0), 2, "2^31"),
    ((2, 1 << 62, X0, 1, 1 << 3, 0, O0), 2, "overflows"),
])
def test_rowsum_invalid_arguments_are_rejected(args, status, needle):
    with pytest.raises(tsm.TsmError) as ei:
        tsm.rowsum(*args, 0)
    assert ei.value.status == status
    assert needle in ei.value.detail


def test_rowsum_empty_succeeds_without_launch():
    assert tsm.rowsum(0, 5, 0, 5, 1, 0, 0, 0) == 0
    assert tsm.tsm_rowsum_kernel_name(0, 5, X0, 5, 1, 0, O0) is None


def test_rowsum_kernel_selection():
    # many short contiguous aligned rows: a wave per row with 16-byte loads
    assert tsm.tsm_rowsum_kernel_name(16384, 1000, X0, 1000, 1, 0, O0) == "rowsum_wave_vec16"
    # rows whose starts are not 16-byte aligned, or a column stride: element loads
    assert tsm.tsm_rowsum_kernel_name(16384, 1001, X0, 1001, 1, 0, O0) == "rowsum_wave_elem"
    assert tsm.tsm_rowsum_kernel_name(16384, 1000, X0, 1, 16384, 1, O0) == "rowsum_wave_elem"
    # few long rows: a workgroup per row
    assert tsm.tsm_rowsum_kernel_name(8, 1 << 20, X0, 1 << 20, 1, 2, O0) == "rowsum_block_vec16"


def test_ragged_n_routes_to_the_tile_kernel():
    """N a multiple of 8 (not of 256) stays on the large-tile kernels; N not a multiple of 8 does not."""
    assert tsm.tsm_gemm_kernel_name(4096, 50256, 4096, A0, 4096, 0, 0, B0, 4096, 1, 0, C0, 50256, 0, 1,
                                    3) == "tile_256x256x64_mi16_st"
    assert tsm.tsm_gemm_kernel_name(4096, 50256, 4096, A0, 4096, 0, 0, B0, 50256, 0, 0, C0, 50256, 0, 1,
                                    3) == "tile_256x256x32_mi16_nn"
    assert tsm.tsm_gemm_kernel_name(4096, 50257, 4096, A0, 4096, 0, 0, B0, 4096, 1, 0, C0, 50260, 0, 1,
                                    3).startswith("masked_")


def test_noalloc_scratch_covers_every_split():
    """The static scratch of the allocation-free entry point (64 MiB) holds every K split the planner makes by
    default: about 256 workgroups with at most one 256 x 256 float32 partial tile each.  Swept over squares,
    decode-like rows, deep K and batches; invalid arguments are rejected as by the other entry points (host logic
    only)."""
    cap = tsm.gemm_noalloc_scratch_bytes()
    assert cap == 64 << 20
    most = 0
    for M in list(range(16, 513, 48)) + list(range(512, 8193, 512)):
        for N in (64, 256, 1024, 4096, 16384):
            for K in (512, 2048, 8192, 65536):
                for batch in (1, 2, 8):
                    most = max(most, tsm.gemm_workspace_bytes(M, N, K, batch))
    assert 0 < most <= cap
    lib = tsm.load()
    st = lib.gemm_strided_batched_noalloc(-1, 8, 8, A0, 8, 0, 0, B0, 8, 0, 0, C0, 8, 0, 1, 0, 0, 0.0, None)
    assert st == tsm.TSM_ERROR_INVALID_VALUE
    st = lib.gemm_strided_batched_noalloc(8, 8, 8, A0, 8, 0, 0, B0, 8, 0, 0, C0, 8, 0, 1, 9, 0, 0.0, None)
    assert st == tsm.TSM_ERROR_INVALID_VALUE and "dtype" in tsm.tsm_last_error_detail()


@pytest.mark.parametrize("act,slope,status,needle", [(3, 0.0, 1, "activation"),
                                                     (tsm.TSM_ACT_LEAKY_RELU, float("nan"), 1, "slope")])
def test_bad_activation_rejected(act, slope, status, needle):
    """Unknown activations and non-finite leaky slopes are rejected on the host before any GPU call."""
    with pytest.raises(tsm.TsmError) as ei:
        tsm.gemm_strided_batched_act(4, 4, 4, 0x7F0000000000, 4, 0, 0, 0x7F1000000000, 4, 0, 0, 0x7F2000000000, 4, 0,
                                     1, 0, act, slope, 0)
    assert ei.value.status == status and needle in ei.value.detail
