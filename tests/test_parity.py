"""GPU path vs the CPU oracle, element by element, through the C ABI (needs an MI355X).

Acceptance per element (fp64): |C_gpu - C_ref| <= K * 2^-24 * sum_k |A_ik * B_kj|,
plus half an f16 ulp of the stored value for f16 output.
"""

import numpy as np
import pytest

import oracle
from gpu_util import DTYPE, LAYOUT, alloc_c, check, run, say, to_device
import tiled_shared_memory_amd as tsm
from workloads import WORKLOADS
from workloads.inputs import F16, BF16, integer_operands, make_operands

pytestmark = pytest.mark.gpu

SMALL = ["single_f16_64x128x128", "largek_f16_256x256x8192", "ragged_f16_1000x1500x777"]


@pytest.fixture(scope="module")
def big_inputs():
    cache = {}

    def get(name):
        if name not in cache:
            say(f"[inputs] generating {name}")
            cache[name] = WORKLOADS[name].operands()
        return cache[name]

    return get


@pytest.mark.parametrize("name", SMALL)
def test_workload_full_parity(orc, name):
    w = WORKLOADS[name]
    A, B = w.operands()
    say(f"[gpu] {name} full parity M={w.M} N={w.N} K={w.K}")
    C = run(A, B, w.M, w.N, w.K, w.in_fmt, w.out_fmt, batch=w.batch, a_layout=w.a_layout, b_layout=w.b_layout,
            kernel=EXPECTED_KERNEL.get(name))
    Cr, S = orc.gemm_rows(A, B, w.M, w.N, w.K, w.in_fmt, batch=w.batch, a_layout=w.a_layout, b_layout=w.b_layout)
    ratio = check(C, Cr, S, w.K, w.out_fmt, name)
    say(f"[gpu] {name}: max err/bound = {ratio:.3e}")


def _sample_cells(rng, batch, M, N, n):
    z = rng.integers(0, batch, n)
    i = rng.integers(0, M, n)
    j = rng.integers(0, N, n)
    # corners and tile edges of every problem
    edge_i = np.array([0, M - 1, min(M - 1, 127), min(M - 1, 128), min(M - 1, 255), min(M - 1, 256)])
    edge_j = np.array([0, N - 1, min(N - 1, 127), min(N - 1, 128), min(N - 1, 255), min(N - 1, 256)])
    ez, ei, ej = np.meshgrid(np.arange(batch), edge_i, edge_j, indexing="ij")
    return (np.concatenate([z, ez.ravel()]), np.concatenate([i, ei.ravel()]), np.concatenate([j, ej.ravel()]))


# the kernels the benchmark times (the large-K workload: without a workspace; its workspace route is tested
# with the K split)
EXPECTED_KERNEL = {"square_bf16_8192": "tile_256x256x64_mi16_st", "skinny_f16_16x16384x8192_b8": "skinny_m16_n256_k64",
                   "largek_f16_256x256x8192": "splitk_", "ragged_f16_1000x1500x777": "masked_64x64x64_vecu",
                   "single_f16_64x128x128": "masked_64x64x64_vec8"}


@pytest.mark.parametrize("name", ["square_bf16_8192", "skinny_f16_16x16384x8192_b8"])
def test_workload_full_size_parity(orc, big_inputs, name):
    """Full-size workloads, every element against the oracle (computed in row chunks to bound host memory), on the
    kernel the benchmark times; C is filled with NaN first, so an element the kernel never wrote fails."""
    import torch

    w = WORKLOADS[name]
    A, B = big_inputs(name)
    say(f"[gpu] {name} M={w.M} N={w.N} K={w.K} batch={w.batch}, every element")
    lda, ldb, ldc = w.lds()
    sA, sB, sC = w.strides()
    code = DTYPE[(w.in_fmt, w.out_fmt)]
    a_buf, a_ptr = to_device(A)
    b_buf, b_ptr = to_device(B)
    c = alloc_c(w.batch, w.M, w.N, ldc, sC, w.out_fmt, fill=float("nan"))
    args = (w.M, w.N, w.K, a_ptr, lda, LAYOUT[w.a_layout], sA, b_ptr, ldb, LAYOUT[w.b_layout], sB, c, ldc, sC,
            w.batch, code)
    assert tsm.tsm_gemm_kernel_name(*args).startswith(EXPECTED_KERNEL[name])
    tsm.gemm_strided_batched_ex(*args, 0)
    torch.cuda.synchronize()
    host = c.float().cpu().numpy().astype(np.float64)[:w.batch * sC].reshape(w.batch, w.M, ldc)[:, :, :w.N]
    del c, a_buf, b_buf
    worst = 0.0
    chunk = 1024
    for z in range(w.batch):
        for r0 in range(0, w.M, chunk):
            r1 = min(w.M, r0 + chunk)
            Cr, S = orc.gemm_rows(A[z:z + 1], B[z:z + 1], w.M, w.N, w.K, w.in_fmt, a_layout=w.a_layout,
                                  b_layout=w.b_layout, row_begin=r0, row_end=r1)
            worst = max(worst, check(host[z:z + 1, r0:r1], Cr, S, w.K, w.out_fmt, f"{name} problem {z} rows {r0}.."))
    say(f"[gpu] {name}: every element within the bound, max err/bound = {worst:.3e}")


EDGE_SHAPES = [(1, 1, 1), (1, 2, 3), (2, 3, 1), (3, 1, 2), (15, 17, 16), (16, 16, 16), (17, 15, 31),
               (31, 33, 3), (33, 31, 6), (127, 129, 33), (128, 128, 32), (129, 127, 65), (130, 257, 100),
               (255, 1, 64), (1, 300, 257), (64, 128, 128), (200, 8, 8), (8, 200, 1000)]


MASKED_VARIANTS = ["masked_128x128x32_vecu", "masked_64x64x64_vecu", "masked_128x128x32_vec8",
                   "masked_64x64x64_vec8"]


@pytest.mark.parametrize("variant", MASKED_VARIANTS)
@pytest.mark.parametrize("shape", [(1, 1, 1), (65, 63, 33), (130, 257, 100), (200, 72, 1000)],
                         ids=lambda s: "x".join(map(str, s)))
def test_masked_variants(orc, monkeypatch, variant, shape):
    """Both tile sizes of the general kernel, forced, in all four layout pairs (16-byte loads where the
    contiguous extents allow them)."""
    M, N, K = shape
    monkeypatch.setenv("TSM_GEMM_KERNEL", variant)
    vec8 = variant.endswith("vec8")
    for a_layout in ("row", "col"):
        for b_layout in ("row", "col"):
            ext_a = K if a_layout == "row" else M
            ext_b = N if b_layout == "row" else K
            if vec8 and (ext_a % 8 or ext_b % 8):
                continue
            A, B = make_operands(M + 2 * N + 3 * K, 1, M, N, K, F16, ("uniform", -1.0, 1.0), a_layout, b_layout)
            say(f"[gpu] {variant} {shape} A:{a_layout} B:{b_layout}")
            C = run(A, B, M, N, K, F16, "f32", a_layout=a_layout, b_layout=b_layout, kernel=variant)
            Cr, S = orc.gemm_rows(A, B, M, N, K, F16, a_layout=a_layout, b_layout=b_layout)
            check(C, Cr, S, K, "f32", f"{variant} {shape} {a_layout}/{b_layout}")


@pytest.mark.parametrize("variant", ["masked_128x128x32_vecu", "masked_64x64x64_vecu"])
@pytest.mark.parametrize("offsets", [(0, 0), (1, 0), (0, 1), (1, 3)], ids=lambda o: f"off{o[0]}{o[1]}")
@pytest.mark.parametrize("pad", [2, 1], ids=["oddld", "evenld"])
def test_masked_realigned_loads(orc, monkeypatch, variant, offsets, pad):
    """The realigned 16-byte loads: operands whose rows start at every 2-byte alignment (odd leading dimensions,
    odd base offsets, odd batch strides), in all four layout pairs, with vectors cut by the contiguous extent
    (K = 203, M = 137, N = 75: odd, so every row and problem is ragged against the 8-element vectors).  With even
    leading dimensions, an operand whose base offset is even too starts every vector on a dword and loads no fifth
    dword: offsets (0, 0), (1, 0), (0, 1) and (1, 3) give both, B, A and neither operand that form."""
    M, N, K, batch = 137, 75, 203, 2
    monkeypatch.setenv("TSM_GEMM_KERNEL", variant)
    for a_layout in ("row", "col"):
        for b_layout in ("row", "col"):
            A, B = make_operands(M + N + K + offsets[0], batch, M, N, K, BF16, ("uniform", -1.0, 1.0), a_layout,
                                 b_layout)
            # padding on odd extents: pad 2 gives odd leading dimensions (consecutive rows alternate between 0 and
            # 2 mod 4 bytes) and odd batch strides (odd rows times odd ld); pad 1 gives even ones
            Ap = np.zeros(A.shape[:2] + (A.shape[2] + pad,), np.uint16)
            Ap[:, :, :A.shape[2]] = A
            Bp = np.zeros(B.shape[:2] + (B.shape[2] + pad,), np.uint16)
            Bp[:, :, :B.shape[2]] = B
            odd = pad % 2 == 0
            assert all(bool(x % 2) == odd for x in (Ap.shape[2], Bp.shape[2], Ap[0].size, Bp[0].size))
            say(f"[gpu] {variant} realigned offsets={offsets} pad={pad} A:{a_layout} B:{b_layout}")
            C = run(Ap, Bp, M, N, K, BF16, "f32", batch=batch, a_layout=a_layout, b_layout=b_layout,
                    lda=Ap.shape[2], ldb=Bp.shape[2], a_off=offsets[0], b_off=offsets[1], fill=float("nan"),
                    kernel=variant)
            Cr, S = orc.gemm_rows(A, B, M, N, K, BF16, batch=batch, a_layout=a_layout, b_layout=b_layout)
            check(C, Cr, S, K, "f32", f"{variant} offsets={offsets} pad={pad} {a_layout}/{b_layout}")


@pytest.mark.parametrize("shape", EDGE_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("in_fmt,out_fmt", [(F16, "f32"), (BF16, "f16"), (F16, "f16"), (BF16, "f32")])
def test_edge_shapes(orc, shape, in_fmt, out_fmt):
    M, N, K = shape
    for a_layout in ("row", "col"):
        for b_layout in ("row", "col"):
            A, B = make_operands(M * 7 + N * 3 + K, 1, M, N, K, in_fmt, ("uniform", -1.0, 1.0), a_layout, b_layout)
            say(f"[gpu] edge {M}x{N}x{K} {in_fmt}->{out_fmt} A:{a_layout} B:{b_layout}")
            C = run(A, B, M, N, K, in_fmt, out_fmt, a_layout=a_layout, b_layout=b_layout)
            Cr, S = orc.gemm_rows(A, B, M, N, K, in_fmt, a_layout=a_layout, b_layout=b_layout)
            check(C, Cr, S, K, out_fmt, f"{shape} {a_layout}/{b_layout}")


@pytest.mark.parametrize("a_off,b_off", [(0, 0), (1, 0), (0, 1), (3, 5)])
def test_padded_and_unaligned_operands(orc, a_off, b_off):
    """Padded leading dimensions and operands starting at odd element offsets (2-byte alignment only)."""
    M, N, K = 100, 136, 72
    lda, ldb, ldc = K + 9, N + 8, N + 5
    A, B = make_operands(5, 1, M, N, K, F16, ("uniform", -1.0, 1.0))
    Ap = np.zeros((1, M, lda), np.uint16)
    Ap[:, :, :K] = A
    Bp = np.zeros((1, K, ldb), np.uint16)
    Bp[:, :, :N] = B
    say(f"[gpu] padded lda={lda} ldb={ldb} ldc={ldc} offsets {a_off},{b_off}")
    C = run(Ap, Bp, M, N, K, F16, "f32", lda=lda, ldb=ldb, ldc=ldc, a_off=a_off, b_off=b_off)
    Cr, S = orc.gemm_rows(A, B, M, N, K, F16)
    check(C, Cr, S, K, "f32", "padded")


def test_ldc_padding_untouched_and_inside_overwritten():
    """Prefill C with a sentinel: every logical cell is overwritten, the ld padding keeps its bits."""
    import torch

    M, N, K, ldc = 70, 90, 40, 97
    A, B = integer_operands(9, 1, M, N, K, F16)
    for fill in (100.0, float("nan")):
        say(f"[gpu] sentinel fill {fill}")
        C, raw = run(A, B, M, N, K, F16, "f32", ldc=ldc, fill=fill, keep=True)
        host = raw.cpu().numpy()
        ai = np.asarray(A[0].view(np.float16), np.float64)
        bi = np.asarray(B[0].view(np.float16), np.float64)
        want = ai @ bi
        assert np.array_equal(C[0], want)
        for i in range(M):
            pad = host[i * ldc + N:(i + 1) * ldc] if i < M - 1 else host[i * ldc + N:i * ldc + N]
            if np.isnan(fill):
                assert np.all(np.isnan(pad))
            else:
                assert np.all(pad == fill)
        tail = host[(M - 1) * ldc + N:]
        assert np.all(np.isnan(tail)) if np.isnan(fill) else np.all(tail == fill)
        torch.cuda.synchronize()



@pytest.mark.parametrize("out_fmt", ["f32", "f16"])
def test_masked_wide_ldc(out_fmt):
    """C rows 2^23 + 8 elements apart: with float32 output, 64 rows of C span more than 2^31 bytes and the general
    kernel's stores take 64-bit addresses; with f16 output they stay relative to the tile's corner, at offsets up
    to 2^30.  Exact integer products; the padding between rows keeps its NaN fill."""
    import torch

    M, N, K, ldc = 5, 72, 96, (1 << 23) + 8
    A, B = integer_operands(21, 1, M, N, K, F16)
    say(f"[gpu] wide ldc {ldc} {out_fmt}")
    C, raw = run(A, B, M, N, K, F16, out_fmt, ldc=ldc, fill=float("nan"), keep=True, kernel="masked_64x64x64")
    ai = np.asarray(A[0].view(np.float16), np.float64)
    bi = np.asarray(B[0].view(np.float16), np.float64)
    want = ai @ bi
    if out_fmt == "f16":
        want = want.astype(np.float16).astype(np.float64)
    assert np.array_equal(C[0], want)
    host = raw.cpu().numpy()
    for i in range(M - 1):
        gap = host[i * ldc + N:i * ldc + N + 4096]
        assert np.all(np.isnan(gap.astype(np.float32))), i
        assert np.all(np.isnan(host[(i + 1) * ldc - 4096:(i + 1) * ldc].astype(np.float32))), i
    torch.cuda.synchronize()


TILE = "tile_256x256x"
TILE_SHAPES = [(256, 256, 128, 1), (512, 768, 384, 1), (256, 512, 1024, 3), (768, 256, 256, 2)]
# every large-tile variant with the B layout it reads
TILE_VARIANTS = [("tile_256x256x32_mi32", "col"), ("tile_256x256x32_mi16", "col"), ("tile_256x256x32_mi16_nn", "row"),
                 ("tile_256x256x64_mi16", "col"), ("tile_256x256x64_mi16_nn", "row"), ("tile_256x256x64_mi16_st", "col")]


@pytest.mark.parametrize("shape", TILE_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("in_fmt,out_fmt", [(BF16, "f16"), (F16, "f32"), (BF16, "f32"), (F16, "f16")])
@pytest.mark.parametrize("variant,b_layout", TILE_VARIANTS, ids=[v for v, _ in TILE_VARIANTS])
def test_tile_kernel(orc, monkeypatch, shape, in_fmt, out_fmt, variant, b_layout):
    """Each large-tile variant (A row-major, 256-multiples, K % 128 == 0; 32- or 64-deep K slabs; B K-contiguous
    or row-major, the latter through the LDS transpose reads) against the oracle."""
    monkeypatch.setenv("TSM_GEMM_KERNEL", variant)
    M, N, K, batch = shape
    A, B = make_operands(M + N + K + batch, batch, M, N, K, in_fmt, ("uniform", -1.0, 1.0), "row", b_layout)
    say(f"[gpu] {variant} {shape} {in_fmt}->{out_fmt}")
    C = run(A, B, M, N, K, in_fmt, out_fmt, batch=batch, a_layout="row", b_layout=b_layout, kernel=variant)
    Cr, S = orc.gemm_rows(A, B, M, N, K, in_fmt, batch=batch, a_layout="row", b_layout=b_layout)
    check(C, Cr, S, K, out_fmt, f"{variant} {shape}")


@pytest.mark.parametrize("variant", ["tile_256x256x32_mi16_nn", "tile_256x256x64_mi16_nn"])
def test_tile_nn_padded_ld_and_strides(orc, monkeypatch, variant):
    """Row-major B with padded ldb (rows of N + 8) and batch strides larger than the matrices."""
    monkeypatch.setenv("TSM_GEMM_KERNEL", variant)
    M, N, K, batch = 512, 256, 384, 2
    lda, ldb, ldc = K + 8, N + 8, N + 12
    A, B = make_operands(98, batch, M, N, K, F16, ("uniform", -1.0, 1.0), "row", "row")
    Ap = np.zeros((batch, M, lda), np.uint16)
    Ap[:, :, :K] = A
    Bp = np.zeros((batch, K + 3, ldb), np.uint16)
    Bp[:, :K, :N] = B
    say(f"[gpu] {variant} padded")
    C = run(Ap, Bp, M, N, K, F16, "f16", batch=batch, lda=lda, ldb=ldb, ldc=ldc, sC=M * ldc + 4, kernel=variant)
    Cr, S = orc.gemm_rows(A, B, M, N, K, F16, batch=batch)
    check(C, Cr, S, K, "f16", "tile nn padded")


def test_tile_nn_large_sampled(orc):
    """A 4096 x 4096 x 4096 row-major product on the default transpose-read kernel, checked on sampled cells."""
    M = N = K = 4096
    A, B = make_operands(97, 1, M, N, K, BF16, ("normal", 1.0 / 64.0), "row", "row")
    say("[gpu] tile nn 4096^3 sampled")
    C = run(A, B, M, N, K, BF16, "f32", kernel=TILE)
    rng = np.random.default_rng(11)
    z, i, j = _sample_cells(rng, 1, M, N, 2000)
    Cp, Sp = orc.gemm_points(A, B, M, N, K, BF16, z, i, j)
    check(C[z, i, j], Cp, Sp, K, "f32", "tile nn 4096 sampled")


@pytest.mark.parametrize("variant", ["tile_256x256x32_mi16", "tile_256x256x64_mi16", "tile_256x256x64_mi16_st"])
def test_tile_kernel_padded_ld_and_strides(orc, monkeypatch, variant):
    """Padded lda/ldb/ldc and batch strides larger than the matrices, still on the tile kernel."""
    monkeypatch.setenv("TSM_GEMM_KERNEL", variant)
    M, N, K, batch = 256, 512, 256, 2
    lda, ldb, ldc = K + 64, K + 8, N + 4
    A, B = make_operands(99, batch, M, N, K, BF16, ("uniform", -1.0, 1.0), "row", "col")
    Ap = np.zeros((batch, M, lda), np.uint16)
    Ap[:, :, :K] = A
    Bp = np.zeros((batch, N, ldb), np.uint16)
    Bp[:, :, :K] = B
    say("[gpu] tile kernel padded")
    C = run(Ap, Bp, M, N, K, BF16, "f32", batch=batch, a_layout="row", b_layout="col", lda=lda, ldb=ldb, ldc=ldc,
            sC=M * ldc + 12, kernel=variant)
    Cr, S = orc.gemm_rows(A, B, M, N, K, BF16, batch=batch, a_layout="row", b_layout="col")
    check(C, Cr, S, K, "f32", f"{variant} padded")


@pytest.mark.parametrize("variant", ["tile_256x256x32_mi16", "tile_256x256x64_mi16", "tile_256x256x64_mi16_st"])
@pytest.mark.parametrize("out_fmt", ["f16", "bf16"])
def test_staged_epilogue_ragged_and_misaligned_rows(orc, monkeypatch, variant, out_fmt):
    """16-bit output through the LDS-staged epilogue: ragged M and N (rows and 8-column groups past them are not
    stored), ldc = N + 4, so every other row of C starts 8 bytes off a 16-byte boundary, and a batch stride that
    shifts the second problem by 8 bytes; C prefilled with NaN, its padding and the rows past M must stay NaN."""
    monkeypatch.setenv("TSM_GEMM_KERNEL", variant)
    M, N, K, batch = 300, 264, 256, 2
    ldc = N + 4
    sC = (M + 3) * ldc  # 81204 elements: 4 mod 8
    A, B = make_operands(103, batch, M, N, K, BF16, ("uniform", -1.0, 1.0), "row", "col")
    say(f"[gpu] staged epilogue {variant} {out_fmt} ldc={ldc} sC={sC}")
    C, raw = run(A, B, M, N, K, BF16, out_fmt, batch=batch, a_layout="row", b_layout="col", ldc=ldc, sC=sC,
                 kernel=variant, fill=float("nan"), keep=True)
    Cr, S = orc.gemm_rows(A, B, M, N, K, BF16, batch=batch, a_layout="row", b_layout="col")
    check(C, Cr, S, K, out_fmt, f"{variant} staged epilogue")
    host = raw.float().cpu().numpy()
    for z in range(batch):
        for i in range(M - 1):
            assert np.all(np.isnan(host[z * sC + i * ldc + N:z * sC + (i + 1) * ldc])), f"padding of row {i} written"
    # the first problem's last row padding and its three spare rows, up to the second problem
    assert np.all(np.isnan(host[(M - 1) * ldc + N:sC])), "C past the first problem's rows was written"
    assert np.all(np.isnan(host[sC + (M - 1) * ldc + N:])), "C past the last row was written"


SKINNY = "skinny_"
SKINNY_SHAPES = [(16, 256, 256, 1), (1, 512, 256, 1), (5, 256, 512, 3), (16, 768, 1024, 2), (12, 256, 256, 2)]


def skinny_variant(M, width, b_layout="row"):
    """Kernel name of the skinny variant for M rows at the given workgroup width (suffix _t: K-contiguous B)."""
    mb = 1 if M <= 16 else 2 if M <= 32 else 4 if M <= 64 else 8
    return f"skinny_m{16 * mb}_n{width}_k64" + ("_t" if b_layout == "col" else "")


@pytest.mark.parametrize("shape", SKINNY_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("in_fmt,out_fmt", [(F16, "f32"), (BF16, "f16"), (F16, "f16"), (BF16, "f32")])
def test_skinny_kernel(orc, shape, in_fmt, out_fmt):
    """The streaming kernel for few rows (row-major A and B) against the oracle, rows past M masked."""
    M, N, K, batch = shape
    A, B = make_operands(M * 1000 + N + K + batch, batch, M, N, K, in_fmt, ("uniform", -1.0, 1.0))
    say(f"[gpu] skinny kernel {shape} {in_fmt}->{out_fmt}")
    C = run(A, B, M, N, K, in_fmt, out_fmt, batch=batch, kernel=SKINNY)
    Cr, S = orc.gemm_rows(A, B, M, N, K, in_fmt, batch=batch)
    check(C, Cr, S, K, out_fmt, f"skinny {shape}")


# every row-block count at both widths (256 only up to 64 rows); M ragged inside its last 16-row block; K from
# one 64-deep slice (the rest of the ring's first round loads zeros) to several rounds plus a partial one
SKINNY_VARIANT_SHAPES = [(1, 64), (13, 64), (16, 256), (17, 64), (30, 256), (32, 64), (33, 64), (47, 256), (64, 64),
                         (65, 64), (100, 64), (128, 64), (5, 128), (32, 128), (49, 128), (64, 128), (97, 128),
                         (128, 128)]
SKINNY_K = [64, 192, 576, 1344]


@pytest.mark.parametrize("M,width", SKINNY_VARIANT_SHAPES, ids=lambda v: str(v))
@pytest.mark.parametrize("K", SKINNY_K)
@pytest.mark.parametrize("b_layout", ["row", "col"])
def test_skinny_variants(orc, monkeypatch, M, width, K, b_layout):
    """Each skinny variant (16, 32, 64 or 128 rows; 64, 128 or 256 columns per workgroup; row-major or
    K-contiguous B) forced, against the oracle."""
    variant = skinny_variant(M, width, b_layout)
    N, batch = {256: (512, 2), 128: (384, 2), 64: (320, 3)}[width]
    monkeypatch.setenv("TSM_GEMM_KERNEL", variant)
    in_fmt, out_fmt = [(F16, "f32"), (BF16, "f16"), (BF16, "bf16"), (F16, "f16")][(M + K) % 4]
    A, B = make_operands(M * 7 + K + width, batch, M, N, K, in_fmt, ("uniform", -1.0, 1.0), "row", b_layout)
    say(f"[gpu] {variant} M={M} N={N} K={K} batch={batch} {in_fmt}->{out_fmt}")
    C = run(A, B, M, N, K, in_fmt, out_fmt, batch=batch, b_layout=b_layout, kernel=variant)
    Cr, S = orc.gemm_rows(A, B, M, N, K, in_fmt, batch=batch, b_layout=b_layout)
    check(C, Cr, S, K, out_fmt, f"{variant} K={K}")


@pytest.mark.parametrize("M,width", [(7, 256), (7, 64), (40, 64), (90, 64)], ids=lambda v: str(v))
def test_skinny_kernel_padded_and_sentinel(orc, monkeypatch, M, width):
    """Padded lda/ldb/ldc holding NaN, C prefilled: the padding is never read, and rows of C past M and the ld
    padding keep their bits."""
    variant = skinny_variant(M, width)
    monkeypatch.setenv("TSM_GEMM_KERNEL", variant)
    N, K, batch = 512, 256, 2
    lda, ldb, ldc = K + 24, N + 64, N + 8
    A, B = make_operands(77 + M, batch, M, N, K, F16, ("uniform", -1.0, 1.0))
    nan16 = np.uint16(0x7E00)
    Ap = np.full((batch, M, lda), nan16, np.uint16)
    Ap[:, :, :K] = A
    Bp = np.full((batch, K, ldb), nan16, np.uint16)
    Bp[:, :, :N] = B
    rows_c = M + 3
    sC = rows_c * ldc
    say(f"[gpu] {variant} padded + sentinel M={M}")
    C, raw = run(Ap, Bp, M, N, K, F16, "f32", batch=batch, lda=lda, ldb=ldb, ldc=ldc, sC=sC, fill=100.0, keep=True,
                 kernel=variant)
    Cr, S = orc.gemm_rows(A, B, M, N, K, F16, batch=batch)
    check(C, Cr, S, K, "f32", f"{variant} padded")
    host = raw.cpu().numpy()
    for z in range(batch):
        for i in range(M):
            o = z * sC + i * ldc
            assert np.all(host[o + N:o + ldc] == 100.0)
        if z < batch - 1:
            assert np.all(host[z * sC + M * ldc:(z + 1) * sC] == 100.0)


def test_skinny_col_b_padded(orc, monkeypatch):
    """K-contiguous B with padded ldb holding NaN past K: the padding is never read."""
    variant = "skinny_m32_n64_k64_t"
    monkeypatch.setenv("TSM_GEMM_KERNEL", variant)
    M, N, K, batch = 24, 192, 640, 2
    ldb = K + 40
    A, B = make_operands(78, batch, M, N, K, F16, ("uniform", -1.0, 1.0), "row", "col")
    Bp = np.full((batch, N, ldb), np.uint16(0x7E00), np.uint16)
    Bp[:, :, :K] = B
    say("[gpu] skinny col-B padded")
    C = run(A, Bp, M, N, K, F16, "f32", batch=batch, b_layout="col", ldb=ldb, kernel=variant)
    Cr, S = orc.gemm_rows(A, B, M, N, K, F16, batch=batch, b_layout="col")
    check(C, Cr, S, K, "f32", "skinny col-B padded")


def test_skinny_decode_sampled(orc):
    """A decode-sized product, 48 x 16384 x 8192 (one problem: the 64-column workgroups), on sampled cells."""
    M, N, K = 48, 16384, 8192
    A, B = make_operands(4242, 1, M, N, K, F16, ("uniform", -0.5, 0.5))
    say("[gpu] skinny decode 48x16384x8192 sampled")
    C = run(A, B, M, N, K, F16, "f32", kernel="skinny_m64_n64_k64")
    rng = np.random.default_rng(12)
    z, i, j = _sample_cells(rng, 1, M, N, 3000)
    Cp, Sp = orc.gemm_points(A, B, M, N, K, F16, z, i, j)
    check(C[z, i, j], Cp, Sp, K, "f32", "skinny decode sampled")


SPLITK = "splitk_"
SPLITK_SHAPES = [(16, 16, 2048, 1), (256, 256, 8192, 1), (48, 80, 4096, 2), (128, 32, 2048, 3)]


@pytest.mark.parametrize("shape", SPLITK_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("in_fmt,out_fmt", [(F16, "f32"), (BF16, "f16"), (BF16, "f32")])
@pytest.mark.parametrize("b_layout", ["row", "col"])
def test_splitk_kernel(orc, shape, in_fmt, out_fmt, b_layout):
    """The deep-K kernel (16 x 16 tiles, K split over 16 waves, fixed-order LDS reduction) against the oracle,
    with B row-major (transposed out of LDS) or K-contiguous."""
    M, N, K, batch = shape
    A, B = make_operands(M + 7 * N + K + batch, batch, M, N, K, in_fmt, ("uniform", -1.0, 1.0), "row", b_layout)
    say(f"[gpu] splitk kernel {shape} {in_fmt}->{out_fmt} B {b_layout}")
    C = run(A, B, M, N, K, in_fmt, out_fmt, batch=batch, b_layout=b_layout, kernel=SPLITK)
    Cr, S = orc.gemm_rows(A, B, M, N, K, in_fmt, batch=batch, b_layout=b_layout)
    check(C, Cr, S, K, out_fmt, f"splitk {shape}")
    # deterministic: the reduction order is fixed
    assert np.array_equal(run(A, B, M, N, K, in_fmt, out_fmt, batch=batch, b_layout=b_layout, kernel=SPLITK), C)


@pytest.mark.parametrize("M,N,batch", [(33, 65, 1), (33, 65, 3), (300, 520, 2)])
def test_k_zero_writes_zeros(M, N, batch):
    """K = 0: C is the empty sum, zeros in every problem of a batch (the batch runs as one flat grid), and the
    ld padding stays untouched."""
    A = np.zeros((batch, M, 0), np.uint16)
    B = np.zeros((batch, 0, N), np.uint16)
    say(f"[gpu] K=0 {M}x{N} batch {batch}")
    C, raw = run(A, B, M, N, 0, F16, "f32", batch=batch, lda=1, ldb=N, ldc=N + 3, sA=0, sB=0, fill=float("nan"),
                 keep=True)
    assert np.all(C == 0.0)
    host = raw.cpu().numpy()[:batch * M * (N + 3)].reshape(batch, M, N + 3)
    assert np.all(np.isnan(host[:, :, N:])), "ld padding written"


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_integer_inputs_bit_exact(orc, name):
    """Entries in {-1, 0, 1}: every float32 partial sum is exact, so the GPU matches the oracle bit for bit
    (f16 output: exact while |C| <= 2048, else within half an ulp)."""
    w = WORKLOADS[name]
    batch = min(w.batch, 2)
    A, B = integer_operands(31, batch, w.M, w.N, w.K, w.in_fmt, -1, 1, w.a_layout, w.b_layout)
    say(f"[gpu] integer {name}")
    C = run(A, B, w.M, w.N, w.K, w.in_fmt, w.out_fmt, batch=batch, a_layout=w.a_layout, b_layout=w.b_layout)
    rng = np.random.default_rng(5)
    z, i, j = _sample_cells(rng, batch, w.M, w.N, 4000)
    Cp, _ = orc.gemm_points(A, B, w.M, w.N, w.K, w.in_fmt, z, i, j, strideA=A[0].size, strideB=B[0].size,
                            a_layout=w.a_layout, b_layout=w.b_layout)
    got = C[z, i, j]
    if w.out_fmt == "f32":
        assert np.array_equal(got, Cp)
    else:
        small = np.abs(Cp) <= 2048
        assert np.array_equal(got[small], Cp[small])
        assert np.all(np.abs(got - Cp) <= oracle.half_ulp_f16(got))


def test_batched_equals_single(orc):
    """Problem z of a strided batch equals a single gemm on problem z, bit for bit."""
    M, N, K, batch = 40, 72, 200, 5
    A, B = make_operands(12, batch, M, N, K, BF16, ("uniform", -1.0, 1.0))
    say("[gpu] batched vs single")
    Cb = run(A, B, M, N, K, BF16, "f32", batch=batch)
    for z in range(batch):
        Cs = run(A[z:z + 1], B[z:z + 1], M, N, K, BF16, "f32")
        assert np.array_equal(Cb[z], Cs[0])
    Cr, S = orc.gemm_rows(A, B, M, N, K, BF16, batch=batch)
    check(Cb, Cr, S, K, "f32", "batched")


def test_broadcast_operand(orc):
    """strideB = 0: every problem multiplies by the same B."""
    M, N, K, batch = 20, 48, 64, 3
    A, B = make_operands(13, batch, M, N, K, F16, ("uniform", -1.0, 1.0))
    say("[gpu] broadcast B")
    C = run(A, B[:1], M, N, K, F16, "f32", batch=batch, sB=0)
    Cr, S = orc.gemm_rows(A, np.repeat(B[:1], batch, 0), M, N, K, F16, batch=batch)
    check(C, Cr, S, K, "f32", "broadcast")


def test_subnormal_f16_operands(orc):
    """f16 subnormals are real inputs (uniform draws produce a few); they must not be flushed."""
    M, N, K = 4, 4, 32
    A = np.full((1, M, K), 0x0001, np.uint16)     # 2^-24
    B = np.full((1, K, N), 0x3C00, np.uint16)     # 1.0
    say("[gpu] f16 subnormal inputs")
    C = run(A, B, M, N, K, F16, "f32")
    Cr, S = orc.gemm_rows(A, B, M, N, K, F16)
    assert np.all(Cr == K * 2.0 ** -24)
    check(C, Cr, S, K, "f32", "subnormal")


COL_A_VARIANTS = [("tile_256x256x32_mi16_tn", "row"), ("tile_256x256x32_mi16_tt", "col"),
                  ("tile_256x256x64_mi16_tt", "col")]
COL_A_SHAPES = [(256, 256, 128, 1), (512, 768, 384, 1), (264, 520, 256, 2), (1000, 256, 512, 1)]


@pytest.mark.parametrize("shape", COL_A_SHAPES, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("in_fmt,out_fmt", [(BF16, "f16"), (F16, "f32")])
@pytest.mark.parametrize("variant,b_layout", COL_A_VARIANTS, ids=[v for v, _ in COL_A_VARIANTS])
def test_tile_col_a(orc, monkeypatch, shape, in_fmt, out_fmt, variant, b_layout):
    """Column-major A (M-contiguous, as in a product with a transposed operand) on the large-tile kernel: its
    slices are transposed out of LDS like a row-major B.  M is a multiple of 8 but not always of 256; A is stored
    with padding rows of NaN beyond M, which must not leak."""
    monkeypatch.setenv("TSM_GEMM_KERNEL", variant)
    M, N, K, batch = shape
    A, B = make_operands(M + 2 * N + K + batch, batch, M, N, K, in_fmt, ("uniform", -1.0, 1.0), "col", b_layout)
    lda = M + 24
    Ap = np.full((batch, K, lda), 0x7E00 if in_fmt == F16 else 0x7FC0, np.uint16)
    Ap[:, :, :M] = A
    say(f"[gpu] {variant} {shape} {in_fmt}->{out_fmt}")
    C = run(Ap, B, M, N, K, in_fmt, out_fmt, batch=batch, a_layout="col", b_layout=b_layout, lda=lda,
            ldc=N + 4, fill=float("nan"), kernel=variant)
    Cr, S = orc.gemm_rows(A, B, M, N, K, in_fmt, batch=batch, a_layout="col", b_layout=b_layout)
    check(C, Cr, S, K, out_fmt, f"{variant} {shape}")


RAGGED_N = [(600, 1000, 256, 1), (256, 8, 128, 2), (300, 264, 384, 1), (512, 1304, 128, 1)]


@pytest.mark.parametrize("shape", RAGGED_N, ids=lambda s: "x".join(map(str, s)))
@pytest.mark.parametrize("variant,b_layout", TILE_VARIANTS, ids=[v for v, _ in TILE_VARIANTS])
def test_tile_ragged_n(orc, monkeypatch, shape, variant, b_layout):
    """N a multiple of 8 but not of 256 (and ragged M) on every large-tile variant.  Row-major B is stored with
    padding columns full of NaN and C with padding full of NaN: neither may leak into or be written by the
    result."""
    monkeypatch.setenv("TSM_GEMM_KERNEL", variant)
    M, N, K, batch = shape
    A, B = make_operands(M + N + K, batch, M, N, K, BF16, ("uniform", -1.0, 1.0), "row", b_layout)
    nan16 = 0x7E00 if BF16 == "f16" else 0x7FC0  # a quiet NaN pattern of the operand format
    if b_layout == "row":
        ldb = N + 24
        Bp = np.full((batch, K, ldb), nan16, np.uint16)
        Bp[:, :, :N] = B
    else:
        ldb = K
        Bp = B
    ldc = N + 8
    say(f"[gpu] ragged N {variant} {shape}")
    C, raw = run(A, Bp, M, N, K, BF16, "f32", batch=batch, b_layout=b_layout, ldb=ldb, ldc=ldc, fill=float("nan"),
                 keep=True, kernel=variant)
    Cr, S = orc.gemm_rows(A, B, M, N, K, BF16, batch=batch, b_layout=b_layout)
    check(C, Cr, S, K, "f32", f"{variant} ragged N {shape}")
    host = raw.cpu().numpy()
    for z in range(batch):
        for i in range(M):
            o = z * M * ldc + i * ldc
            assert np.all(np.isnan(host[o + N:o + ldc])), f"C padding written at problem {z} row {i}"


def test_batch_larger_than_one_flat_grid(orc):
    """A batch whose tiles would need 2^32 or more work-items in one 1-D grid (2^24 + 3 problems of one 64 x 64
    tile, 256 threads each) runs as 2-D grids of at most 65535 problems.  A and B are broadcast (stride 0), so
    every problem's C equals the oracle's one product; C starts as NaN, so an unwritten problem fails."""
    import torch

    M = N = K = 16
    batch = (1 << 24) + 3
    A, B = make_operands(5, 1, M, N, K, F16, ("uniform", -1.0, 1.0), "row", "row")
    a_buf, a_ptr = to_device(A)
    b_buf, b_ptr = to_device(B)
    c = torch.full((batch * M * N,), float("nan"), dtype=torch.float16, device="cuda")
    args = (M, N, K, a_ptr, K, LAYOUT["row"], 0, b_ptr, N, LAYOUT["row"], 0, c, N, M * N, batch, DTYPE[(F16, "f16")])
    assert tsm.tsm_gemm_kernel_name(*args).startswith("masked_")
    say(f"[gpu] broadcast batch of {batch} problems {M}x{N}x{K}")
    tsm.gemm_strided_batched_ex(*args, 0)
    torch.cuda.synchronize()
    cv = c.view(batch, M * N)
    assert bool(torch.isfinite(cv).all())
    assert bool((cv == cv[0]).all())
    Cr, S = orc.gemm_rows(A, B, M, N, K, F16)
    first = cv[0].float().cpu().numpy().astype(np.float64).reshape(1, M, N)
    check(first, Cr, S, K, "f16", "broadcast batch")
