"""Epilogue variants against the oracle, through the C ABI: bf16 output and a fused activation.

Every kernel family is forced in turn (through TSM_GEMM_KERNEL) with f16 and
bf16 operands, bf16 output, and ReLU / leaky ReLU applied to the float32 result
before the conversion.  Acceptance: |C - act(C_ref)| <= oracle.bound(...).
"""

import numpy as np
import pytest

import oracle
from gpu_util import check, run, say
from workloads.inputs import BF16, F16, integer_operands, make_operands

import tiled_shared_memory_amd as tsm

pytestmark = pytest.mark.gpu

# (kernel, shape M x N x K x batch, A layout, B layout) that the kernel accepts
FAMILIES = [
    ("masked_128x128x32_vecu", (130, 257, 100, 2), "col", "row"),
    ("masked_128x128x32_vec8", (200, 136, 96, 1), "row", "col"),
    ("masked_64x64x64_vecu", (65, 63, 33, 3), "row", "row"),
    ("masked_64x64x64_vec8", (72, 80, 64, 1), "col", "col"),
    ("tile_256x256x64_mi16", (600, 512, 256, 2), "row", "col"),
    ("tile_256x256x64_mi16_st", (600, 512, 768, 2), "row", "col"),
    ("tile_256x256x32_mi16", (256, 512, 384, 1), "row", "col"),
    ("tile_256x256x32_mi32", (256, 256, 128, 1), "row", "col"),
    ("tile_256x256x32_mi16_nn", (512, 256, 256, 1), "row", "row"),
    ("tile_256x256x64_mi16_nn", (256, 256, 256, 2), "row", "row"),
    ("tile_256x256x32_mi16_tn", (264, 256, 256, 2), "col", "row"),
    ("tile_256x256x32_mi16_tt", (256, 264, 128, 1), "col", "col"),
    ("tile_256x256x64_mi16_tt", (520, 256, 256, 2), "col", "col"),
    ("skinny_m16_n256_k64", (13, 512, 512, 2), "row", "row"),
    ("skinny_m64_n64_k64", (40, 320, 192, 2), "row", "row"),
    ("skinny_m128_n64_k64", (100, 128, 128, 1), "row", "row"),
    ("skinny_m128_n128_k64", (100, 384, 192, 2), "row", "row"),
    ("skinny_m32_n128_k64", (20, 256, 320, 1), "row", "row"),
    ("splitk_16x16_w16", (48, 32, 4096, 1), "row", "row"),
    ("splitk_16x16_w16_t", (32, 48, 2048, 2), "row", "col"),
    ("skinny_m32_n64_k64_t", (20, 192, 320, 2), "row", "col"),
]
ACTS = [(tsm.TSM_ACT_NONE, 0.0), (tsm.TSM_ACT_RELU, 0.0), (tsm.TSM_ACT_LEAKY_RELU, 0.1),
        (tsm.TSM_ACT_LEAKY_RELU, -1.5)]


@pytest.mark.parametrize("family", FAMILIES, ids=[f[0] for f in FAMILIES])
@pytest.mark.parametrize("in_fmt,out_fmt", [(BF16, "bf16"), (F16, "bf16"), (F16, "f32"), (BF16, "f16")])
@pytest.mark.parametrize("act,slope", ACTS, ids=["none", "relu", "leaky0.1", "leaky-1.5"])
def test_epilogue(orc, monkeypatch, family, in_fmt, out_fmt, act, slope):
    variant, (M, N, K, batch), a_layout, b_layout = family
    monkeypatch.setenv("TSM_GEMM_KERNEL", variant)
    A, B = make_operands(M + N + K + act, batch, M, N, K, in_fmt, ("uniform", -1.0, 1.0), a_layout, b_layout)
    say(f"[gpu] epilogue {variant} {in_fmt}->{out_fmt} act={act} slope={slope}")
    C = run(A, B, M, N, K, in_fmt, out_fmt, batch=batch, a_layout=a_layout, b_layout=b_layout, kernel=variant,
            act=act, slope=slope)
    Cr, S = orc.gemm_rows(A, B, M, N, K, in_fmt, batch=batch, a_layout=a_layout, b_layout=b_layout)
    check(C, Cr, S, K, out_fmt, f"{variant} act={act}", act=act, slope=slope)
    if act == tsm.TSM_ACT_RELU:
        assert C.min() >= 0.0


def test_bf16_output_integer_exact(orc):
    """Integer entries with |C| <= 256: bf16 holds every such integer, so the output equals the oracle."""
    M, N, K = 512, 512, 128
    A, B = integer_operands(61, 1, M, N, K, BF16, -1, 1, "row", "col")
    say("[gpu] bf16 output integers")
    C = run(A, B, M, N, K, BF16, "bf16", b_layout="col")
    Cr, _ = orc.gemm_rows(A, B, M, N, K, BF16, b_layout="col")
    assert np.array_equal(C, Cr)


def test_activation_on_the_headline_kernel_sampled(orc):
    """4096^3 bf16 -> bf16 with leaky ReLU on the default (64-deep) kernel: sampled cells."""
    M = N = K = 4096
    A, B = make_operands(62, 1, M, N, K, BF16, ("normal", 1.0 / 64.0), "row", "col")
    say("[gpu] leaky ReLU 4096^3 bf16")
    C = run(A, B, M, N, K, BF16, "bf16", b_layout="col", kernel="tile_256x256x64_mi16",
            act=tsm.TSM_ACT_LEAKY_RELU, slope=0.01)
    rng = np.random.default_rng(63)
    z, i, j = np.zeros(3000, np.int64), rng.integers(0, M, 3000), rng.integers(0, N, 3000)
    Cp, Sp = orc.gemm_points(A, B, M, N, K, BF16, z, i, j, b_layout="col")
    check(C[z, i, j], Cp, Sp, K, "bf16", "leaky 4096", act=tsm.TSM_ACT_LEAKY_RELU, slope=0.01)
    assert np.any(C < 0) and np.any(C > 0)
