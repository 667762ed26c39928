"""Seeded random GEMM calls against the oracle (needs an MI355X).

Sizes are drawn around tile edges, layouts, padded leading dimensions, operand
base offsets, batches, all six dtype codes and the three activations at
random, and each call takes whatever kernel the library picks.  A few larger
aligned cases reach the large-tile kernels.  Every case prints its parameters
before it runs, so a failure names a reproducible case.
"""

import numpy as np
import pytest

from gpu_util import check, run, say
from workloads.inputs import BF16, F16, make_operands

import tiled_shared_memory_amd as tsm

pytestmark = pytest.mark.gpu

FORMATS = [(F16, "f32"), (F16, "f16"), (BF16, "f32"), (BF16, "f16"), (F16, "bf16"), (BF16, "bf16")]
EDGES = [1, 2, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]


def draw_case(i):
    rng = np.random.default_rng(1000 + i)

    def dim(hi):
        return int(rng.choice(EDGES)) if rng.random() < 0.5 else int(rng.integers(1, hi))

    M, N, K = dim(400), dim(400), dim(700)
    batch = int(rng.integers(1, 4))
    in_fmt, out_fmt = FORMATS[int(rng.integers(0, len(FORMATS)))]
    a_layout, b_layout = rng.choice(["row", "col"]), rng.choice(["row", "col"])
    pad = [int(rng.choice([0, 0, 1, 8, 13])) for _ in range(3)]
    off = [int(rng.choice([0, 0, 1, 3, 8])) for _ in range(2)]
    act = int(rng.integers(0, 3))
    slope = float(rng.choice([0.01, 0.5, -2.0]))
    return dict(M=M, N=N, K=K, batch=batch, in_fmt=in_fmt, out_fmt=out_fmt, a_layout=str(a_layout),
                b_layout=str(b_layout), pad=pad, off=off, act=act, slope=slope, seed=2000 + i)


def run_case(orc, c, kernel=None):
    M, N, K, batch = c["M"], c["N"], c["K"], c["batch"]
    A, B = make_operands(c["seed"], batch, M, N, K, c["in_fmt"], ("uniform", -1.0, 1.0), c["a_layout"],
                         c["b_layout"])
    # embed each stored matrix in a wider one (padded leading dimension)
    pa, pb, pc = c["pad"]
    Ap = np.zeros(A.shape[:2] + (A.shape[2] + pa,), np.uint16)
    Ap[:, :, :A.shape[2]] = A
    Bp = np.zeros(B.shape[:2] + (B.shape[2] + pb,), np.uint16)
    Bp[:, :, :B.shape[2]] = B
    ldc = N + pc
    C = run(Ap, Bp, M, N, K, c["in_fmt"], c["out_fmt"], batch=batch, a_layout=c["a_layout"], b_layout=c["b_layout"],
            lda=Ap.shape[2], ldb=Bp.shape[2], ldc=ldc, a_off=c["off"][0], b_off=c["off"][1], fill=float("nan"),
            act=c["act"], slope=c["slope"], kernel=kernel)
    Cr, S = orc.gemm_rows(A, B, M, N, K, c["in_fmt"], batch=batch, a_layout=c["a_layout"], b_layout=c["b_layout"])
    check(C, Cr, S, K, c["out_fmt"], str(c), act=c["act"], slope=c["slope"])


@pytest.mark.parametrize("i", range(160))
def test_random_call(orc, i):
    c = draw_case(i)
    say(f"[gpu] fuzz {i}: {c}")
    run_case(orc, c)


@pytest.mark.parametrize("case", [
    dict(M=3840, N=4104, K=256, batch=1, in_fmt=BF16, out_fmt="bf16", a_layout="row", b_layout="col", pad=[0, 0, 8],
         off=[0, 0], act=2, slope=0.25, seed=3001),
    dict(M=2000, N=4096, K=384, batch=2, in_fmt=F16, out_fmt="f16", a_layout="row", b_layout="row", pad=[8, 8, 0],
         off=[0, 0], act=1, slope=0.0, seed=3002),
    dict(M=16, N=1024, K=512, batch=3, in_fmt=F16, out_fmt="f32", a_layout="row", b_layout="row", pad=[0, 0, 0],
         off=[0, 0], act=0, slope=0.0, seed=3003),
], ids=["tile_col_b", "tile_row_b", "skinny"])
def test_aligned_large_call(orc, case):
    """Larger aligned calls that the library sends to its fast kernels."""
    say(f"[gpu] fuzz large {case}")
    kernel = {"col": "tile_256x256x64", "row": "tile_256x256x32_mi16_nn"}[case["b_layout"]] if case["M"] > 16 \
        else "skinny_"
    run_case(orc, case, kernel)
