"""Seeded input generators (CPU only)."""

import numpy as np
import pytest

from workloads import WORKLOADS
from workloads.inputs import BF16, F16, bits_to_f64, draw_matrix_bits, make_operands, round_f64_to_bits


def _edge_values():
    v = [0.0, -0.0, 1.0, -1.0, 65504.0, 65520.0, 65519.99, 1e6, -1e6, 2.0 ** -24, 2.0 ** -25,
         3 * 2.0 ** -26, 2.0 ** -26, 2.0 ** -14, 2.0 ** -14 - 2.0 ** -25, 1.0 + 2.0 ** -11,
         1.0 + 3 * 2.0 ** -11, 1.0 + 2.0 ** -11 + 2.0 ** -40, np.inf, -np.inf, 5e-324, 1e-300, 1e300]
    return np.array(v)


def test_f16_rounding_matches_numpy():
    rng = np.random.default_rng(0)
    x = np.concatenate([
        rng.uniform(-1, 1, 400000),
        rng.standard_normal(300000) * 1000.0,
        rng.uniform(-1, 1, 200000) * 2.0 ** -14,   # subnormal range
        np.exp2(rng.uniform(-30, 17, 100000)) * rng.choice([-1, 1], 100000),
        _edge_values(),
    ])
    # exact ties between f16 neighbours, both parities
    h = np.arange(0, 0x7BFF, 7, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).view(np.float16).astype(np.float64)
    x = np.concatenate([x, (lo + hi) / 2, -(lo + hi) / 2])
    got = round_f64_to_bits(x, F16)
    with np.errstate(over="ignore"):
        ref = x.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f16_nan():
    assert (round_f64_to_bits(np.array([np.nan]), F16)[0] & 0x7C00) == 0x7C00
    assert (round_f64_to_bits(np.array([np.nan]), F16)[0] & 0x3FF) != 0


def _nearest_bf16_bruteforce(x):
    """Nearest bf16 by comparing with both float32-truncation neighbours; ties to even."""
    out = np.empty(x.size, dtype=np.uint16)
    for t, v in enumerate(x):
        f = np.float32(v)  # not used for the answer, only to find candidates near v
        base = int(np.array([f], np.float32).view(np.uint32)[0] >> 16) & 0xFFFF
        cands = {(base + d) & 0xFFFF for d in (-2, -1, 0, 1, 2)}
        best = None
        for c in cands:
            cv = float((np.array([c << 16], np.uint32)).view(np.float32)[0])
            if np.isnan(cv) or np.isinf(cv):
                continue
            if (cv < 0) != (v < 0) and cv != 0:
                continue
            d = abs(cv - v)
            key = (d, c & 1)
            if best is None or key < best[0]:
                best = (key, c)
        out[t] = best[1]
    return out


def test_bf16_rounding_is_nearest_even():
    rng = np.random.default_rng(1)
    x = np.concatenate([rng.uniform(-1, 1, 3000), rng.standard_normal(3000) * 0.011,
                        np.exp2(rng.uniform(-130, 100, 2000)) * rng.choice([-1, 1], 2000)])
    # exact ties: midpoints of bf16 neighbours
    h = rng.integers(0x0080, 0x7F00, 500).astype(np.uint32)
    lo = (h << 16).view(np.float32).astype(np.float64)
    hi = ((h + 1) << 16).view(np.float32).astype(np.float64)
    x = np.concatenate([x, (lo + hi) / 2])
    got = round_f64_to_bits(x, BF16)
    ref = _nearest_bf16_bruteforce(x)
    # -0.0 / +0.0 patterns differ only for values that round to zero; compare values
    assert np.array_equal(bits_to_f64(got, BF16), bits_to_f64(ref, BF16))


def test_bf16_no_double_rounding():
    # 1 + 2^-8 + 2^-30: float32 rounding first would give the tie 1 + 2^-8, then even -> 1.0;
    # rounding straight from float64 must give 1 + 2^-7.
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -30])
    assert bits_to_f64(round_f64_to_bits(x, BF16), BF16)[0] == 1.0 + 2.0 ** -7


def test_values_do_not_depend_on_worker_count():
    for dist in (("uniform", -1.0, 1.0), ("normal", 0.5)):
        a = draw_matrix_bits(5, 1, 2, dist, 200, 29, F16, workers=1)
        b = draw_matrix_bits(5, 1, 2, dist, 200, 29, F16, workers=7)
        assert np.array_equal(a, b)


def test_blocks_are_distinct_streams():
    a = draw_matrix_bits(5, 0, 0, ("uniform", -1.0, 1.0), 128, 16, F16)
    assert not np.array_equal(a[:64], a[64:])
    b = draw_matrix_bits(5, 1, 0, ("uniform", -1.0, 1.0), 128, 16, F16)
    assert not np.array_equal(a, b)


def test_layout_is_storage_transpose():
    A1, B1 = make_operands(3, 2, 5, 6, 7, BF16, ("uniform", -1.0, 1.0), "row", "row")
    A2, B2 = make_operands(3, 2, 5, 6, 7, BF16, ("uniform", -1.0, 1.0), "col", "col")
    assert np.array_equal(A1, A2.transpose(0, 2, 1))
    assert np.array_equal(B1, B2.transpose(0, 2, 1))


def test_determinism_per_seed():
    w = WORKLOADS["single_f16_64x128x128"]
    A1, B1 = w.operands()
    A2, B2 = w.operands()
    assert np.array_equal(A1, A2) and np.array_equal(B1, B2)
    assert A1.shape == (1, 64, 128) and B1.shape == (1, 128, 128)
    a = bits_to_f64(A1, F16)
    assert a.min() >= -1.0 and a.max() <= 1.0 and a.std() > 0.5


@pytest.mark.parametrize("name", list(WORKLOADS))
def test_workload_definitions(name):
    w = WORKLOADS[name]
    lda, ldb, ldc = w.lds()
    assert ldc == w.N
    assert lda == (w.K if w.a_layout == "row" else w.M)
    assert ldb == (w.N if w.b_layout == "row" else w.K)
    assert w.flops == 2 * w.M * w.N * w.K * w.batch


def test_algorithmic_bytes():
    # A and B read once, C written once (f16 C for the square bf16 workload)
    assert WORKLOADS["single_f16_64x128x128"].bytes == 16384 + 32768 + 32768
    assert WORKLOADS["square_bf16_8192"].bytes == 3 * 8192 * 8192 * 2
    assert WORKLOADS["skinny_f16_16x16384x8192_b8"].bytes == 8 * (16 * 8192 * 2 + 8192 * 16384 * 2 + 16 * 16384 * 4)


@pytest.mark.parametrize("dist", [("normal", 0.0, 1.0), ("uniform", -1.0), ("laplace", 1.0)])
def test_malformed_distribution_is_rejected(dist):
    with pytest.raises(ValueError):
        draw_matrix_bits(0, 0, 0, dist, 4, 4, F16)
