"""The CPU oracle against its pins (CPU only)."""

import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


def test_oracle_bound_helpers():
    import numpy as np

    import oracle

    # half an f16 ulp: 2^-11 at 1.0, 2^-25 at and below the subnormal range, 16 at 32768
    assert oracle.half_ulp_f16(np.array([1.0]))[0] == 2.0 ** -11
    assert oracle.half_ulp_f16(np.array([0.0]))[0] == 2.0 ** -25
    assert oracle.half_ulp_f16(np.array([2.0 ** -20]))[0] == 2.0 ** -25
    assert oracle.half_ulp_f16(np.array([-32768.0]))[0] == 16.0
    b = oracle.bound(8, np.array([2.0]), "f32")
    assert b[0] == 8 * 2.0 ** -24 * 2.0
