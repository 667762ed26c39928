"""The CPU oracle against its pins (CPU only)."""

import numpy as np
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(orc, pin):
    pin(orc)


def test_bf16_half_ulp_and_activation_helpers(orc):
    """half_ulp_bf16 is half the gap to the next bf16 value (every positive finite pattern, decoded by the
    oracle); the activations match their definitions on hand-picked values."""
    import oracle as o

    bits = np.arange(0x0001, 0x7F7F, dtype=np.uint32).astype(np.uint16)  # positive finite bf16 below the largest
    x = orc.decode(bits, "bf16")
    nxt = orc.decode((bits.astype(np.uint32) + 1).astype(np.uint16), "bf16")
    assert np.array_equal(o.half_ulp_bf16(x), (nxt - x) / 2)
    assert np.array_equal(o.half_ulp_bf16(-x), (nxt - x) / 2)
    v = np.array([-3.0, -0.5, -0.0, 0.0, 0.25, 7.0])
    assert np.array_equal(o.activate(v, o.ACT_NONE), v)
    assert np.array_equal(o.activate(v, o.ACT_RELU), [0.0, 0.0, 0.0, 0.0, 0.25, 7.0])
    assert np.array_equal(o.activate(v, o.ACT_LEAKY_RELU, 0.125), [-0.375, -0.0625, 0.0, 0.0, 0.25, 7.0])


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
