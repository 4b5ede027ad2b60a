"""The CPU oracle against what fixes its answers independently of itself.

Each pin is defined in tests/pins.py with the source of its expected values.
"""

import pytest

import pins


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_pin_holds(pin):
    assert pin(None) is None


def test_round_to_f32_definition():
    """The rational rounding helper used by the float32-model pin is itself
    checked against numpy's float64→float32 conversion on values exact in
    float64 (a single rounding there), including ties and subnormals."""
    import numpy as np
    from fractions import Fraction

    rng = np.random.default_rng(5)
    vals = list(rng.standard_normal(2000) * 2.0 ** rng.integers(-140, 100, 2000))
    one = 1.0
    ulp = 2.0 ** -23
    vals += [one + ulp / 2, one + 3 * ulp / 2, -(one + ulp / 2), 2.0 ** -149 / 2 * 3,
             2.0 ** -149 / 2, 0.0, 2.0 ** -126 * (1 - 2.0 ** -24)]
    for v in vals:
        got = pins.round_to_f32(Fraction(float(v)))
        want = float(np.float32(v))
        assert got == want, (v, got, want)
