"""The CPU oracle against its pins (no GPU needed)."""
import pytest

import oracle_pins


@pytest.mark.parametrize("pin", oracle_pins.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(oracle, pin):
    pin(oracle)


def test_exact_rounding_helper_matches_numpy():
    """The test-side exact rounding agrees with numpy on binary64 inputs, so the
    brute-force pin rests on two independent roundings."""
    from fractions import Fraction

    import numpy as np
    rng = np.random.default_rng(3)
    xs = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.integers(-9, 5, 2000),
                         [65519.99, 65520.0, 2.0 ** -25, 3 * 2.0 ** -26, 1 + 2.0 ** -11]])
    for x in xs:
        with np.errstate(over="ignore"):
            want = int(np.array([x]).astype(np.float16).view(np.uint16)[0])
        got = oracle_pins.exact_to_f16_bits(Fraction(float(x)))
        assert got == want or (want == 0x8000 and got == 0), (x, hex(got), hex(want))
