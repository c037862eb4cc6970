"""The oracle against its pins (CPU only).  See tests/oracle_pins.py for what
each pin ties the oracle to."""
import pytest

import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_pin(orc, pin):
    fails = pin(orc)
    assert not fails, "\n".join(fails[:20])


def test_exact_reference_rounding_helper():
    """The test-side rational rounding agrees with struct's binary16 codec on
    values that are exactly representable or exact midpoints."""
    import struct
    from fractions import Fraction

    for bits in list(range(0, 0x7C00, 97)) + [0x0001, 0x03FF, 0x0400, 0x7BFF]:
        v = struct.unpack("<e", struct.pack("<H", bits))[0]
        assert P.fraction_to_fp16_bits(Fraction(v)) == bits
    # midpoint 2^-25 ties to 0, 3*2^-25 ties to 2 quanta, 65520 overflows
    assert P.fraction_to_fp16_bits(Fraction(1, 2 ** 25)) == 0
    assert P.fraction_to_fp16_bits(Fraction(3, 2 ** 25)) == 2
    assert P.fraction_to_fp16_bits(Fraction(65520)) == 0x7C00
    assert P.fraction_to_fp16_bits(Fraction(65519)) == 0x7BFF
    assert P.fraction_to_fp16_bits(Fraction(2049)) == 0x6800
