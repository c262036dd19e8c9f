"""Pins of the oracle's codecs against the OCP format definitions.

The E2M1 value set and the E4M3 anchor values below are the published OCP
FP4/FP8 facts, typed here as numbers; the tie cases are worked by hand.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F

# OCP E2M1 magnitudes of codes 0..7
E2M1_SPEC = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_value_set():
    vals = F.e2m1_decode(np.arange(16))
    assert list(vals[:8]) == E2M1_SPEC
    assert list(-vals[8:]) == E2M1_SPEC
    assert np.signbit(vals[8])          # code 8 is -0


def test_e4m3_anchor_values():
    d = lambda b: float(F.e4m3_decode(b))
    assert d(0x7E) == 448.0             # largest finite
    assert d(0x01) == 2.0 ** -9         # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9     # largest subnormal
    assert d(0x08) == 2.0 ** -6         # smallest normal
    assert d(0x38) == 1.0
    assert d(0x39) == 1.125
    assert d(0x40) == 2.0
    assert d(0x00) == 0.0
    assert d(0xB8) == -1.0
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert F.E4M3_MAX == 448.0


def test_e4m3_monotone_and_spacing():
    v = F.e4m3_decode(np.arange(0x7F))
    assert np.all(np.diff(v) > 0)
    # 8 values per binade above the subnormals: spacing doubles every 8 codes
    for e in range(1, 15):
        seg = v[8 * e: 8 * e + 8]
        assert np.all(np.diff(seg) == seg[0] / 8)


def test_e4m3_encode_roundtrip_all_bytes():
    b = np.arange(0x7F)
    assert np.array_equal(F.e4m3_encode_nonneg(F.e4m3_decode(b)), b)


def test_e2m1_encode_roundtrip_all_codes():
    assert np.array_equal(F.e2m1_encode_magnitude(np.array(E2M1_SPEC)), np.arange(8))


@pytest.mark.parametrize("v,code", [
    (0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6),
    (0.2499, 0), (0.2501, 1), (4.99, 6), (5.01, 7), (6.0, 7), (0.0, 0),
])
def test_e2m1_ties_and_neighbours(v, code):
    assert int(F.e2m1_encode_magnitude(np.float32(v))) == code


@pytest.mark.parametrize("t,byte", [
    (1.0625, 0x38),             # tie 1.0 / 1.125 -> even 0x38
    (1.1875, 0x3A),             # tie 1.125 / 1.25 -> even 0x3A
    (1.5 * 2 ** -9, 0x02),      # tie between subnormals 1 and 2 -> even
    (0.5 * 2 ** -9, 0x00),      # tie 0 / 2^-9 -> 0
    (0.51 * 2 ** -9, 0x01),
    (432.0, 0x7E),              # tie 416 / 448 -> 0x7E (even)
    (440.0, 0x7E), (420.0, 0x7D), (448.0, 0x7E),
    (7.5 * 2 ** -9, 0x08),      # tie 7*2^-9 / 2^-6 -> even 0x08
])
def test_e4m3_ties(t, byte):
    assert int(F.e4m3_encode_nonneg(np.float64(t))) == byte


def _nearest_fraction(values, x):
    """Brute-force nearest (ties -> even index) with exact rationals."""
    fx = Fraction(x)
    best = None
    for i, v in enumerate(values):
        d = abs(Fraction(v) - fx)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def test_encoders_match_bruteforce_on_random_values():
    rng = np.random.default_rng(7)
    v = rng.uniform(0, 6, 400).astype(np.float32)
    got = F.e2m1_encode_magnitude(v)
    assert [_nearest_fraction(E2M1_SPEC, float(x)) for x in v] == list(got)
    e4 = [float(x) for x in F.e4m3_decode(np.arange(0x7F))]
    t = np.exp(rng.uniform(np.log(2.0 ** -11), np.log(448.0), 400)).astype(np.float32)
    got = F.e4m3_encode_nonneg(t)
    assert [_nearest_fraction(e4, float(x)) for x in t] == list(got)


def test_bf16_rounding():
    one = 1.0
    u = 2.0 ** -7                       # bf16 ulp at 1.0
    bits = F.round_to_bf16(np.array([one, one + u / 2, one + 3 * u / 2, one + u / 2 + 2.0 ** -30,
                                     -2.5, 3.0e38 / 2 ** 10, 0.0]))
    back = F.bf16_bits_to_f32(bits).astype(np.float64)
    assert back[0] == 1.0
    assert back[1] == 1.0               # tie -> even
    assert back[2] == 1.0 + 2 * u       # tie -> even (up)
    assert back[3] == 1.0 + u           # above the tie -> up
    assert back[4] == -2.5
    assert bits[6] == 0
    # direct rounding from float64 differs from float64 -> float32 -> bf16 here:
    x = 1.0 + u / 2 + 2.0 ** -40        # just above a bf16 tie, rounds to 1.0 in f32
    assert F.bf16_bits_to_f32(F.round_to_bf16(np.array([x])))[0] == 1.0 + u
