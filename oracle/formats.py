"""Element and scale codecs of NVFP4: E2M1 values and E4M3 block scales.

The README ("NVFP4 MegaMoE Kernel", section "What We Have", grouped GEMM) says
NVFP4 carries 4-bit values with one FP8 scale per 16 elements; the value set
{0, +-0.5, +-1, +-1.5, +-2, +-3, +-4, +-6} is E2M1 and the scale is OCP E4M3
("fn": bias 7, max 448, no infinities).  The underflow threshold 6 * 2**-9 of
the README's "Correctness Bugs Fixed" table (bug 4) is E2M1's largest value
times E4M3's smallest subnormal, which pins the scale format to OCP E4M3.

Decoders are the format definitions written out.  Encoders are "nearest
representable value, ties to the even code": candidates are taken from the
decoded table and compared in float64, where every candidate and every fp32
input is exact, so the comparison itself cannot round.
"""

import numpy as np

# ---------------------------------------------------------------- E2M1 (FP4)


def e2m1_magnitude(code3):
    """|value| of a 3-bit E2M1 magnitude code (exponent 2 bits, bias 1,
    mantissa 1 bit; exponent field 0 is subnormal with step 0.5)."""
    code3 = np.asarray(code3, dtype=np.int64)
    e = code3 >> 1
    m = code3 & 1
    normal = np.ldexp(1.0 + m / 2.0, (e - 1).astype(np.int32))
    sub = m * 0.5
    return np.where(e == 0, sub, normal)


def e2m1_decode(code4):
    """Signed value (float64) of a 4-bit E2M1 code; bit 3 is the sign."""
    code4 = np.asarray(code4, dtype=np.int64)
    mag = e2m1_magnitude(code4 & 7)
    return np.where(code4 & 8, -mag, mag)


_E2M1_TABLE = e2m1_magnitude(np.arange(8))  # ascending: 0 .5 1 1.5 2 3 4 6


def _nearest_ties_even(table, v):
    """Index of the nearest entry of the ascending ``table`` to each v >= 0,
    ties going to the even index.  ``v`` must lie within [table[0], table[-1]]."""
    v = np.asarray(v, dtype=np.float64)
    j = np.searchsorted(table, v, side="left")
    j = np.clip(j, 1, len(table) - 1)
    lo, hi = j - 1, j
    dlo = v - table[lo]
    dhi = table[hi] - v
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    return np.where(pick_hi, hi, lo)


def e2m1_encode_magnitude(v):
    """3-bit code of the E2M1 magnitude nearest to v (0 <= v <= 6), ties to
    the even code (round-to-nearest-even on the E2M1 grid)."""
    v = np.asarray(v, dtype=np.float64)
    if np.any(v < 0) or np.any(v > 6) or np.any(np.isnan(v)):
        raise ValueError("e2m1_encode_magnitude expects 0 <= v <= 6")
    return _nearest_ties_even(_E2M1_TABLE, v).astype(np.uint8)


# ---------------------------------------------------------------- E4M3 (FP8)


def e4m3_decode(byte):
    """Value (float64) of an OCP E4M3 byte: sign, 4-bit exponent (bias 7),
    3-bit mantissa; exponent 0 is subnormal (step 2**-9); S.1111.111 is NaN;
    there is no infinity."""
    b = np.asarray(byte, dtype=np.int64)
    s = (b >> 7) & 1
    e = (b >> 3) & 15
    m = b & 7
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int32))
    sub = np.ldexp(m / 8.0, -6)
    mag = np.where(e == 0, sub, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return np.where(s == 1, -mag, mag)


E4M3_MAX = 448.0
# non-negative finite E4M3 values, ascending with the byte code 0x00..0x7E
_E4M3_TABLE = e4m3_decode(np.arange(0x7F))


def e4m3_encode_nonneg(t):
    """E4M3 byte of the value nearest to t (0 <= t <= 448), ties to the even
    byte.  Callers saturate first (min(t, 448))."""
    t = np.asarray(t, dtype=np.float64)
    if np.any(t < 0) or np.any(t > E4M3_MAX) or np.any(np.isnan(t)):
        raise ValueError("e4m3_encode_nonneg expects 0 <= t <= 448")
    return _nearest_ties_even(_E4M3_TABLE, t).astype(np.uint8)


# ---------------------------------------------------------------- BF16


def bf16_bits_to_f32(bits):
    """float32 array holding the values of raw bfloat16 bit patterns."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def round_to_bf16(x):
    """bfloat16 bit patterns of float64 values, rounded to nearest with ties to
    even directly from float64 (no double rounding through float32).  Finite
    inputs in bfloat16's normal range, or zero."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                     # x = m * 2**e, 0.5 <= |m| < 1
    r = np.rint(np.ldexp(m, 8))            # 8 significant bits, ties to even
    val = np.ldexp(r, e - 8)               # exact
    f32 = val.astype(np.float32)           # exact: val is bf16-representable
    return (f32.view(np.uint32) >> 16).astype(np.uint16)
