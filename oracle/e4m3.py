"""OCP FP8 E4M3 ("FN" variant) codec, written from the format's definition.

Test infrastructure only (see the package docstring).

Format: sign bit, 4 exponent bits with bias 7, 3 mantissa bits -- the "(4, 3)
bit" quantizer printed in the ModelOpt log of [DF-15170] "Logs". The FN
variant has no infinities; exponent 15 with mantissa 7 is NaN, so the largest
finite magnitude is 1.75 * 2**8 = 448. Exponent 0 encodes subnormals
m * 2**-9.

Encoding follows the reference quantizer's op order ([CF-157] "Verification":
divide, then clamp to the finite range, then round to float8): values are
first saturated to [-448, 448] (so +-Inf map to +-448), then rounded to the
nearest representable value with ties to the even code. The sign is kept,
so a negative value that rounds to zero gives the code 0x80 (-0). NaN maps to
0x7F with its sign bit (0xFF for a negative NaN); the pages do not say, this
is the reading adopted (and what torch's own cast does).
"""

import numpy as np

EXP_BIAS = 7
MAX_FINITE = 448.0
NAN_CODE = 0x7F


def decode(codes):
    """E4M3 codes (uint8 array) -> float64 values, from the bit fields."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c & 0x80) != 0, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    normal = np.ldexp(1.0 + m / 8.0, (e - EXP_BIAS).astype(np.int32))
    subnormal = np.ldexp(m.astype(np.float64), -9)
    mag = np.where(e == 0, subnormal, normal)
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# Non-negative finite codes 0x00..0x7E in code order; their values increase
# strictly with the code (checked by the tests), so the table is sorted.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = decode(_POS_CODES.astype(np.uint8))


def encode(values):
    """float64 values -> E4M3 codes: saturate, then round to nearest even.

    For a magnitude a (after saturation) the two neighbouring representable
    magnitudes lo <= a <= hi are found in the sorted table of the 127
    non-negative finite values; a goes to the nearer one, and a tie (a equal
    to their midpoint, which is exact in float64) goes to the code whose
    lowest bit -- the mantissa's lowest bit -- is 0.
    """
    v = np.asarray(values, dtype=np.float64)
    neg = np.signbit(v)
    isnan = np.isnan(v)
    a = np.minimum(np.where(isnan, 0.0, np.abs(v)), MAX_FINITE)
    hi = np.searchsorted(_POS_VALUES, a, side="left")  # first value >= a
    lo = np.maximum(hi - 1, 0)
    vlo = _POS_VALUES[lo]
    vhi = _POS_VALUES[hi]
    mid = (vlo + vhi) / 2.0
    even = np.where(lo % 2 == 0, lo, hi)
    code = np.where(a < mid, lo, np.where(a > mid, hi, even))
    code = np.where(vhi == a, hi, code)
    code = np.where(isnan, NAN_CODE, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


def midpoints():
    """The 126 rounding midpoints between consecutive non-negative codes."""
    return (_POS_VALUES[:-1] + _POS_VALUES[1:]) / 2.0
