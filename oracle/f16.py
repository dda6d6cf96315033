"""IEEE binary16 (fp16) helpers for the oracle, from the format's definition.

Test infrastructure only (see the package docstring).

The FP16 activation variants ([TRT-17476] "Test Coverage": the fused
SwiGLU is exercised on BF16 and FP16 inputs) carry 16-bit IEEE halves:
1 sign, 5 exponent bits with bias 15, 10 mantissa bits. Normal values run
from 2**-14 to 65504 with 11 significant bits; below 2**-14 the spacing
stays at the subnormal quantum 2**-24. Exponent field 31 holds the
infinities (mantissa 0) and NaNs.
"""

import numpy as np

MAX_FINITE = 65504.0  # (2 - 2**-10) * 2**15
MIN_NORMAL = 2.0**-14
QUANTUM_MIN = 2.0**-24


def decode(bits):
    """uint16 binary16 bit patterns -> float64 values, from the field layout."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b & 0x8000, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    m = (b & 0x3FF).astype(np.float64)
    val = np.where(e == 0, m * QUANTUM_MIN, np.ldexp(1.0 + m / 1024.0, np.maximum(e, 1) - 15))
    val = np.where(e == 31, np.where(m == 0, np.inf, np.nan), val)
    return sign * val


def round_rne(v):
    """Round float64 values to the nearest binary16 value, ties to even.

    A finite nonzero v with 2**(e-1) <= |v| < 2**e has spacing 2**(e-11)
    (11 significant bits), floored at 2**-24 below the normal range. A
    magnitude that rounds above 65504 -- from 65520, the midpoint to the
    next power of two, upwards -- becomes an infinity of the same sign.
    Returns float64 holding binary16 values.
    """
    v = np.asarray(v, dtype=np.float64)
    finite = np.isfinite(v) & (v != 0)
    _, e = np.frexp(np.where(finite, v, 1.0))
    quantum = np.ldexp(1.0, np.maximum(e - 11, -24))
    r = np.round(np.where(finite, v, 0.0) / quantum) * quantum  # half-to-even
    r = np.where(np.abs(r) > MAX_FINITE, np.copysign(np.inf, v), r)
    return np.where(finite, r, v)


def ulp(v):
    """Spacing of binary16 values at |v| (float64)."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(v)
    e = np.where(v > 0, e, -1000)  # zero: the subnormal quantum
    return np.ldexp(1.0, np.maximum(e - 11, -24))
