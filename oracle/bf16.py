"""bfloat16 helpers for the oracle, from the format's definition.

Test infrastructure only (see the package docstring).

bfloat16 is the upper half of an IEEE binary32: 1 sign, 8 exponent, 7
mantissa bits. The activations and outputs of the layer are bf16
([DF-15170] "Reproduction" loads the pipeline in torch.bfloat16).
"""

import numpy as np


def bits_to_f32(bits):
    """uint16 bf16 bit patterns -> float32 values (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def round_rne(v):
    """Round float64 values to the nearest bfloat16 value, ties to even.

    A finite nonzero v with 2**(e-1) <= |v| < 2**e has bf16 spacing
    2**(e-8) (8 significant bits); below the normal range the spacing stays
    at the subnormal quantum 2**-133. Magnitudes that round above the largest
    finite bf16 become infinities. Returns float64 holding bf16 values.
    """
    v = np.asarray(v, dtype=np.float64)
    out = np.array(v, copy=True)
    finite = np.isfinite(v) & (v != 0)
    _, e = np.frexp(np.where(finite, v, 1.0))
    quantum = np.ldexp(1.0, np.maximum(e - 8, -133))
    r = np.round(np.where(finite, v, 0.0) / quantum) * quantum  # half-to-even
    max_bf16 = np.ldexp(255.0 / 128.0, 127)  # 0x7F7F
    r = np.where(np.abs(r) > max_bf16, np.copysign(np.inf, v), r)
    out = np.where(finite, r, out)
    return out


def ulp(v):
    """Spacing of bf16 values at |v| (float64): the gap from |v| to the next
    larger bf16 value, 2**(e-8) for 2**(e-1) <= |v| < 2**e, and the subnormal
    quantum 2**-133 below the normal range and at zero."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(v)
    e = np.where(v > 0, e, -1000)  # zero: the subnormal quantum
    return np.ldexp(1.0, np.maximum(e - 8, -133))
