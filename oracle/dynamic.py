"""Dynamic per-tensor FP8 activation quantization: the scale from a runtime amax.

Test infrastructure only (see the package docstring).

The pages keep a dynamically quantized FP8 path beside the static one
([TRT-17476] "What changed": BF16, dynamic FP8 and other models keep the
fused topology; "Test Coverage": static and dynamic FP8 resolution are both
tested), but do not spell out its scale. The plainest reading consistent with
the static path: the scale is the max calibrator's rule -- the one behind the
amax values the pages print for the static checkpoint ([DF-15170] "Logs":
a per-tensor MaxCalibrator amax, and input_scale = amax / 448 maps it to the
largest E4M3 value) -- applied at run time to the tensor being quantized;
the codes then follow the static rule with that scale.

Readings where the pages are silent (each pinned in tests/test_oracle_dynamic.py):
  * amax is max |x| over the finite elements; NaN and +-Inf do not enter it
    (they then quantize like any other element: NaN -> NaN code, +-Inf ->
    +-448), so one stray non-finite value does not wipe out the scale.
  * s = fl32(amax) / fl32(448) in float32 (IEEE division), raised to 2^-126
    when smaller (all-zero or tiny tensors), so 1 / s stays a normal float;
    with amax = 0 every code is a signed zero whatever the scale.
"""

import numpy as np

from . import linear

E4M3_MAX = 448.0
MIN_SCALE = 2.0**-126


def amax_finite(x):
    """max |x| over the finite elements of x (0.0 if there are none)."""
    v = np.abs(np.asarray(x, dtype=np.float64)).ravel()
    v = v[np.isfinite(v)]
    return float(v.max()) if v.size else 0.0


def dynamic_scale(x):
    """float32 scale fl32(amax) / fl32(448), at least 2^-126."""
    with np.errstate(all="ignore"):
        s = np.float32(amax_finite(x)) / np.float32(E4M3_MAX)
    return float(max(s, np.float32(MIN_SCALE)))


def quantize_dynamic(x):
    """(codes, scale): the static quantization of x with its own dynamic scale."""
    s = dynamic_scale(x)
    return linear.quantize_static(x, s), s
