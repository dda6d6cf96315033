"""Pins of the oracle's ulp helpers, which set the width of several GPU acceptance checks.

Each helper must equal the gap between a value and the next representable value of its format, taken
from an independent source: torch's bf16 bit patterns (the activation and output format of the layer,
[DF-15170] "Reproduction" runs the pipeline in torch.bfloat16), numpy's binary16 and float32 spacing.
An ulp that is too wide (an exponent off by one) loosens every check built on it, one that is too
narrow fails them; both are caught here, over every finite bf16 and binary16 value.
"""

import numpy as np
import torch

from oracle import bf16, f16, linear


def _bf16_values(lo, hi):
    """float64 values of the bf16 bit patterns [lo, hi), from torch's own reinterpretation."""
    bits = torch.arange(lo, hi, dtype=torch.int32).to(torch.int16)
    return bits.view(torch.bfloat16).to(torch.float64).numpy()


def test_bf16_ulp_is_the_gap_to_the_next_value_for_every_finite_pattern():
    # non-negative finite patterns 0x0000..0x7F7F; the gap of pattern b is value(b + 1) - value(b)
    v = _bf16_values(0, 0x7F80)  # 0x7F80 is +inf: v[-1] is the largest finite value
    gap = np.diff(v)
    assert np.all(gap > 0)
    assert np.array_equal(bf16.ulp(v[:-1]), gap)
    # the sign does not matter
    neg = _bf16_values(0x8000, 0xFF80)
    assert np.array_equal(bf16.ulp(neg[:-1]), gap)
    # the largest finite value has the spacing of its binade (2^127 .. 2^128: 2^120)
    assert bf16.ulp(v[-1]) == 2.0**120 == v[-1] - v[-2]


def test_bf16_ulp_subnormal_floor_and_zero():
    assert bf16.ulp(0.0) == 2.0**-133
    assert bf16.ulp(2.0**-133) == 2.0**-133
    assert bf16.ulp(2.0**-126) == 2.0**-133  # the smallest normal: the same quantum as the subnormals
    assert bf16.ulp(1.0) == 2.0**-7 and bf16.ulp(1.9921875) == 2.0**-7 and bf16.ulp(2.0) == 2.0**-6


def test_bf16_ulp_between_representable_values():
    # a value strictly inside (b, b + 1) has the gap of that interval: the bf16 value at or below a
    # float32 is its bit pattern with the low 16 bits cleared
    rng = np.random.default_rng(5)
    v32 = (rng.standard_normal(200000) * np.exp2(rng.integers(-120, 120, 200000))).astype(np.float32)
    v32 = v32[np.isfinite(v32) & (v32 != 0)]
    below = (np.abs(v32).view(np.uint32) & np.uint32(0xFFFF0000)).view(np.float32).astype(np.float64)
    nxt = ((np.abs(v32).view(np.uint32) & np.uint32(0xFFFF0000)) + np.uint32(0x10000)).view(np.float32)
    ok = np.isfinite(nxt)
    assert np.array_equal(bf16.ulp(v32.astype(np.float64))[ok], nxt[ok].astype(np.float64) - below[ok])


def test_f16_ulp_is_numpy_spacing_for_every_finite_pattern():
    h = np.arange(0, 0x7C00, dtype=np.uint16).view(np.float16)  # non-negative finite binary16
    sp = np.spacing(h[:-1]).astype(np.float64)
    assert np.array_equal(f16.ulp(h[:-1].astype(np.float64)), sp)
    assert f16.ulp(65504.0) == 32.0


def test_f32_ulp_is_numpy_spacing():
    rng = np.random.default_rng(6)
    v = (rng.standard_normal(200000) * np.exp2(rng.integers(-149, 127, 200000))).astype(np.float32)
    v = np.concatenate([v, np.float32([2.0**-149, 2.0**-126, 1.0, np.nextafter(np.float32(2), np.float32(0))])])
    v = np.abs(v[np.isfinite(v) & (v != 0)])
    v = v[v < np.float32(3.0e38)]
    assert np.array_equal(linear.f32_ulp(v.astype(np.float64)), np.spacing(v).astype(np.float64))
    assert linear.f32_ulp(0.0) == 2.0**-149
