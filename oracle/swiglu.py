"""Two-input SwiGLU, h = silu(g) * u, emitted as E4M3 or bf16.

Test infrastructure only (see the package docstring).

[TRT-17476] "What changed": the split gated MLP computes SiLU(G) * U from
two separate tensors and quantizes the result straight to FP8 with the
down projection's static input scale; on 16-bit steps ("Denoising-step
activation precision") it emits 16-bit output instead.

Readings (the pages are silent):
  * silu(g) = g / (1 + exp(-g)), evaluated in float64; h is not rounded to
    bf16 before quantization ("quantizing the result directly").
  * FP8 output: code = e4m3.encode(h / s_h) with the same saturating
    round-to-nearest-even rule as the activation quantizer.
  * A GPU evaluates exp in float32, so its h differs from this float64 h by
    a few float32 ulps. Where h / s_h lies within relative 2**-20 of an E4M3
    rounding midpoint, both neighbouring codes are accepted
    (``near_midpoint``). Outside that band the codes must be identical.
  * bf16 output: within one bf16 ulp of bf16_rne(h).
  * FP16 inputs ([TRT-17476] "Test Coverage" runs the fused SwiGLU on BF16
    and FP16 shapes): the same float64 h from the half-precision values;
    FP8 output as above, FP16 output within one binary16 ulp of
    f16_rne(h), which overflows to an infinity from 65520 up.
The pages print no worked SwiGLU values; the pins are scipy's logistic
function, the reflection identity silu(-g) = silu(g) - g, special values
and torch's bf16 cast (tests/test_oracle_swiglu_policy.py).
"""

import numpy as np

from . import bf16, e4m3, f16

NEAR_TIE_REL = 2.0**-20


def silu(g):
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_2in(g, u):
    """h = silu(g) * u in float64."""
    return silu(g) * np.asarray(u, dtype=np.float64)


def swiglu_2in_quant(g, u, out_scale):
    """E4M3 codes of silu(g) * u / s_h, and the float64 quotient itself."""
    with np.errstate(all="ignore"):
        t = swiglu_2in(g, u) / float(np.float32(out_scale))
    return e4m3.encode(t), t


def swiglu_2in_bf16(g, u):
    """bf16_rne(silu(g) * u) as float64 values."""
    return bf16.round_rne(swiglu_2in(g, u))


def swiglu_2in_f16(g, u):
    """f16_rne(silu(g) * u) as float64 values (FP16 in, FP16 out)."""
    return f16.round_rne(swiglu_2in(g, u))


def near_midpoint(t, rel=NEAR_TIE_REL):
    """True where |t| lies within relative `rel` of an E4M3 rounding midpoint."""
    a = np.abs(np.asarray(t, dtype=np.float64))
    mids = e4m3.midpoints()
    idx = np.clip(np.searchsorted(mids, a), 1, len(mids) - 1)
    near = np.minimum(np.abs(a - mids[idx - 1]), np.abs(a - mids[idx]))
    near = np.minimum(near, np.abs(a - mids[0]))
    return near <= rel * np.maximum(a, mids[0])
