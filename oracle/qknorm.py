"""Per-head QK RMSNorm followed by rotary position embedding (RoPE).

Test infrastructure only (see the package docstring).

[TRT-17476] "It is also faster": with separate projections, the per-head
RMSNorm of Q and K and the rotary embedding read contiguous Linear outputs
(the fused QKV hands them strided views), which is where the pages place
the end-to-end gain. [DF-15170] "Logs" shows the processor viewing a
projection as [tokens, heads, head_dim] and receiving a precomputed
rotary embedding.

The pages fix neither the RMSNorm epsilon nor the RoPE variant. Readings:
  * RMSNorm over each head's head_dim values x: y = x / sqrt(mean(x^2) + eps)
    * w, with a learned weight w of head_dim values and eps > 0 given by
    the caller (1e-6 in the workloads).
  * RoPE in the rotate-half form on the normalized values: for i < D/2,
    with the caller's per-token tables c = cos[t, i], s = sin[t, i],
      out[i]       = y[i] c - y[i + D/2] s
      out[i + D/2] = y[i + D/2] c + y[i] s
    i.e. the pair (y[i], y[i + D/2]) as a complex number times exp(i theta).
  * Norm first, then RoPE (the order in which the pages list them).
Everything is float64 here; the result is rounded to bf16 by the caller of
the GPU path only.
"""

import numpy as np


def rms_norm(x, weight, eps):
    """y = x / sqrt(mean(x^2, last axis) + eps) * weight, float64."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + float(eps)) * np.asarray(weight, dtype=np.float64)


def rope_rotate_half(y, cos, sin):
    """Rotate the pairs (y[..., i], y[..., i + D/2]) by the angles of cos/sin.

    y [..., T, H, D]; cos, sin [T, D/2] (broadcast over heads).
    """
    y = np.asarray(y, dtype=np.float64)
    half = y.shape[-1] // 2
    c = np.asarray(cos, dtype=np.float64)[:, None, :]
    s = np.asarray(sin, dtype=np.float64)[:, None, :]
    a, b = y[..., :half], y[..., half:]
    return np.concatenate([a * c - b * s, b * c + a * s], axis=-1)


def qk_norm_rope(x, heads, weight, cos, sin, eps):
    """x [T, heads * D] -> RoPE(RMSNorm(x per head)) as [T, heads * D], float64."""
    x = np.asarray(x, dtype=np.float64)
    t = x.shape[0]
    d = x.shape[1] // heads
    y = rms_norm(x.reshape(t, heads, d), weight, eps)
    return rope_rotate_half(y, cos, sin).reshape(t, heads * d)


def qk_norm_rope_bound(x, heads, weight, cos, sin, eps, out_ulp):
    """Largest |gpu - exact| for a float32 evaluation rounded once to the output.

    In float32 the sum of D squares has relative error at most D u, the
    reciprocal square root a few ulps, and the scaling by r and the weight
    and each RoPE product one rounding each, so every normalized value
    carries relative error below (D / 2 + 8) u and a RoPE output below
    (D / 2 + 10) u (|y_a c| + |y_b s|) <= (D / 2 + 10) u (|y_a| + |y_b|);
    one rounding to the output format adds at most one of its ulps.
    """
    x = np.asarray(x, dtype=np.float64)
    t = x.shape[0]
    d = x.shape[1] // heads
    u = 2.0**-24
    y = np.abs(rms_norm(x.reshape(t, heads, d), weight, eps))
    half = d // 2
    pair = y[..., :half] + y[..., half:]
    err = (d / 2 + 10) * u * np.concatenate([pair, pair], axis=-1).reshape(t, heads * d)
    ref = qk_norm_rope(x, heads, weight, cos, sin, eps)
    return err + out_ulp(np.abs(ref) + err)
