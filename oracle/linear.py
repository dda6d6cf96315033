"""Static per-tensor FP8 linear layer: quantization and the two GEMM modes.

Test infrastructure only (see the package docstring).

Layouts follow nn.Linear with bias=False ([DF-15170] "Logs" prints the
4096 -> 4096 projection with bias=False): activation x is [M, K], weight W is
[N, K] (out_features x in_features, K contiguous), output y = x W^T is
[M, N].
"""

import numpy as np

from . import e4m3


def quantize_static(x, input_scale):
    """E4M3 codes of x / input_scale with a fixed, calibrated scale.

    [CF-157] "Verification": the activation quantizer divides by the exported
    input_scale, clamps, then rounds to float8. x holds bf16 values (as
    float32); the quotient is the IEEE correctly rounded float32 division of
    float32(x) by float32(input_scale) -- NumPy's float32 divide -- and the
    codes come from e4m3.encode (saturate to +-448, round to nearest even).
    """
    x32 = np.asarray(x, dtype=np.float32)
    s32 = np.float32(input_scale)
    with np.errstate(all="ignore"):
        quotient = x32 / s32
    return e4m3.encode(quotient.astype(np.float64))


def gemm_w8a8(q, qw, input_scale, weight_scale):
    """W8A8: y = (sum_k dec(q)[m,k] dec(qW)[n,k]) * s_in * s_w, float64.

    [CF-157] "Verification": a real FP8 x FP8 GEMM whose result is rescaled by
    the two per-tensor scales ([TRT-17476] "Description": one weight scale and
    one input scale per projection). Every E4M3 value is an integer multiple
    of 2**-9 and |value| <= 448, so each product is a multiple of 2**-18 below
    2**17.6 and, for K <= 2**16, every partial sum stays below 2**53 units of
    2**-18: the float64 dot product is exact in any summation order.
    Returns the exact (unrounded) float64 result y_ref of shape [M, N].
    """
    a = e4m3.decode(q)
    b = e4m3.decode(qw)
    acc = a @ b.T
    return acc * float(np.float32(input_scale)) * float(np.float32(weight_scale))


def gemm_w8a16(x, qw, weight_scale):
    """W8A16: y = s_w * sum_k x[m,k] dec(qW)[n,k] in float64; input_scale unused.

    [TRT-17476] "Denoising-step activation precision": on 16-bit steps the
    resident FP8 weight is dequantized with its own weight_scale and the
    activation stays in 16 bits; input_scale is not used. The pages round
    s_w * dec(qW) to the activation dtype before the GEMM ([DF-14664]
    "Behavior": dequant + F.linear); the exact product is used here, which
    that path approximates within the GEMM tolerance.

    The activation may be bf16, fp16 or float32 ([DF-14664] "Tests" lists an
    FP32 W8A16 case): the definition is the same, taken on the values.
    """
    xf = np.asarray(x, dtype=np.float64)
    b = e4m3.decode(qw)
    return (xf @ b.T) * float(np.float32(weight_scale))


def f32_ulp(v):
    """Spacing of float32 values at |v| (float64), floored at 2**-149."""
    v = np.abs(np.asarray(v, dtype=np.float64))
    _, e = np.frexp(v)
    e = np.where(v > 0, e, -1000)  # zero: the subnormal quantum
    return np.ldexp(1.0, np.maximum(e - 24, -149))


def gemm_w8a16_bound(x, qw, weight_scale, n_terms, out_ulp):
    """Largest |y - y_ref| of a W8A16 product accumulated in float32.

    The arithmetic bound for y = round_out(fl32(s_w * A)), where A is a
    float32 sum, in any order, of n_terms exact products whose true sum is
    sum_k x dec(qW): |A - sum| <= gamma * S with S = sum_k |x dec(qW)| and
    gamma = n u / (1 - n u), u = 2**-24 (the standard bound for recursive or
    blocked summation); the scale multiply adds a relative u, and rounding
    to the output format at most one ulp of the output (out_ulp) at the
    largest magnitude the value can take. For 16-bit activations each
    product is exact in float32 and n_terms = K; a float32 activation split
    into three bf16 pieces gives 3 K exact products.
    """
    u = 2.0**-24
    n = float(n_terms)
    gamma = n * u / (1.0 - n * u)
    s_w = float(np.float32(weight_scale))
    xa = np.abs(np.asarray(x, dtype=np.float64))
    S = (xa @ np.abs(e4m3.decode(qw)).T) * s_w
    y_ref = gemm_w8a16(x, qw, weight_scale)
    acc_err = gamma * (1.0 + u) * S + u * np.abs(y_ref)
    return acc_err + out_ulp(np.abs(y_ref) + acc_err)


def qkv_shared(x, qws, input_scales, weight_scales, mode):
    """Shared-input projections: quantize x once, then one GEMM per weight.

    [TRT-17476] "What changed": Q/K/V (or gate/up) quantize the shared
    activation once and hand the same FP8 tensor to every projection, each
    with its own weight_scale; the input scales of the group must be
    identical (checked bitwise here, as the library does at the boundary).
    On 16-bit steps ("Denoising-step activation precision") the sharing
    stands down: no quantization, each projection runs W8A16.
    Returns (codes or None, [y_i]).
    """
    s32 = [np.float32(s) for s in input_scales]
    if any(s.view(np.uint32) != s32[0].view(np.uint32) for s in s32):
        raise ValueError("input scales of a shared group must be bitwise equal")
    if mode == "W8A8":
        q = quantize_static(x, s32[0])
        return q, [gemm_w8a8(q, qw, s32[0], sw) for qw, sw in zip(qws, weight_scales)]
    if mode == "W8A16":
        return None, [gemm_w8a16(x, qw, sw) for qw, sw in zip(qws, weight_scales)]
    raise ValueError("mode must be 'W8A8' or 'W8A16'")


def fused_requant(qw, weight_scale, shared_scale):
    """Codes a fused loader stores when it keeps one scale for a group.

    [TRT-17476] "Description": a fused per-tensor FP8 linear holds a single
    weight scale, max(s), and re-quantizes each member onto it,
    qW' = FP8-round(s_i * qW_i / max(s)), a second rounding on top of the
    calibrated one. The arithmetic precision of that step is not stated;
    float32 is the reading adopted: fl32(fl32(s_i * dec(qW_i)) / max(s)),
    then e4m3.encode.
    """
    deq = (e4m3.decode(qw).astype(np.float32) * np.float32(weight_scale)).astype(np.float32)
    with np.errstate(all="ignore"):
        ratio = (deq / np.float32(shared_scale)).astype(np.float32)
    return e4m3.encode(ratio.astype(np.float64))


def within_gemm_tolerance(y, y_ref):
    """Elementwise GEMM acceptance: |y - y_ref| <= 2**-7 |y_ref| + 1e-3 rms(y_ref)."""
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    rms = float(np.sqrt(np.mean(y_ref * y_ref))) if y_ref.size else 0.0
    return np.abs(y - y_ref) <= 2.0**-7 * np.abs(y_ref) + 1e-3 * rms
