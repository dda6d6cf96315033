"""Pins for the oracle's W8A8 / W8A16 GEMMs, shared-QKV and fused re-quantization.

Exact integer brute force (codes decoded by torch's independent float8 cast,
summed as Python integers), exact rational brute force, identity-weight
special cases and the invariants the pages state.
"""

from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3, linear
from workloads import config1, normal_bf16, random_e4m3_codes


def codes(shape, seed):
    return random_e4m3_codes(shape, seed).numpy()


def torch_values(c):
    return torch.from_numpy(np.asarray(c, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def test_w8a8_equals_integer_brute_force():
    m, n, k = 5, 7, 48  # distinct sizes: a transposed operand cannot pass
    q, qw = codes((m, k), 1), codes((n, k), 2)
    qi = (torch_values(q) * 512).astype(np.int64)  # every E4M3 value is a multiple of 2^-9
    wi = (torch_values(qw) * 512).astype(np.int64)
    y = linear.gemm_w8a8(q, qw, 1.0, 1.0)
    for i in range(m):
        for j in range(n):
            exact = sum(int(qi[i, t]) * int(wi[j, t]) for t in range(k))
            assert y[i, j] * 2**18 == exact


def test_w8a8_applies_both_scales():
    q, qw = codes((3, 32), 3), codes((4, 32), 4)
    s_in, s_w = np.float32(0.0012), np.float32(3.1e-5)
    base = linear.gemm_w8a8(q, qw, 1.0, 1.0)
    y = linear.gemm_w8a8(q, qw, s_in, s_w)
    assert np.allclose(y, base * float(s_in) * float(s_w), rtol=1e-15, atol=0)


def test_w8a8_identity_weight_returns_dequantized_activation():
    k = 64
    q = codes((9, k), 5)
    ident = np.where(np.eye(k, dtype=bool), 0x38, 0x00).astype(np.uint8)  # 0x38 = 1.0
    s_in = np.float32(0.01)
    y = linear.gemm_w8a8(q, ident, s_in, 1.0)
    assert np.array_equal(y, torch_values(q) * float(s_in))


def test_w8a8_zero_inputs():
    q = np.zeros((4, 32), np.uint8)
    qw = codes((6, 32), 6)
    assert np.all(linear.gemm_w8a8(q, qw, 1.0, 1.0) == 0)


def test_w8a8_exact_at_large_k():
    """All-448 operands at K = 16384: the float64 sum is exact (no rounding)."""
    k = 16384
    q = np.full((1, k), 0x7E, np.uint8)
    qw = np.full((2, k), 0x7E, np.uint8)
    qw[1, ::2] = 0xFE
    y = linear.gemm_w8a8(q, qw, 1.0, 1.0)
    assert y[0, 0] == 448.0 * 448.0 * k
    assert y[0, 1] == 0.0


def test_w8a16_equals_rational_brute_force():
    m, n, k = 3, 4, 40
    x = normal_bf16((m, k), 0.35, 8).float().numpy()
    qw = codes((n, k), 9)
    s_w = np.float32(0.02 / 448)
    y = linear.gemm_w8a16(x, qw, s_w)
    wv = torch_values(qw)
    for i in range(m):
        for j in range(n):
            exact = sum(Fraction(float(x[i, t])) * Fraction(float(wv[j, t])) for t in range(k)) * Fraction(float(s_w))
            assert abs(Fraction(y[i, j]) - exact) <= abs(exact) * Fraction(1, 2**50) + Fraction(1, 2**120)


def test_w8a16_identity_weight_returns_input_exactly():
    k = 128
    x = normal_bf16((6, k), 0.35, 10).float().numpy()
    ident = np.where(np.eye(k, dtype=bool), 0x38, 0x00).astype(np.uint8)
    y = linear.gemm_w8a16(x, ident, 1.0)
    assert np.array_equal(bf16.round_rne(y), x.astype(np.float64))


def test_w8a16_ignores_input_scale_and_differs_from_w8a8():
    case = config1()
    x = case.x.float().numpy()
    qw = linear.quantize_static(case.w.float().numpy(), case.weight_scale)
    y16 = linear.gemm_w8a16(x, qw, case.weight_scale)
    q = linear.quantize_static(x, case.input_scale)
    y8 = linear.gemm_w8a8(q, qw, case.input_scale, case.weight_scale)
    assert not np.allclose(y16, y8)
    # 16-bit activations land closer to the unquantized product than FP8 ones
    ref = x.astype(np.float64) @ case.w.double().numpy().T
    err16 = np.sqrt(np.mean((y16 - ref) ** 2))
    err8 = np.sqrt(np.mean((y8 - ref) ** 2))
    assert err16 < err8


def test_qkv_shared_quantizes_once_and_rejects_unequal_scales():
    x = normal_bf16((8, 64), 0.35, 11).float().numpy()
    qws = [codes((16, 64), 12 + i) for i in range(3)]
    sw = [1e-4, 7e-5, 4.5e-5]
    q, ys = linear.qkv_shared(x, qws, [0.002] * 3, sw, "W8A8")
    assert np.array_equal(q, linear.quantize_static(x, 0.002))
    for qw, s, y in zip(qws, sw, ys):
        assert np.array_equal(y, linear.gemm_w8a8(q, qw, 0.002, s))
    q16, ys16 = linear.qkv_shared(x, qws, [0.002] * 3, sw, "W8A16")
    assert q16 is None
    for qw, s, y in zip(qws, sw, ys16):
        assert np.array_equal(y, linear.gemm_w8a16(x, qw, s))
    with pytest.raises(ValueError):
        linear.qkv_shared(x, qws, [0.002, np.nextafter(np.float32(0.002), np.float32(1)), 0.002], sw, "W8A8")


def test_tolerance_rule():
    y_ref = np.array([100.0, -100.0, 0.0, 1.0])
    rms = np.sqrt(np.mean(y_ref**2))
    ok = linear.within_gemm_tolerance(y_ref + 2.0**-7 * np.abs(y_ref) + 0.999e-3 * rms, y_ref)
    assert ok.all()
    bad = linear.within_gemm_tolerance(y_ref + 2.0**-7 * np.abs(y_ref) + 1.01e-3 * rms, y_ref)
    assert not bad.any()
