"""Pins for the oracle's per-head QK RMSNorm + RoPE (CPU only)."""

import numpy as np

from oracle import bf16, qknorm


def tables(t, half, seed, base=10000.0):
    """Rotate-half RoPE tables for positions 0..t-1 (float32, as a caller passes them)."""
    pos = np.arange(t, dtype=np.float64)[:, None]
    inv = base ** (-np.arange(half, dtype=np.float64) / half)
    ang = pos * inv + np.random.default_rng(seed).uniform(0, 0.1)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def test_rms_norm_closed_forms():
    d = 128
    c = 0.37
    y = qknorm.rms_norm(np.full((1, d), c), np.ones(d), 1e-6)
    assert np.allclose(y, c / np.sqrt(c * c + 1e-6), rtol=1e-15)
    rng = np.random.default_rng(1)
    x = rng.normal(0, 2, (5, 3, d))
    w = rng.normal(1, 0.1, d)
    eps = 1e-6
    # textbook form through a library norm: x sqrt(D) / sqrt(||x||^2 + D eps)
    ref = x * np.sqrt(d) / np.sqrt(np.linalg.norm(x, axis=-1, keepdims=True) ** 2 + d * eps) * w
    assert np.allclose(qknorm.rms_norm(x, w, eps), ref, rtol=1e-13)
    # eps = 0: unit root-mean-square and scale invariance
    y0 = qknorm.rms_norm(x, np.ones(d), 0.0)
    assert np.allclose(np.sqrt(np.mean(y0 * y0, axis=-1)), 1.0, rtol=1e-14)
    assert np.allclose(qknorm.rms_norm(7.5 * x, w, 0.0), qknorm.rms_norm(x, w, 0.0), rtol=1e-14)
    # the epsilon matters for small inputs (a dropped eps fails this)
    small = np.full((1, d), 1e-4)
    assert abs(qknorm.rms_norm(small, np.ones(d), 1e-6)[0, 0] - 1.0) > 0.04


def test_rope_closed_forms():
    rng = np.random.default_rng(2)
    t, h, d = 6, 2, 64
    y = rng.normal(0, 1, (t, h, d))
    one = np.ones((t, d // 2))
    zero = np.zeros((t, d // 2))
    assert np.array_equal(qknorm.rope_rotate_half(y, one, zero), y)
    quarter = qknorm.rope_rotate_half(y, zero, one)  # 90 degrees: (a, b) -> (-b, a)
    assert np.array_equal(quarter[..., : d // 2], -y[..., d // 2:])
    assert np.array_equal(quarter[..., d // 2:], y[..., : d // 2])


def test_rope_is_complex_multiplication():
    rng = np.random.default_rng(3)
    t, h, d = 9, 3, 128
    y = rng.normal(0, 1, (t, h, d))
    c, s = tables(t, d // 2, 4)
    out = qknorm.rope_rotate_half(y, c, s)
    z = (y[..., : d // 2] + 1j * y[..., d // 2:]) * (c.astype(np.float64) + 1j * s.astype(np.float64))[:, None, :]
    assert np.allclose(out[..., : d // 2], z.real, rtol=0, atol=1e-14)
    assert np.allclose(out[..., d // 2:], z.imag, rtol=0, atol=1e-14)
    # the interleaved pairing (2i, 2i + 1) is a different map
    zi = (y[..., 0::2] + 1j * y[..., 1::2]) * (c.astype(np.float64) + 1j * s.astype(np.float64))[:, None, :]
    assert not np.allclose(out[..., : d // 2], zi.real)


def test_rope_composes_and_preserves_pair_norms():
    rng = np.random.default_rng(5)
    t, h, d = 4, 2, 64
    y = rng.normal(0, 1, (t, h, d))
    a1 = rng.uniform(-3, 3, (t, d // 2))
    a2 = rng.uniform(-3, 3, (t, d // 2))
    two = qknorm.rope_rotate_half(qknorm.rope_rotate_half(y, np.cos(a1), np.sin(a1)), np.cos(a2), np.sin(a2))
    one = qknorm.rope_rotate_half(y, np.cos(a1 + a2), np.sin(a1 + a2))
    assert np.allclose(two, one, atol=1e-13)
    r = qknorm.rope_rotate_half(y, np.cos(a1), np.sin(a1))
    assert np.allclose(r[..., :32] ** 2 + r[..., 32:] ** 2, y[..., :32] ** 2 + y[..., 32:] ** 2, rtol=1e-13)


def test_norm_then_rope_order():
    rng = np.random.default_rng(6)
    t, h, d = 5, 4, 128
    x = rng.normal(0, 0.35, (t, h * d))
    w = rng.normal(1, 0.2, d)
    c, s = tables(t, d // 2, 7)
    out = qknorm.qk_norm_rope(x, h, w, c, s, 1e-6)
    two_step = qknorm.rope_rotate_half(qknorm.rms_norm(x.reshape(t, h, d), w, 1e-6), c, s).reshape(t, h * d)
    assert np.array_equal(out, two_step)
    # RoPE first, then the norm, differs once the weight is not uniform
    rev = qknorm.rms_norm(qknorm.rope_rotate_half(x.reshape(t, h, d), c, s), w, 1e-6).reshape(t, h * d)
    assert not np.allclose(out, rev, rtol=1e-3)
    # heads are normalized separately: scaling one head leaves the others alone
    x2 = x.copy()
    x2[:, :d] *= 100.0
    out2 = qknorm.qk_norm_rope(x2, h, w, c, s, 1e-6)
    assert np.allclose(out2[:, d:], out[:, d:], rtol=1e-15)


def _sim_float32(x, heads, w, c, s, eps):
    """The kernel's arithmetic in float32: sum of squares, rsqrt, scale, RoPE."""
    x = np.asarray(x, dtype=np.float32)
    t = x.shape[0]
    d = x.shape[1] // heads
    xh = x.reshape(t, heads, d)
    ss = np.zeros((t, heads), dtype=np.float32)
    for i in range(d):
        ss = (ss + xh[..., i] * xh[..., i]).astype(np.float32)
    r = (np.float32(1) / np.sqrt((ss * np.float32(1.0 / d) + np.float32(eps)).astype(np.float32))).astype(np.float32)
    y = ((xh * r[..., None]).astype(np.float32) * w.astype(np.float32)).astype(np.float32)
    half = d // 2
    a, b = y[..., :half], y[..., half:]
    cc, sn = c[:, None, :], s[:, None, :]
    o = np.concatenate([(a * cc - b * sn).astype(np.float32), (b * cc + a * sn).astype(np.float32)], axis=-1)
    return o.reshape(t, heads * d)


def test_bound_covers_float32_evaluation():
    rng = np.random.default_rng(8)
    t, h, d = 64, 4, 128
    x = bf16.round_rne(rng.normal(0, 0.35, (t, h * d)))
    w = bf16.round_rne(rng.normal(1, 0.2, d))
    c, s = tables(t, d // 2, 9)
    got = bf16.round_rne(_sim_float32(x, h, w, c, s, 1e-6).astype(np.float64))
    ref = qknorm.qk_norm_rope(x, h, w, c, s, 1e-6)
    bound = qknorm.qk_norm_rope_bound(x, h, w, c, s, 1e-6, bf16.ulp)
    assert np.all(np.abs(got - ref) <= bound)
    # and it is tight: about one bf16 ulp, far below a plausible mistake
    assert np.all(bound <= 1.01 * bf16.ulp(np.abs(ref)) + 2.0**-16 * 8)
    wrong = bf16.round_rne(_sim_float32(x, h, w, s, c, 1e-6).astype(np.float64))  # cos and sin swapped
    assert np.mean(np.abs(wrong - ref) > bound) > 0.5
