"""Pins for the oracle's binary16 helpers, FP16 SwiGLU and the W8A16 bound (CPU only)."""

import numpy as np

from oracle import bf16, e4m3, f16, linear, swiglu

ALL16 = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)


def test_decode_matches_numpy_half_on_every_pattern():
    ours = f16.decode(ALL16)
    lib = ALL16.view(np.float16).astype(np.float64)
    nan = np.isnan(lib)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], lib[~nan])
    assert np.array_equal(np.signbit(ours[~nan]), np.signbit(lib[~nan]))


def test_decode_field_examples():
    assert f16.decode([0x3C00, 0x7BFF, 0x0001, 0x0400, 0xC000, 0x7C00, 0xFC00]).tolist() == [
        1.0, 65504.0, 2.0**-24, 2.0**-14, -2.0, np.inf, -np.inf]


def test_round_trip_every_finite_pattern():
    vals = f16.decode(ALL16)
    fin = np.isfinite(vals)
    assert np.array_equal(f16.round_rne(vals[fin]), vals[fin])


def test_round_matches_numpy_cast_including_ties_and_overflow():
    rng = np.random.default_rng(7)
    v = np.concatenate([
        rng.normal(0, 1, 20000),
        rng.normal(0, 3e4, 20000),
        rng.normal(0, 1e-5, 20000),  # subnormal range
        np.ldexp(rng.uniform(-1, 1, 5000), rng.integers(-30, 18, 5000)),
    ])
    # exact midpoints between neighbouring finite halves: ties to even
    fin = f16.decode(ALL16[:0x7C00]).astype(np.float64)
    mids = (fin[:-1] + fin[1:]) / 2
    v = np.concatenate([v, mids, -mids, [65519.99, 65520.0, 7e4, -7e4, 2.0**-25, 3 * 2.0**-26]])
    with np.errstate(over="ignore"):
        lib = v.astype(np.float16).astype(np.float64)
    assert np.array_equal(f16.round_rne(v), lib)


def test_round_special_values():
    r = f16.round_rne([65520.0, -65520.0, 65519.0, 2.0**-25, -(2.0**-25), 3 * 2.0**-26, np.inf, 0.0])
    assert r.tolist() == [np.inf, -np.inf, 65504.0, 0.0, 0.0, 2.0**-24, np.inf, 0.0]
    assert np.signbit(r[4])  # a negative underflow keeps its sign
    assert np.isnan(f16.round_rne(np.nan))


def test_ulp_examples():
    assert f16.ulp([1.0, 1.5, 65504.0, 2.0**-14, 1e-7, 0.0]).tolist() == [2.0**-10, 2.0**-10, 32.0, 2.0**-24, 2.0**-24, 2.0**-24]


# ---------------------------------------------------------- FP16 SwiGLU


def test_swiglu_f16_special_cases():
    g = np.array([0.0, 2.0, 20.0, 300.0, -300.0])
    u = np.array([5.0, 0.0, 3.0, 300.0, 7.0])
    out = swiglu.swiglu_2in_f16(g, u)
    assert out[0] == 0 and out[1] == 0
    assert out[2] == f16.round_rne(20.0 * 3.0 / (1 + np.exp(-20.0)))  # ~ g * u
    assert out[3] == np.inf  # 90000 overflows binary16
    assert out[4] == 0.0


def test_swiglu_f16_is_rounded_product_and_differs_from_bf16():
    rng = np.random.default_rng(3)
    g = f16.round_rne(rng.normal(0, 2, 4000))
    u = f16.round_rne(rng.normal(0, 2, 4000))
    h = swiglu.swiglu_2in(g, u)
    out = swiglu.swiglu_2in_f16(g, u)
    assert np.array_equal(out, h.astype(np.float16).astype(np.float64))  # numpy's RNE cast
    assert np.all(np.abs(out - h) <= f16.ulp(h) / 2)
    assert np.mean(out != bf16.round_rne(h)) > 0.5  # 11 vs 8 significant bits


# ------------------------------------------- W8A16 float32-accumulation bound


def _sim_fp32_accumulate(terms):
    """Left-to-right float32 summation of float64-exact product rows."""
    acc = np.zeros(terms.shape[:-1], dtype=np.float32)
    for k in range(terms.shape[-1]):
        acc = (acc + terms[..., k].astype(np.float32)).astype(np.float32)
    return acc


def _split3(x):
    """x = hi + mid + lo, each a bf16 value (truncation of the remainder)."""
    x = np.asarray(x, dtype=np.float32)
    hi = (x.view(np.uint32) & 0xFFFF0000).view(np.float32)
    r = (x - hi).astype(np.float32)
    mid = (r.view(np.uint32) & 0xFFFF0000).view(np.float32)
    lo = (r - mid).astype(np.float32)
    return hi, mid, lo


def test_split3_is_exact_and_bf16():
    rng = np.random.default_rng(11)
    x = rng.normal(0, 0.35, 100000).astype(np.float32)
    parts = _split3(x)
    for p in parts:
        assert np.all((p.view(np.uint32) & 0xFFFF) == 0)
    assert np.array_equal(parts[0].astype(np.float64) + parts[1] + parts[2], x.astype(np.float64))


def test_bound_covers_simulated_fp32_accumulation():
    rng = np.random.default_rng(12)
    M, N, K = 6, 5, 384
    x = rng.normal(0, 0.35, (M, K)).astype(np.float32)
    qw = e4m3.encode(rng.normal(0, 60, (N, K)))
    s_w = np.float32(0.02 / 448 * 60)
    w = e4m3.decode(qw)
    hi, mid, lo = _split3(x)
    # per output: 3 K products, piece-major within each 64-element block
    terms = []
    for k0 in range(0, K, 64):
        for p in (hi, mid, lo):
            terms.append(p[:, None, k0:k0 + 64].astype(np.float64) * w[None, :, k0:k0 + 64])
    terms = np.concatenate(terms, axis=-1)
    y = (_sim_fp32_accumulate(terms) * s_w).astype(np.float32)
    y_ref = linear.gemm_w8a16(x, qw, s_w)
    bound = linear.gemm_w8a16_bound(x, qw, s_w, 3 * K, linear.f32_ulp)
    assert np.all(np.abs(y - y_ref) <= bound)
    # worst case far below that of a bf16-rounded activation (2**-9 of S)
    S = (np.abs(x).astype(np.float64) @ np.abs(w).T) * float(s_w)
    assert np.all(bound <= 2.0**-12 * S + 2 * linear.f32_ulp(y_ref))


def test_bound_of_one_term_is_an_ulp():
    x = np.array([[1.2345678, -3.25e-3, 7.5]], dtype=np.float32)
    qw = np.where(np.eye(3, dtype=bool), np.uint8(0x38), np.uint8(0))  # identity, 1.0
    b = linear.gemm_w8a16_bound(x, qw, 1.0, 1, linear.f32_ulp)
    assert np.all(b <= 3 * linear.f32_ulp(x))
    assert linear.f32_ulp(1.0) == 2.0**-23 and linear.f32_ulp(0.0) == 2.0**-149
