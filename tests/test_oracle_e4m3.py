"""Pins for the oracle's E4M3 codec and static quantizer (CPU only).

The codec is checked against the format's closed-form values, against an
independent library (torch's CPU float8_e4m3fn cast), and against a brute
force nearest-code search, so that a wrong bias, a wrong tie rule or a
missing saturation fails here.
"""

import json
import os

import numpy as np
import pytest
import torch

from oracle import bf16, e4m3, linear
from workloads import all_bf16_patterns, config1

ALL = np.arange(256, dtype=np.uint8)
FINITE = ALL[(ALL & 0x7F) != 0x7F]


def torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, dtype=np.uint8)).view(torch.float8_e4m3fn).double().numpy()


def torch_encode(values_f32):
    t = torch.from_numpy(np.asarray(values_f32, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_decode_closed_forms():
    d = e4m3.decode
    assert d(0x7E) == 448.0  # 1.75 * 2^8, largest finite
    assert d(0x77) == 240.0  # 1.875 * 2^7
    assert d(0x38) == 1.0  # exponent field 7 = bias
    assert d(0x08) == 2.0**-6  # smallest normal
    assert d(0x01) == 2.0**-9  # smallest subnormal
    assert d(0x07) == 7 * 2.0**-9  # largest subnormal
    assert d(0xB8) == -1.0
    assert d(0x00) == 0.0 and not np.signbit(d(0x00))
    assert d(0x80) == 0.0 and np.signbit(d(0x80))
    assert np.isnan(d(0x7F)) and np.isnan(d(0xFF))
    assert np.count_nonzero(np.isnan(d(ALL))) == 2


def test_decode_matches_torch_for_all_codes():
    ours = e4m3.decode(ALL)
    ref = torch_decode(ALL)
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(ours[ok], ref[ok])
    assert np.array_equal(np.signbit(ours[ok]), np.signbit(ref[ok]))


def test_values_increase_with_code():
    v = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(v) > 0)


def test_round_trip_every_finite_code():
    assert np.array_equal(e4m3.encode(e4m3.decode(FINITE)), FINITE)


def test_saturation():
    enc = e4m3.encode
    for v in (448.0, 448.5, 449.0, 464.0, 479.0, 1e6, np.inf):
        assert enc(v) == 0x7E, v
        assert enc(-v) == 0xFE, v
    assert enc(432.0) == 0x7E  # tie between 416 (odd code) and 448 (even code)
    assert enc(431.99) == 0x7D


def test_ties_go_to_even_code():
    vals = e4m3.decode(np.arange(0x7F, dtype=np.uint8))
    for c in range(0x7E):
        mid = (vals[c] + vals[c + 1]) / 2
        even = c if c % 2 == 0 else c + 1
        assert e4m3.encode(mid) == even
        assert e4m3.encode(np.nextafter(mid, -np.inf)) == c
        assert e4m3.encode(np.nextafter(mid, np.inf)) == c + 1
        assert e4m3.encode(-mid) == even | 0x80


def test_signed_zero_and_underflow():
    enc = e4m3.encode
    assert enc(0.0) == 0x00
    assert enc(-0.0) == 0x80
    assert enc(-(2.0**-11)) == 0x80
    assert enc(2.0**-10) == 0x00  # tie between 0 and 2^-9 -> even (0)
    assert enc(3 * 2.0**-10) == 0x02  # tie between 1 and 2 -> code 2
    assert enc(np.nextafter(2.0**-10, 1)) == 0x01


def test_nan_keeps_sign():
    assert e4m3.encode(np.nan) == 0x7F
    assert e4m3.encode(-np.nan) == 0xFF


def brute_force_encode(v):
    """Nearest finite code by exhaustive search, ties to the even code."""
    if np.isnan(v):
        return 0xFF if np.signbit(v) else 0x7F
    sign = 0x80 if np.signbit(v) else 0
    a = min(abs(v), 448.0)
    best, best_d = None, None
    for c in range(0x7F):
        d = abs(a - e4m3.decode(c))
        if best is None or d < best_d or (d == best_d and c % 2 == 0):
            best, best_d = c, d
    return best | sign


def test_encode_matches_brute_force():
    rng = np.random.default_rng(7)
    vals = np.concatenate(
        [
            rng.normal(0, 100, 300),
            rng.normal(0, 0.01, 300),
            rng.uniform(-500, 500, 100),
            e4m3.midpoints()[:40],
            [0.0, -0.0, np.inf, -np.inf, 2.0**-10, 3 * 2.0**-10],
        ]
    )
    ours = e4m3.encode(vals)
    for v, c in zip(vals, ours):
        assert c == brute_force_encode(v), v


def test_encode_matches_torch_cast_after_clamp():
    rng = np.random.default_rng(11)
    mids = e4m3.midpoints().astype(np.float32)
    vals = np.concatenate(
        [
            rng.normal(0, 50, 20000).astype(np.float32),
            rng.normal(0, 0.003, 20000).astype(np.float32),
            mids,
            np.nextafter(mids, np.float32(np.inf)),
            np.nextafter(mids, np.float32(-np.inf)),
            -mids,
        ]
    ).astype(np.float32)
    clamped = np.clip(vals, -448, 448)
    assert np.array_equal(e4m3.encode(vals.astype(np.float64)), torch_encode(clamped))


@pytest.mark.parametrize("scale", [1.0, 0.5430 / 448, 1e-3, 3.7, 2.0**-7, 1.0 + 2.0**-23, 0.02 / 448])
def test_quantize_every_bf16_pattern_matches_reference_op_sequence(scale):
    """x / s -> clamp(+-448) -> cast, as torch's own CPU ops, on all 65,536 inputs."""
    x = all_bf16_patterns()
    s = np.float32(scale)
    ref = (x.float() / torch.tensor(s)).clamp(-448, 448).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    ours = linear.quantize_static(bf16.bits_to_f32(x.view(torch.int16).numpy().view(np.uint16)), s)
    assert np.array_equal(ours, ref)


def test_calibrated_amax_from_log_maps_to_full_scale(golden_dir):
    with open(os.path.join(golden_dir, "calibration_log.json")) as f:
        log = json.load(f)
    s_in = np.float32(log["input_amax"]) / np.float32(448)
    amax_bf16 = float(torch.tensor(log["input_amax"]).to(torch.bfloat16).float())
    assert linear.quantize_static(np.float32(amax_bf16), s_in) == 0x7E
    assert linear.quantize_static(np.float32(-amax_bf16), s_in) == 0xFE
    # the weight amax, with its own scale, is the largest weight code too
    s_w = np.float32(log["weight_amax"]) / np.float32(448)
    w_bf16 = float(torch.tensor(log["weight_amax"]).to(torch.bfloat16).float())
    assert linear.quantize_static(np.float32(w_bf16), s_w) in (0x7D, 0x7E)


def test_config1_saturates_about_one_percent():
    case = config1()
    q = linear.quantize_static(case.x.float().numpy(), case.input_scale)
    frac = np.mean((q & 0x7F) == 0x7E)
    assert 0.001 < frac < 0.05, frac


def test_bf16_rounding_matches_torch_cast_from_float32():
    rng = np.random.default_rng(3)
    v = np.concatenate([rng.normal(0, 1, 10000), rng.normal(0, 1e-38, 100), rng.normal(0, 1e38, 100)])
    v32 = v.astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).double().numpy()
    assert np.array_equal(bf16.round_rne(v32.astype(np.float64)), ref)
