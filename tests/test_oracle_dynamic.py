"""Pins of the dynamic per-tensor FP8 oracle (oracle/dynamic.py).

The scale is the max-calibration rule applied at run time; these checks tie
it to what that rule must do: the amax element lands on the largest E4M3
code (as the printed calibration amax does for the static scale), the codes
are invariant under power-of-two rescaling of the tensor, non-finite
elements do not move the scale, and the degenerate tensors (all zero, tiny)
take the documented floor.
"""

import json
import os

import numpy as np
import torch

from oracle import dynamic, e4m3, linear
from workloads import normal_bf16


def bf16_values(t):
    return t.float().numpy().astype(np.float64)


def test_amax_element_is_full_scale():
    x = bf16_values(normal_bf16((64, 96), 0.35, 31))
    q, s = dynamic.quantize_dynamic(x)
    i = np.unravel_index(np.argmax(np.abs(x)), x.shape)
    assert q[i] & 0x7F == 0x7E  # 448
    assert s == float(np.float32(np.abs(x).max()) / np.float32(448))
    # every code stays inside the finite range and some other code is below full scale
    assert np.all((q & 0x7F) <= 0x7E) and np.any((q & 0x7F) < 0x7E)


def test_printed_calibration_amax_as_a_tensor(golden_dir):
    # a tensor whose largest magnitude is the printed input amax behaves like the static checkpoint
    with open(os.path.join(golden_dir, "calibration_log.json")) as f:
        log = json.load(f)
    a = float(torch.tensor(log["input_amax"]).to(torch.bfloat16).float())
    x = np.array([0.0, 0.1, -a, 0.25], dtype=np.float64)
    q, s = dynamic.quantize_dynamic(x)
    assert s == float(np.float32(a) / np.float32(448))
    assert q[2] == 0xFE and q[0] == 0x00


def test_power_of_two_rescaling_leaves_codes_unchanged():
    x = bf16_values(normal_bf16((40, 64), 1.0, 32))
    q0, s0 = dynamic.quantize_dynamic(x)
    for k in (-20, -3, 5, 30):
        qk, sk = dynamic.quantize_dynamic(x * 2.0**k)
        assert np.array_equal(qk, q0)
        assert sk == s0 * 2.0**k


def test_non_finite_elements_do_not_move_the_scale():
    x = bf16_values(normal_bf16((8, 32), 0.5, 33))
    s = dynamic.dynamic_scale(x)
    y = x.copy()
    y[0, 0], y[1, 1], y[2, 2] = np.inf, -np.inf, np.nan
    qy, sy = dynamic.quantize_dynamic(y)
    assert sy == s
    assert qy[0, 0] == 0x7E and qy[1, 1] == 0xFE and (qy[2, 2] & 0x7F) == 0x7F
    mask = np.ones_like(x, dtype=bool)
    mask[0, 0] = mask[1, 1] = mask[2, 2] = False
    assert np.array_equal(qy[mask], linear.quantize_static(x, s)[mask])


def test_all_zero_and_tiny_tensors_take_the_floor():
    z = np.zeros((4, 16))
    q, s = dynamic.quantize_dynamic(z)
    assert s == 2.0**-126 and np.all(q == 0)
    zn = -z
    assert np.all(dynamic.quantize_dynamic(zn)[0] == 0x80)  # negative zeros keep their sign
    t = np.zeros((2, 16))
    t[0, 3] = 2.0**-133  # the smallest bf16 subnormal
    q, s = dynamic.quantize_dynamic(t)
    assert s == 2.0**-126
    assert q[0, 3] == e4m3.encode(np.array([2.0**-7]))[0]  # 2^-133 / 2^-126
    only_nan = np.full((1, 16), np.nan)
    assert dynamic.dynamic_scale(only_nan) == 2.0**-126


def test_scale_is_the_float32_quotient():
    # amax values whose quotient by 448 is not representable: the scale is the float32 division
    for a in (1.0, 3.0, 0.5430, 1e-30, 3.0e38):
        ab = float(torch.tensor(a).to(torch.bfloat16).float())
        s = dynamic.dynamic_scale(np.array([ab, -ab / 2]))
        assert np.float32(s) == np.float32(ab) / np.float32(448)
        assert abs(s - ab / 448.0) <= np.spacing(np.float32(s))
