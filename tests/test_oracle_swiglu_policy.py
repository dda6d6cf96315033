"""Pins for the oracle's SwiGLU and step policy (CPU only)."""

import copy
import json
import os

import numpy as np
import pytest
import scipy.special

from oracle import bf16, e4m3, policy, swiglu


# ---------------------------------------------------------------- SwiGLU


def test_silu_matches_library_logistic():
    g = np.linspace(-30, 30, 2001)
    ref = g * scipy.special.expit(g)
    assert np.allclose(swiglu.silu(g), ref, rtol=1e-14, atol=1e-300)


def test_swiglu_special_cases():
    g = np.array([0.0, 2.0, -3.0, 50.0, -800.0, 800.0])
    u = np.array([5.0, 0.0, 0.0, 1.5, 2.0, 0.25])
    h = swiglu.swiglu_2in(g, u)
    assert h[0] == 0 and h[1] == 0 and h[2] == 0
    assert abs(h[3] - 75.0) < 1e-12  # large gate: silu(g) -> g
    assert h[4] == 0.0  # very negative gate underflows to zero without NaN
    assert h[5] == 200.0


def test_silu_reflection_identity():
    g = np.linspace(-10, 10, 101)
    assert np.allclose(swiglu.silu(-g), swiglu.silu(g) - g, rtol=0, atol=1e-14)


def test_swiglu_quant_is_encode_of_quotient():
    rng = np.random.default_rng(1)
    g, u = rng.normal(0, 0.45, 5000), rng.normal(0, 0.45, 5000)
    s_h = np.float32(1.7 / 448)
    codes, t = swiglu.swiglu_2in_quant(g, u, s_h)
    assert np.array_equal(codes, e4m3.encode(swiglu.swiglu_2in(g, u) / float(s_h)))
    assert np.allclose(t * float(s_h), swiglu.swiglu_2in(g, u), rtol=1e-15)


def test_near_midpoint_flags_only_the_band():
    mids = e4m3.midpoints()
    assert swiglu.near_midpoint(mids).all()
    assert swiglu.near_midpoint(-mids * (1 + 2.0**-22)).all()
    assert not swiglu.near_midpoint(mids * (1 + 2.0**-18)).any()
    vals = e4m3.decode(np.arange(1, 0x7F, dtype=np.uint8))  # representable values sit far from midpoints
    assert not swiglu.near_midpoint(vals).any()


def test_swiglu_bf16_output_is_rounded_product():
    g = np.array([0.5, -1.25, 3.0])
    u = np.array([1.0, 2.0, -0.75])
    out = swiglu.swiglu_2in_bf16(g, u)
    assert np.array_equal(out, bf16.round_rne(swiglu.swiglu_2in(g, u)))
    assert np.all(np.abs(out - swiglu.swiglu_2in(g, u)) <= bf16.ulp(out) / 2)


# ---------------------------------------------------------------- policy


@pytest.fixture(scope="module")
def golden(golden_dir):
    with open(os.path.join(golden_dir, "step_traces.json")) as f:
        return json.load(f)


def expand(runs):
    out = []
    for mode, n in runs:
        out += [mode] * n
    return out


def test_printed_traces(golden):
    pol = golden["policy"]
    for case in golden["traces"]:
        assert policy.trace(pol, case["num_steps"]) == expand(case["runs"]), case["source"]


def test_first_w8a8_step_is_step_three_of_eight(golden):
    t = policy.trace(golden["policy"], 8)
    assert t.index("W8A8") == golden["first_w8a8_step"]["step"]


def test_cfg_branches_agree_and_mode_depends_only_on_step(golden):
    pol = golden["policy"]
    for n in (2, 5, 8, 35):
        a = policy.trace(pol, n)
        b = [policy.step_mode(copy.deepcopy(pol), "generation", i, n) for i in range(n)]
        assert a == b


def test_reasoner_is_not_step_gated(golden):
    pol = dict(golden["policy"], first_steps=0)
    assert set(policy.trace(pol, 8, tower="reasoner")) == {golden["reasoner"]["mode"]}
    assert policy.trace(pol, 8)[0] == "W8A8"  # generation step 0 is outside a 0-step window
    pol8 = dict(pol, reasoner="a8")
    assert set(policy.trace(pol8, 8, tower="reasoner")) == {"W8A8"}


def test_no_policy_is_all_w8a8():
    assert policy.trace(None, 8) == ["W8A8"] * 8
    assert policy.trace(None, 3, tower="reasoner") == ["W8A8"] * 3


def test_overlapping_windows_run_16_bit(golden):
    pol = dict(golden["policy"], first_steps=4, last_steps=4)
    assert policy.trace(pol, 6) == ["W8A16"] * 6
    assert policy.trace(dict(golden["policy"], first_steps=0, last_steps=0), 5) == ["W8A8"] * 5


@pytest.mark.parametrize(
    "mutate",
    [
        lambda p: p.update(extra=1),
        lambda p: p.pop("overlap"),
        lambda p: p.pop("last_steps"),
        lambda p: p.update(schema_version=2),
        lambda p: p.update(schema_version=True),
        lambda p: p.update(type="sigma_range"),
        lambda p: p.update(index_space="timestep"),
        lambda p: p.update(default_mode="w8a16"),
        lambda p: p.update(overlap="a8"),
        lambda p: p.update(first_steps=-1),
        lambda p: p.update(last_steps=1.5),
        lambda p: p.update(first_steps=False),
        lambda p: p.update(reasoner="nvfp4"),
    ],
)
def test_policy_fails_closed(golden, mutate):
    pol = copy.deepcopy(golden["policy"])
    mutate(pol)
    with pytest.raises(policy.PolicyError):
        policy.validate(pol)
    with pytest.raises(policy.PolicyError):
        policy.step_mode(pol, "generation", 0, 8)
