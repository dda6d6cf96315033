"""Host-side checks of the C ABI (no GPU needed).

The library must load and export every entry point include/fp8lin.h
declares. The pure host calls (policy, strerror, counters) run for real; the
GPU entry points are called only with arguments the validation refuses, or
with zero rows (a no-op), so nothing touches a device.
"""

import copy
import ctypes
import json
import os
import re

import pytest

import w8a16_linear_layers_amd as fp8lin
from oracle import policy as opolicy

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000  # a 16-byte aligned stand-in for a device pointer; never dereferenced


def declared_functions():
    with open(os.path.join(ROOT, "include", "fp8lin.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^(?:int32_t|int64_t|const char\*)\s+(fp8lin_\w+)\(", text, re.M)))


def test_library_exports_every_declared_entry_point(lib):
    names = declared_functions()
    assert len(names) == 24, names
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(fp8lin.EXPORTS)


def test_strerror_covers_every_status():
    for st in range(0, -8, -1):
        msg = fp8lin.fp8lin_strerror(st)
        assert msg and msg != "unknown status"
    assert fp8lin.fp8lin_strerror(-99) == "unknown status"


def test_launch_count_rejects_unknown_kind():
    assert fp8lin.fp8lin_launch_count(-1) == -1
    assert fp8lin.fp8lin_launch_count(9) == -1
    assert fp8lin.fp8lin_launch_count(0) >= 0


# ---------------------------------------------------------------- policy


@pytest.fixture(scope="module")
def golden(golden_dir):
    with open(os.path.join(golden_dir, "step_traces.json")) as f:
        return json.load(f)


def c_trace(pol, n, tower=fp8lin.TOWER_GENERATION):
    names = {fp8lin.MODE_W8A8: "W8A8", fp8lin.MODE_W8A16: "W8A16"}
    return [names[fp8lin.fp8lin_step_policy(pol, tower, i, n)] for i in range(n)]


def test_c_policy_reproduces_printed_traces(golden):
    pol = fp8lin.policy_from_json(golden["policy"])
    assert fp8lin.fp8lin_policy_validate(pol) == 0
    for case in golden["traces"]:
        expected = []
        for mode, n in case["runs"]:
            expected += [mode] * n
        assert c_trace(pol, case["num_steps"]) == expected, case["source"]


def test_c_policy_matches_oracle_on_a_grid(golden):
    for first in range(0, 5):
        for last in range(0, 5):
            for reasoner in ("a16", "a8"):
                doc = dict(golden["policy"], first_steps=first, last_steps=last, reasoner=reasoner)
                pol = fp8lin.policy_from_json(doc)
                for n in range(1, 12):
                    assert c_trace(pol, n) == opolicy.trace(doc, n)
                    assert c_trace(pol, n, fp8lin.TOWER_REASONER) == opolicy.trace(doc, n, "reasoner")


def test_null_policy_runs_w8a8():
    assert fp8lin.policy_from_json("null") is None
    assert c_trace(None, 8) == ["W8A8"] * 8


def test_policy_step_bounds():
    for step, n in ((-1, 8), (8, 8), (0, 0)):
        with pytest.raises(fp8lin.Fp8LinError) as e:
            fp8lin.fp8lin_step_policy(None, 0, step, n)
        assert e.value.status == fp8lin.EINVAL
    with pytest.raises(fp8lin.Fp8LinError):
        fp8lin.fp8lin_step_policy(None, 2, 0, 8)


MUTATIONS = [
    lambda p: p.update(extra=1),
    lambda p: p.pop("overlap"),
    lambda p: p.pop("reasoner"),
    lambda p: p.update(schema_version=2),
    lambda p: p.update(schema_version=True),
    lambda p: p.update(type="sigma_range"),
    lambda p: p.update(index_space="timestep"),
    lambda p: p.update(default_mode="w8a16"),
    lambda p: p.update(overlap="a8"),
    lambda p: p.update(first_steps=-1),
    lambda p: p.update(last_steps=1.5),
    lambda p: p.update(first_steps=None),
    lambda p: p.update(reasoner="nvfp4"),
]


@pytest.mark.parametrize("mutate", MUTATIONS)
def test_c_policy_fails_closed(golden, mutate):
    doc = copy.deepcopy(golden["policy"])
    mutate(doc)
    with pytest.raises(opolicy.PolicyError):  # the oracle refuses it too
        opolicy.validate(doc)
    pol = fp8lin.policy_from_json(doc)
    assert fp8lin.fp8lin_policy_validate(pol) == fp8lin.EPOLICY
    with pytest.raises(fp8lin.Fp8LinError) as e:
        fp8lin.fp8lin_step_policy(pol, 0, 0, 8)
    assert e.value.status == fp8lin.EPOLICY


def test_policy_validate_null_pointer(lib):
    assert lib.fp8lin_policy_validate(None) == fp8lin.EINVAL


# ---------------------------------------------------------------- argument validation


def q(lib, x=FAKE, out=FAKE, rows=4, cols=64, s=0.01):
    return lib.fp8lin_quantize_static(x, out, rows, cols, s, None)


def test_quantize_validation(lib):
    nan, inf = float("nan"), float("inf")
    assert q(lib, x=None) == fp8lin.EINVAL
    assert q(lib, rows=-1) == fp8lin.EINVAL
    assert q(lib, cols=24) == fp8lin.ELAYOUT
    assert q(lib, x=FAKE + 8) == fp8lin.ELAYOUT
    assert q(lib, out=FAKE + 4) == fp8lin.ELAYOUT
    for s in (0.0, -1.0, nan, inf, 1e-39, 2.0**127):
        assert q(lib, s=s) == fp8lin.ESCALE, s
    assert q(lib, cols=1 << 24) == fp8lin.EUNSUPPORTED
    before = fp8lin.fp8lin_launch_count(fp8lin.KERNEL_QUANTIZE)
    assert q(lib, rows=0) == fp8lin.OK  # zero rows: a no-op that launches nothing
    assert fp8lin.fp8lin_launch_count(fp8lin.KERNEL_QUANTIZE) == before


def g8(lib, qx=FAKE, qw=FAKE, y=FAKE, M=4, N=64, K=64, ldy=64, si=0.01, sw=0.001):
    return lib.fp8lin_gemm_w8a8(qx, qw, y, M, N, K, ldy, si, sw, None)


def test_gemm_w8a8_validation(lib):
    assert g8(lib, qw=None) == fp8lin.EINVAL
    assert g8(lib, K=0) == fp8lin.EINVAL
    assert g8(lib, N=0) == fp8lin.EINVAL
    assert g8(lib, K=40) == fp8lin.ELAYOUT
    assert g8(lib, N=60, ldy=64) == fp8lin.ELAYOUT
    assert g8(lib, ldy=56) == fp8lin.ELAYOUT
    assert g8(lib, y=FAKE + 2) == fp8lin.ELAYOUT
    assert g8(lib, si=float("nan")) == fp8lin.ESCALE
    assert g8(lib, sw=0.0) == fp8lin.ESCALE
    assert g8(lib, si=2.0**-100, sw=2.0**-100) == fp8lin.ESCALE  # product underflows
    assert g8(lib, M=1 << 31) == fp8lin.EUNSUPPORTED
    # the tile plans count 256-row tiles in 32 bits: M + 255 must not overflow
    assert g8(lib, M=(1 << 31) - 255, K=16) == fp8lin.EUNSUPPORTED
    assert g8(lib, K=1 << 22) == fp8lin.EUNSUPPORTED
    assert g8(lib, N=1 << 22, ldy=1 << 22) == fp8lin.EUNSUPPORTED
    assert g8(lib, ldy=1 << 22) == fp8lin.EUNSUPPORTED
    before = fp8lin.fp8lin_launch_count(fp8lin.KERNEL_GEMM_W8A8)
    assert g8(lib, M=0) == fp8lin.OK
    assert fp8lin.fp8lin_launch_count(fp8lin.KERNEL_GEMM_W8A8) == before


def test_gemm_w8a16_refuses_quantized_activation(lib):
    args = (FAKE, FAKE, FAKE, 4, 64, 64, 64, 0.001, None)
    assert lib.fp8lin_gemm_w8a16(args[0], fp8lin.DT_E4M3, *args[1:]) == fp8lin.EDTYPE
    assert lib.fp8lin_gemm_w8a16(args[0], 7, *args[1:]) == fp8lin.EINVAL
    assert lib.fp8lin_gemm_w8a16(FAKE, fp8lin.DT_BF16, FAKE, FAKE, 4, 64, 40, 64, 0.001, None) == fp8lin.ELAYOUT
    assert lib.fp8lin_gemm_w8a16(FAKE, fp8lin.DT_BF16, FAKE, FAKE, 0, 64, 64, 64, 0.001, None) == fp8lin.OK
    # float32 needs the workspace entry point; binary16 is accepted
    assert lib.fp8lin_gemm_w8a16(args[0], fp8lin.DT_F32, *args[1:]) == fp8lin.EDTYPE
    assert lib.fp8lin_gemm_w8a16(FAKE, fp8lin.DT_F16, FAKE, FAKE, 0, 64, 64, 64, 0.001, None) == fp8lin.OK
    assert lib.fp8lin_gemm_w8a16(FAKE, fp8lin.DT_F16, FAKE, FAKE, 4, 64, 40, 64, 0.001, None) == fp8lin.ELAYOUT


def g16f32(lib, x=FAKE, w=FAKE, y=FAKE, M=4, N=64, K=64, ldy=64, sw=0.001, ws=FAKE, wsb=None):
    if wsb is None:
        wsb = lib.fp8lin_w8a16_f32_workspace_bytes(M, K)
    return lib.fp8lin_gemm_w8a16_f32(x, w, y, M, N, K, ldy, sw, ws, wsb, None)


def test_gemm_w8a16_f32_validation(lib):
    ws = lib.fp8lin_w8a16_f32_workspace_bytes
    assert ws(4, 64) == 4 * 3 * 64 * 2
    assert ws(4, 80) == 4 * 3 * 128 * 2  # rows padded to 64 values
    assert ws(0, 64) == 0
    assert ws(-1, 64) == -1 and ws(4, 1 << 20) == -1
    assert g16f32(lib, wsb=4 * 3 * 64 * 2 - 1) == fp8lin.EINVAL
    assert g16f32(lib, ws=None) == fp8lin.EINVAL
    assert g16f32(lib, ws=FAKE + 8) == fp8lin.ELAYOUT
    assert g16f32(lib, x=FAKE + 4) == fp8lin.ELAYOUT
    assert g16f32(lib, K=40) == fp8lin.ELAYOUT
    assert g16f32(lib, K=1 << 20) == fp8lin.EUNSUPPORTED
    assert g16f32(lib, ldy=32) == fp8lin.ELAYOUT
    assert g16f32(lib, sw=0.0) == fp8lin.ESCALE
    before = [fp8lin.fp8lin_launch_count(k) for k in (fp8lin.KERNEL_SPLIT, fp8lin.KERNEL_GEMM_W8A16)]
    assert g16f32(lib, M=0, x=None, y=None, ws=None, wsb=0) == fp8lin.OK
    assert [fp8lin.fp8lin_launch_count(k) for k in (fp8lin.KERNEL_SPLIT, fp8lin.KERNEL_GEMM_W8A16)] == before


def grp(lib, n=(64, 64, 64), si=0.01, sw=(0.001, 0.001, 0.001), qx=FAKE, M=4, K=64, nproj=3):
    vp, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    k = len(n)
    return lib.fp8lin_gemm_w8a8_group(
        qx, M, K, nproj, (vp * k)(*[FAKE] * k), (i64 * k)(*n), (f32 * k)(*sw), si, (vp * k)(*[FAKE] * k), None
    )


def test_gemm_w8a8_group_validation(lib):
    assert grp(lib, nproj=0) == fp8lin.EINVAL
    assert grp(lib, nproj=5, n=(64,) * 5, sw=(0.001,) * 5) == fp8lin.EINVAL
    assert grp(lib, qx=None) == fp8lin.EINVAL
    assert grp(lib, qx=FAKE + 8) == fp8lin.ELAYOUT
    assert grp(lib, K=40) == fp8lin.ELAYOUT
    assert grp(lib, n=(64, 60, 64)) == fp8lin.ELAYOUT
    assert grp(lib, si=float("inf")) == fp8lin.ESCALE
    assert grp(lib, sw=(0.001, 0.0, 0.001)) == fp8lin.ESCALE
    assert grp(lib, si=2.0**-100, sw=(2.0**-100,) * 3) == fp8lin.ESCALE  # alpha underflows
    assert grp(lib, K=1 << 22) == fp8lin.EUNSUPPORTED
    assert grp(lib, M=(1 << 31) - 255, K=16) == fp8lin.EUNSUPPORTED
    before = fp8lin.fp8lin_launch_count(fp8lin.KERNEL_GEMM_W8A8)
    assert grp(lib, M=0) == fp8lin.OK
    assert fp8lin.fp8lin_launch_count(fp8lin.KERNEL_GEMM_W8A8) == before


def gus(lib, qx=FAKE, M=4, K=64, wg=FAKE, wu=FAKE, inter=64, si=0.01, sg=0.001, su=0.001, sh=0.02, h=FAKE):
    return lib.fp8lin_gate_up_swiglu_w8a8(qx, M, K, wg, wu, inter, si, sg, su, sh, h, None)


def test_gate_up_swiglu_validation(lib):
    assert gus(lib, qx=None) == fp8lin.EINVAL
    assert gus(lib, h=None) == fp8lin.EINVAL
    assert gus(lib, wu=None) == fp8lin.EINVAL
    assert gus(lib, inter=0) == fp8lin.EINVAL
    assert gus(lib, inter=40) == fp8lin.ELAYOUT  # I must be a multiple of 16
    assert gus(lib, K=40) == fp8lin.ELAYOUT
    assert gus(lib, wg=FAKE + 8) == fp8lin.ELAYOUT
    assert gus(lib, h=FAKE + 4) == fp8lin.ELAYOUT
    assert gus(lib, sh=0.0) == fp8lin.ESCALE
    assert gus(lib, su=float("nan")) == fp8lin.ESCALE
    assert gus(lib, si=2.0**-100, sg=2.0**-100) == fp8lin.ESCALE  # alpha underflows
    assert gus(lib, inter=1 << 22) == fp8lin.EUNSUPPORTED
    assert gus(lib, K=1 << 22) == fp8lin.EUNSUPPORTED
    assert gus(lib, M=(1 << 31) - 255, K=16) == fp8lin.EUNSUPPORTED
    before = fp8lin.fp8lin_launch_count(fp8lin.KERNEL_GATE_UP_SWIGLU)
    assert gus(lib, M=0, qx=None, h=None) == fp8lin.OK
    assert fp8lin.fp8lin_launch_count(fp8lin.KERNEL_GATE_UP_SWIGLU) == before


def gus16(lib, x=FAKE, dt=0, M=4, K=64, wg=FAKE, wu=FAKE, inter=64, sg=0.001, su=0.001, h=FAKE):
    return lib.fp8lin_gate_up_swiglu_w8a16(x, dt, M, K, wg, wu, inter, sg, su, h, None)


def test_gate_up_swiglu_w8a16_validation(lib):
    assert gus16(lib, dt=fp8lin.DT_E4M3) == fp8lin.EDTYPE  # the 16-bit step refuses FP8 activations
    assert gus16(lib, dt=7) == fp8lin.EINVAL
    assert gus16(lib, dt=fp8lin.DT_F32) == fp8lin.EDTYPE
    assert gus16(lib, dt=fp8lin.DT_F16, inter=24) == fp8lin.ELAYOUT  # binary16 passes the dtype check
    assert gus16(lib, x=None) == fp8lin.EINVAL
    assert gus16(lib, wg=None) == fp8lin.EINVAL
    assert gus16(lib, inter=24) == fp8lin.ELAYOUT
    assert gus16(lib, K=40) == fp8lin.ELAYOUT
    assert gus16(lib, h=FAKE + 2) == fp8lin.ELAYOUT
    assert gus16(lib, sg=float("inf")) == fp8lin.ESCALE
    assert gus16(lib, inter=1 << 22) == fp8lin.EUNSUPPORTED
    before = fp8lin.fp8lin_launch_count(fp8lin.KERNEL_GATE_UP_SWIGLU)
    assert gus16(lib, M=0, x=None, h=None) == fp8lin.OK
    assert fp8lin.fp8lin_launch_count(fp8lin.KERNEL_GATE_UP_SWIGLU) == before


def qdyn(lib, x=FAKE, q=FAKE, rows=4, cols=64, scale=FAKE, ws=FAKE):
    return lib.fp8lin_quantize_dynamic(x, q, rows, cols, scale, ws, None)


def test_quantize_dynamic_validation(lib):
    assert qdyn(lib, x=None) == fp8lin.EINVAL
    assert qdyn(lib, scale=None) == fp8lin.EINVAL
    assert qdyn(lib, ws=None) == fp8lin.EINVAL
    assert qdyn(lib, cols=24) == fp8lin.ELAYOUT
    assert qdyn(lib, scale=FAKE + 2) == fp8lin.ELAYOUT
    assert qdyn(lib, ws=FAKE + 1) == fp8lin.ELAYOUT
    assert qdyn(lib, cols=1 << 24) == fp8lin.EUNSUPPORTED
    before = [fp8lin.fp8lin_launch_count(k) for k in (fp8lin.KERNEL_AMAX, fp8lin.KERNEL_QUANTIZE)]
    assert qdyn(lib, rows=0, x=None, q=None, scale=None, ws=None) == fp8lin.OK  # empty: nothing launched
    assert [fp8lin.fp8lin_launch_count(k) for k in (fp8lin.KERNEL_AMAX, fp8lin.KERNEL_QUANTIZE)] == before


def test_gemm_dev_scale_validation(lib):
    def g(qx=FAKE, qw=FAKE, y=FAKE, M=4, N=64, K=64, ldy=64, sd=FAKE, sw=0.001):
        return lib.fp8lin_gemm_w8a8_dev_scale(qx, qw, y, M, N, K, ldy, sd, sw, None)

    assert g(sd=None) == fp8lin.EINVAL
    assert g(sd=FAKE + 2) == fp8lin.ELAYOUT
    assert g(K=40) == fp8lin.ELAYOUT
    assert g(sw=float("nan")) == fp8lin.ESCALE
    assert g(M=0) == fp8lin.OK


def qkv(lib, scales_in=(0.01, 0.01, 0.01), n=(64, 64, 64), mode=0, ws=FAKE, nproj=3):
    vp, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    k = len(n)
    return lib.fp8lin_qkv_shared(
        FAKE, 4, 64, nproj, (vp * k)(*[FAKE] * k), (i64 * k)(*n), (f32 * k)(*[0.001] * k),
        (f32 * k)(*scales_in), (vp * k)(*[FAKE] * k), ws, mode, None,
    )


def test_qkv_shared_validation(lib):
    nudged = float(ctypes.c_float(0.01).value) * (1 + 2**-23)
    assert qkv(lib, scales_in=(0.01, nudged, 0.01)) == fp8lin.ESCALE
    assert qkv(lib, mode=fp8lin.MODE_W8A16, scales_in=(0.01, 0.02, 0.01)) == fp8lin.ESCALE
    assert qkv(lib, n=(64, 60, 64)) == fp8lin.ELAYOUT
    assert qkv(lib, ws=None) == fp8lin.EINVAL  # W8A8 needs the workspace
    assert qkv(lib, mode=5) == fp8lin.EINVAL
    assert qkv(lib, nproj=0) == fp8lin.EINVAL
    assert qkv(lib, nproj=5, n=(64,) * 5, scales_in=(0.01,) * 5) == fp8lin.EINVAL


def test_swiglu_validation(lib):
    f = lib.fp8lin_swiglu_2in_quant
    assert f(FAKE, FAKE, FAKE, 3, 4, 64, 0.1, None) == fp8lin.EINVAL
    assert f(FAKE, FAKE, FAKE, fp8lin.DT_E4M3, 4, 40, 0.1, None) == fp8lin.ELAYOUT
    assert f(FAKE, FAKE + 2, FAKE, fp8lin.DT_E4M3, 4, 64, 0.1, None) == fp8lin.ELAYOUT
    assert f(FAKE, FAKE, FAKE, fp8lin.DT_E4M3, 4, 64, 0.0, None) == fp8lin.ESCALE
    assert f(FAKE, FAKE, FAKE, fp8lin.DT_BF16, 0, 64, 0.0, None) == fp8lin.OK  # scale unused for bf16


def test_swiglu_2in_validation(lib):
    f = lib.fp8lin_swiglu_2in
    BF, F16, E4, F32 = fp8lin.DT_BF16, fp8lin.DT_F16, fp8lin.DT_E4M3, fp8lin.DT_F32
    assert f(FAKE, FAKE, 9, FAKE, E4, 4, 64, 0.1, None) == fp8lin.EINVAL
    assert f(FAKE, FAKE, F16, FAKE, 9, 4, 64, 0.1, None) == fp8lin.EINVAL
    assert f(FAKE, FAKE, E4, FAKE, E4, 4, 64, 0.1, None) == fp8lin.EDTYPE
    assert f(FAKE, FAKE, F32, FAKE, F32, 4, 64, 0.1, None) == fp8lin.EDTYPE
    assert f(FAKE, FAKE, F16, FAKE, BF, 4, 64, 0.1, None) == fp8lin.EDTYPE  # 16-bit out = in format
    assert f(FAKE, FAKE, BF, FAKE, F16, 4, 64, 0.1, None) == fp8lin.EDTYPE
    assert f(FAKE, FAKE, F16, FAKE, E4, 4, 40, 0.1, None) == fp8lin.ELAYOUT
    assert f(FAKE, FAKE, F16, FAKE, E4, 4, 64, 0.0, None) == fp8lin.ESCALE
    before = fp8lin.fp8lin_launch_count(fp8lin.KERNEL_SWIGLU)
    assert f(None, None, F16, None, F16, 0, 64, 0.0, None) == fp8lin.OK
    assert fp8lin.fp8lin_launch_count(fp8lin.KERNEL_SWIGLU) == before


def qkn(lib, q=FAKE, k=FAKE, qo=FAKE, ko=FAKE, t=4, qh=2, kh=2, d=128, wq=None, wk=None, c=FAKE, s=FAKE, eps=1e-6):
    return lib.fp8lin_qk_norm_rope(q, k, qo, ko, t, qh, kh, d, wq, wk, c, s, eps, None)


def test_qk_norm_rope_validation(lib):
    assert qkn(lib, d=96) == fp8lin.EUNSUPPORTED
    assert qkn(lib, d=256) == fp8lin.EUNSUPPORTED
    assert qkn(lib, eps=0.0) == fp8lin.EINVAL
    assert qkn(lib, eps=float("nan")) == fp8lin.EINVAL
    assert qkn(lib, qh=0) == fp8lin.EINVAL
    assert qkn(lib, t=-1) == fp8lin.EINVAL
    assert qkn(lib, q=None) == fp8lin.EINVAL
    assert qkn(lib, c=None) == fp8lin.EINVAL
    assert qkn(lib, k=None) == fp8lin.EINVAL  # K heads without a K tensor
    assert qkn(lib, k=FAKE + 8) == fp8lin.ELAYOUT
    assert qkn(lib, s=FAKE + 4) == fp8lin.ELAYOUT
    assert qkn(lib, wq=FAKE + 2) == fp8lin.ELAYOUT
    assert qkn(lib, t=1 << 31) == fp8lin.EUNSUPPORTED
    before = fp8lin.fp8lin_launch_count(fp8lin.KERNEL_QK_NORM_ROPE)
    assert qkn(lib, t=0, q=None, k=None, qo=None, ko=None, c=None, s=None) == fp8lin.OK
    assert fp8lin.fp8lin_launch_count(fp8lin.KERNEL_QK_NORM_ROPE) == before


def qnr(lib, nproj=3, n=(256, 256, 256), qx=FAKE, M=4, K=64, c=FAKE, s=FAKE, wq=None, eps=1e-6, si=0.01):
    vp, i64, f32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float
    k = len(n)
    return lib.fp8lin_qkv_w8a8_norm_rope(qx, M, K, nproj, (vp * k)(*[FAKE] * k), (i64 * k)(*n), (f32 * k)(*[0.001] * k),
                                         si, (vp * k)(*[FAKE] * k), wq, None, c, s, eps, None)


def test_qkv_norm_rope_validation(lib):
    assert qnr(lib, nproj=1, n=(256,)) == fp8lin.EINVAL
    assert qnr(lib, nproj=4, n=(256,) * 4) == fp8lin.EINVAL
    assert qnr(lib, n=(192, 256, 256)) == fp8lin.ELAYOUT  # Q not whole heads of 128
    assert qnr(lib, n=(256, 200, 256)) == fp8lin.ELAYOUT
    assert qnr(lib, c=None) == fp8lin.EINVAL
    assert qnr(lib, s=FAKE + 4) == fp8lin.ELAYOUT
    assert qnr(lib, wq=FAKE + 2) == fp8lin.ELAYOUT
    assert qnr(lib, eps=0.0) == fp8lin.EINVAL
    assert qnr(lib, si=0.0) == fp8lin.ESCALE
    before = fp8lin.fp8lin_launch_count(fp8lin.KERNEL_GEMM_W8A8)
    assert qnr(lib, M=0, qx=None, c=None, s=None) == fp8lin.OK
    assert fp8lin.fp8lin_launch_count(fp8lin.KERNEL_GEMM_W8A8) == before


def gsk(lib, M=4, N=64, K=256, ldy=64, splits=2, ws=FAKE, wsb=None, si=0.01, sw=0.001, qx=FAKE):
    if wsb is None:
        wsb = splits * M * N * 4
    return lib.fp8lin_gemm_w8a8_splitk(qx, FAKE, FAKE, M, N, K, ldy, si, sw, splits, ws, wsb, None)


def test_gemm_splitk_validation(lib):
    assert gsk(lib, splits=3) == fp8lin.EINVAL
    assert gsk(lib, splits=8) == fp8lin.EINVAL
    assert gsk(lib, K=16 * 4 + 16, splits=4) == fp8lin.ELAYOUT  # K not a multiple of 16 * splits
    assert gsk(lib, wsb=2 * 4 * 64 * 4 - 1) == fp8lin.EINVAL
    assert gsk(lib, ws=None) == fp8lin.EINVAL
    assert gsk(lib, ws=FAKE + 8) == fp8lin.ELAYOUT
    assert gsk(lib, si=0.0) == fp8lin.ESCALE
    assert gsk(lib, ldy=32) == fp8lin.ELAYOUT
    before = [fp8lin.fp8lin_launch_count(k) for k in (fp8lin.KERNEL_GEMM_W8A8, fp8lin.KERNEL_SPLITK_REDUCE)]
    assert gsk(lib, M=0, qx=None, ws=None, wsb=0) == fp8lin.OK
    assert gsk(lib, M=0, qx=None, splits=1) == fp8lin.OK
    assert [fp8lin.fp8lin_launch_count(k) for k in (fp8lin.KERNEL_GEMM_W8A8, fp8lin.KERNEL_SPLITK_REDUCE)] == before


def gsk16(lib, M=2, N=64, K=64, ldy=64, sw=0.5, splits=2, ws=FAKE, wsb=2 * 2 * 64 * 4, x=FAKE, dt=fp8lin.DT_BF16):
    return lib.fp8lin_gemm_w8a16_splitk(x, dt, FAKE, FAKE, M, N, K, ldy, sw, splits, ws, wsb, None)


def test_gemm_w8a16_splitk_validation(lib):
    """Every failing call returns before any launch (no GPU here); M = 0 is a no-op."""
    assert gsk16(lib, splits=3) == fp8lin.EINVAL
    assert gsk16(lib, dt=fp8lin.DT_E4M3) == fp8lin.EDTYPE
    assert gsk16(lib, dt=fp8lin.DT_F32) == fp8lin.EDTYPE
    assert gsk16(lib, dt=fp8lin.DT_F16) == fp8lin.EUNSUPPORTED  # the reduction writes bf16
    assert gsk16(lib, K=16 * 4 + 16, splits=4) == fp8lin.ELAYOUT
    assert gsk16(lib, wsb=2 * 2 * 64 * 4 - 1) == fp8lin.EINVAL
    assert gsk16(lib, ws=None) == fp8lin.EINVAL
    assert gsk16(lib, ws=FAKE + 8) == fp8lin.ELAYOUT
    assert gsk16(lib, x=FAKE + 8) == fp8lin.ELAYOUT
    assert gsk16(lib, sw=float("nan")) == fp8lin.ESCALE
    assert gsk16(lib, ldy=32) == fp8lin.ELAYOUT
    before = [fp8lin.fp8lin_launch_count(k) for k in (fp8lin.KERNEL_GEMM_W8A16, fp8lin.KERNEL_SPLITK_REDUCE)]
    assert gsk16(lib, M=0, x=None, ws=None, wsb=0) == fp8lin.OK
    assert gsk16(lib, M=0, x=None, splits=1) == fp8lin.OK
    assert [fp8lin.fp8lin_launch_count(k) for k in (fp8lin.KERNEL_GEMM_W8A16, fp8lin.KERNEL_SPLITK_REDUCE)] == before


def test_gemm_splitk_choice_is_one(lib):
    """No split beats the unsplit call: where 256 x 256 tiles would leave the device underfilled it runs
    128 x 128 tiles."""
    for choice in (lib.fp8lin_gemm_w8a8_splitk_choice, lib.fp8lin_gemm_w8a16_splitk_choice):
        for m, n, k in ((16384, 4096, 4096), (8192, 4096, 4096), (1024, 4096, 4096), (1024, 4096, 1024),
                        (128, 512, 512), (0, 4096, 4096)):
            assert choice(m, n, k) == 1


def skna(lib, qx=FAKE, qw=FAKE, y=FAKE, M=1024, N=4096, K=4096, ldy=4096, si=0.01, sw=0.001, splits=2):
    return lib.fp8lin_gemm_w8a8_splitk_noalloc(qx, qw, y, M, N, K, ldy, si, sw, splits, None)


def test_gemm_w8a8_splitk_noalloc_validation(lib):
    """Everything is refused before the scratch array is looked up or anything is enqueued."""
    assert skna(lib, splits=3) == fp8lin.EINVAL
    assert skna(lib, qw=None) == fp8lin.EINVAL
    assert skna(lib, K=4096 + 16, splits=2) == fp8lin.ELAYOUT  # K a multiple of 16 * splits
    assert skna(lib, qx=FAKE + 4) == fp8lin.ELAYOUT
    assert skna(lib, si=float("nan")) == fp8lin.ESCALE
    # the float32 partials must fit the 32 MiB scratch array: 4 x 1024 x 4096 x 4 bytes is 64 MiB
    assert fp8lin.SCRATCH_BYTES == 32 * 1024 * 1024
    assert skna(lib, splits=4) == fp8lin.EUNSUPPORTED
    assert skna(lib, M=1025, splits=2) == fp8lin.EUNSUPPORTED
    before = [fp8lin.fp8lin_launch_count(k) for k in (fp8lin.KERNEL_GEMM_W8A8, fp8lin.KERNEL_SPLITK_REDUCE)]
    assert skna(lib, M=0, qx=None, y=None) == fp8lin.OK
    assert [fp8lin.fp8lin_launch_count(k) for k in (fp8lin.KERNEL_GEMM_W8A8, fp8lin.KERNEL_SPLITK_REDUCE)] == before
