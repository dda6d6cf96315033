"""GPU parity: dynamic per-tensor FP8 quantization and the GEMM with a device input scale.

The device scale must equal the oracle's float32 scale exactly and the codes
must equal the oracle's bit for bit (the static rule with that scale);
fp8lin_gemm_w8a8_dev_scale must equal fp8lin_gemm_w8a8 with the same scale
given on the host, bit for bit.
"""

import numpy as np
import pytest
import torch

import w8a16_linear_layers_amd as fp8lin
from oracle import dynamic, linear
from tests.helpers import announce, assert_gemm_close, f32, sample_rows, u8
from workloads import config1, config3, normal_bf16, random_e4m3_codes

pytestmark = pytest.mark.gpu


def run_dynamic(x_cpu, gpu, ws=None, scale=None):
    q, s = fp8lin.fp8lin_quantize_dynamic(x_cpu.to(gpu), scale=scale, workspace=ws)
    torch.cuda.synchronize()
    return u8(q), float(s.cpu()[0])


def check(x_cpu, gpu, **kw):
    got, s = run_dynamic(x_cpu, gpu, **kw)
    ref, s_ref = dynamic.quantize_dynamic(f32(x_cpu))
    assert s == s_ref, (s, s_ref)
    assert np.array_equal(got, ref), "mismatches: %d" % np.count_nonzero(got != ref)
    return s


@pytest.mark.parametrize("sigma,seed", [(0.35, 1), (1.0, 2), (1e-3, 3), (300.0, 4), (1e-30, 5), (1e30, 6)])
def test_normal_tensors(gpu, sigma, seed):
    announce("dynamic quantize sigma=%g" % sigma)
    check(normal_bf16((300, 1040), sigma, seed), gpu)


@pytest.mark.parametrize("shape", [(1, 16), (37, 208), (3, 5, 64), (513, 4096 + 16)])
def test_ragged_shapes(gpu, shape):
    announce("dynamic quantize ragged %s" % (shape,))
    check(normal_bf16(shape, 0.5, 7), gpu)


def test_non_finite_elements(gpu):
    announce("dynamic quantize with inf/nan")
    x = normal_bf16((64, 128), 0.35, 8)
    x[0, 0], x[5, 17], x[63, 127] = float("inf"), float("-inf"), float("nan")
    s = check(x, gpu)
    finite = f32(x)[np.isfinite(f32(x))]
    assert s == float(np.float32(np.abs(finite).max()) / np.float32(448))


def test_degenerate_tensors(gpu):
    announce("dynamic quantize degenerate")
    assert check(torch.zeros((8, 64), dtype=torch.bfloat16), gpu) == 2.0**-126
    assert check(-torch.zeros((8, 64), dtype=torch.bfloat16), gpu) == 2.0**-126
    t = torch.zeros((4, 32), dtype=torch.bfloat16)
    t[2, 5] = 2.0**-133
    assert check(t, gpu) == 2.0**-126
    nan = torch.full((2, 16), float("nan"), dtype=torch.bfloat16)
    check(nan, gpu)
    big = normal_bf16((16, 64), 1.0, 9) * 3.0e38 / 5
    check(big, gpu)


def test_full_size_activation(gpu):
    case = config3()
    announce("dynamic quantize x %s" % (tuple(case.x.shape),))
    check(case.x, gpu)


def test_workspace_and_scale_reused(gpu):
    announce("dynamic quantize buffers reused")
    ws = torch.empty(1, dtype=torch.int32, device=gpu)
    sc = torch.empty(1, dtype=torch.float32, device=gpu)
    check(normal_bf16((64, 256), 4.0, 10), gpu, ws=ws, scale=sc)
    # a second tensor with a much smaller amax: the workspace is cleared on every call
    check(normal_bf16((64, 256), 0.01, 11), gpu, ws=ws, scale=sc)


@pytest.mark.parametrize("m,k,n", [(300, 528, 1040), (16384, 4096, 4096)])
def test_gemm_dev_scale(gpu, m, k, n):
    announce("gemm_w8a8 dev scale m=%d k=%d n=%d" % (m, k, n))
    x = (config3(m=m, k=k, n=n).x if m == 16384 else normal_bf16((m, k), 0.35, 12))
    qw = random_e4m3_codes((n, k), 13).to(gpu)
    sw = 3.1e-4
    q, s_dev = fp8lin.fp8lin_quantize_dynamic(x.to(gpu))
    y = fp8lin.fp8lin_gemm_w8a8_dev_scale(q, qw, s_dev, sw)
    s = float(s_dev.cpu()[0])
    y_host = fp8lin.fp8lin_gemm_w8a8(q, qw, s, sw)
    torch.cuda.synchronize()
    assert torch.equal(y, y_host)
    rows = sample_rows(m, 96, 14) if m > 4096 else np.arange(m)
    assert s == dynamic.dynamic_scale(f32(x))
    ref = linear.gemm_w8a8(u8(q)[rows], u8(qw), s, sw)
    assert_gemm_close(f32(y)[rows], ref, "dev scale")


def test_dynamic_step_config1(gpu):
    """quantize_dynamic + gemm_dev_scale against the oracle's dynamic chain."""
    announce("dynamic step config1")
    case = config1()
    qw = fp8lin.fp8lin_quantize_static(case.w.to(gpu), case.weight_scale)
    q, s_dev = fp8lin.fp8lin_quantize_dynamic(case.x.to(gpu))
    y = fp8lin.fp8lin_gemm_w8a8_dev_scale(q, qw, s_dev, case.weight_scale)
    q_ref, s_ref = dynamic.quantize_dynamic(f32(case.x))
    assert np.array_equal(u8(q), q_ref)
    ref = linear.gemm_w8a8(q_ref, linear.quantize_static(f32(case.w), case.weight_scale), s_ref, case.weight_scale)
    assert_gemm_close(y, ref, "dynamic step")
