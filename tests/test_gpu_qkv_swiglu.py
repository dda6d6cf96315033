"""GPU parity: shared-QKV projections and the two-input SwiGLU.

Shared QKV: the workspace codes equal the oracle's quantization bit for bit,
each projection meets the GEMM tolerance, the grouped launch equals three
separate calls, and the single quantization is checked by launch count
(one per W8A8 call, none on a 16-bit step), as the pages' tests check it by
storage identity rather than by dtype.

SwiGLU: E4M3 codes equal the oracle's except where silu(g) u / s_h lies
within relative 2^-20 of a rounding midpoint (both neighbours accepted, the
count reported); bf16 output within one bf16 ulp of the exact product.
"""

import numpy as np
import pytest
import torch

import w8a16_linear_layers_amd as fp8lin
from oracle import bf16 as obf16
from oracle import linear, swiglu
from tests.helpers import announce, assert_gemm_close, check_swiglu_codes, f32, sample_rows, u8
from workloads import config3, config4, normal_bf16, random_e4m3_codes

pytestmark = pytest.mark.gpu


def quantized_group(case, gpu):
    qg, qr = [], []
    for w, s in zip(case.ws, case.weight_scales):
        qg.append(fp8lin.fp8lin_quantize_static(w.to(gpu), s))
        qr.append(linear.quantize_static(f32(w), s))
        assert np.array_equal(u8(qg[-1]), qr[-1])
    return qg, qr


@pytest.mark.parametrize("m,k,n", [(300, 528, 264), (16384, 4096, 4096)])
def test_qkv_shared_w8a8(gpu, m, k, n):
    announce("qkv_shared w8a8 m=%d k=%d n=%d" % (m, k, n))
    case = config3(m=m, k=k, n=n)
    qg, qr = quantized_group(case, gpu)
    x = case.x.to(gpu)
    sin = [case.input_scale] * 3
    c0 = [fp8lin.fp8lin_launch_count(i) for i in range(4)]
    outs, ws = fp8lin.fp8lin_qkv_shared(x, qg, case.weight_scales, sin, fp8lin.MODE_W8A8)
    c1 = [fp8lin.fp8lin_launch_count(i) for i in range(4)]
    torch.cuda.synchronize()
    assert c1[fp8lin.KERNEL_QUANTIZE] - c0[fp8lin.KERNEL_QUANTIZE] == 1
    assert c1[fp8lin.KERNEL_GEMM_W8A8] - c0[fp8lin.KERNEL_GEMM_W8A8] == 1
    assert all(o.is_contiguous() and o.shape == (m, n) for o in outs)
    xr = f32(case.x)
    rows = sample_rows(m, 160, 5) if m > 4096 else np.arange(m)
    qx_ref = linear.quantize_static(xr[rows], case.input_scale)
    assert np.array_equal(u8(ws)[rows], qx_ref)
    for i in range(3):
        ref = linear.gemm_w8a8(qx_ref, qr[i], case.input_scale, case.weight_scales[i])
        assert_gemm_close(f32(outs[i])[rows], ref, "proj %d" % i)
    # the grouped launch equals separate calls on the same codes, bit for bit
    for i in range(3):
        y = fp8lin.fp8lin_gemm_w8a8(ws, qg[i], case.input_scale, case.weight_scales[i])
        assert torch.equal(y, outs[i])


@pytest.mark.parametrize("m,k,ns", [(300, 528, (264, 136, 520)), (16384, 4096, (4096, 4096, 4096)), (77, 64, (8, 24))])
def test_gemm_w8a8_group(gpu, m, k, ns):
    """One launch over the projections of a group equals the oracle per projection."""
    announce("gemm_w8a8_group m=%d k=%d n=%s" % (m, k, ns))
    case = config3(m=m, k=k, n=max(ns))
    ws = [w[:n] for w, n in zip(case.ws, ns)]
    sw = case.weight_scales[: len(ns)]
    qg = [fp8lin.fp8lin_quantize_static(w.contiguous().to(gpu), s) for w, s in zip(ws, sw)]
    qx = fp8lin.fp8lin_quantize_static(case.x.to(gpu), case.input_scale)
    c0 = fp8lin.fp8lin_launch_count(fp8lin.KERNEL_GEMM_W8A8)
    outs = fp8lin.fp8lin_gemm_w8a8_group(qx, qg, case.input_scale, sw)
    assert fp8lin.fp8lin_launch_count(fp8lin.KERNEL_GEMM_W8A8) - c0 == 1
    torch.cuda.synchronize()
    rows = sample_rows(m, 160, 9) if m > 4096 else np.arange(m)
    qx_ref = linear.quantize_static(f32(case.x)[rows], case.input_scale)
    for i, (w, s) in enumerate(zip(ws, sw)):
        assert outs[i].shape == (m, ns[i]) and outs[i].is_contiguous()
        ref = linear.gemm_w8a8(qx_ref, linear.quantize_static(f32(w.contiguous()), s), case.input_scale, s)
        assert_gemm_close(f32(outs[i])[rows], ref, "group proj %d" % i)


@pytest.mark.parametrize("k", [384, 640])
def test_four_ragged_projections_many_tiles(gpu, k):
    """Four projections of ragged widths in one launch (the W8A8 group and the W8A16 shared call) at 4100 rows:
    17 x 25 = 425 tiles of 256 x 256 for 256 compute units, so workgroups cross projection boundaries and
    change tiles after an odd number of 128-byte W8A8 stages (3, 5). Rows from every M-tile against the
    oracle, per projection."""
    m, ns = 4100, (264, 4104, 136, 1032)
    announce("four ragged projections m=%d k=%d" % (m, k))
    q = random_e4m3_codes((m, k), 100 + k)
    qws = [random_e4m3_codes((n, k), 200 + n + k) for n in ns]
    x = normal_bf16((m, k), 0.35, 300 + k)
    s_in, sw = 1.7e-3, [3.1e-5, 2.2e-5, 4.7e-5, 1.3e-5]
    qwg = [w.to(gpu) for w in qws]
    outs8 = fp8lin.fp8lin_gemm_w8a8_group(q.to(gpu), qwg, s_in, sw)
    outs16, ws = fp8lin.fp8lin_qkv_shared(x.to(gpu), qwg, sw, [s_in] * 4, fp8lin.MODE_W8A16)
    torch.cuda.synchronize()
    assert ws is None
    rows = np.unique(np.concatenate([sample_rows(m, 48, k), np.arange(k % 256, m, 256), [m - 1]]))
    qr, xr = q.numpy()[rows], f32(x)[rows]
    for i in range(4):
        assert outs8[i].shape == (m, ns[i]) and outs16[i].shape == (m, ns[i])
        assert_gemm_close(f32(outs8[i])[rows], linear.gemm_w8a8(qr, qws[i].numpy(), s_in, sw[i]), "w8a8 proj %d" % i)
        assert_gemm_close(f32(outs16[i])[rows], linear.gemm_w8a16(xr, qws[i].numpy(), sw[i]), "w8a16 proj %d" % i)


def test_qkv_shared_w8a16_stands_down(gpu):
    announce("qkv_shared w8a16")
    case = config3(m=520, k=1024, n=512)
    qg, qr = quantized_group(case, gpu)
    x = case.x.to(gpu)
    c0 = [fp8lin.fp8lin_launch_count(i) for i in range(4)]
    outs, ws = fp8lin.fp8lin_qkv_shared(x, qg, case.weight_scales, [case.input_scale] * 3, fp8lin.MODE_W8A16)
    c1 = [fp8lin.fp8lin_launch_count(i) for i in range(4)]
    torch.cuda.synchronize()
    assert ws is None
    assert c1[fp8lin.KERNEL_QUANTIZE] == c0[fp8lin.KERNEL_QUANTIZE]
    assert c1[fp8lin.KERNEL_GEMM_W8A16] - c0[fp8lin.KERNEL_GEMM_W8A16] == 1
    xr = f32(case.x)
    for i in range(3):
        assert_gemm_close(outs[i], linear.gemm_w8a16(xr, qr[i], case.weight_scales[i]), "proj %d" % i)
        assert torch.equal(outs[i], fp8lin.fp8lin_gemm_w8a16(x, qg[i], case.weight_scales[i]))


def test_qkv_shared_refuses_unequal_input_scales(gpu):
    announce("qkv_shared unequal scales")
    case = config3(m=64, k=256, n=128)
    qg, _ = quantized_group(case, gpu)
    s = np.float32(case.input_scale)
    bad = [float(s), float(np.nextafter(s, np.float32(1))), float(s)]
    with pytest.raises(fp8lin.Fp8LinError) as e:
        fp8lin.fp8lin_qkv_shared(case.x.to(gpu), qg, case.weight_scales, bad, fp8lin.MODE_W8A8)
    assert e.value.status == fp8lin.ESCALE


def test_gate_up_group(gpu):
    """nproj = 2 (split gated MLP): one quantization feeding gate and up."""
    announce("gate/up group")
    case = config4(m=256, hidden=512, inter=1024, cal_rows=64)
    x = case.x.to(gpu)
    ws = [case.w_gate, case.w_up]
    ss = [case.s_gate, case.s_up]
    qg = [fp8lin.fp8lin_quantize_static(w.to(gpu), s) for w, s in zip(ws, ss)]
    outs, codes = fp8lin.fp8lin_qkv_shared(x, qg, ss, [case.input_scale] * 2, fp8lin.MODE_W8A8)
    xr = f32(case.x)
    qx = linear.quantize_static(xr, case.input_scale)
    assert np.array_equal(u8(codes), qx)
    for o, w, s in zip(outs, ws, ss):
        assert_gemm_close(o, linear.gemm_w8a8(qx, linear.quantize_static(f32(w), s), case.input_scale, s), "gate/up")


# ---------------------------------------------------------------- SwiGLU


@pytest.mark.parametrize("shape", [(1, 16), (37, 208), (1000, 1040)])
def test_swiglu_fp8_small(gpu, shape):
    announce("swiglu fp8 %s" % (shape,))
    g = normal_bf16(shape, 0.45, 51)
    u = normal_bf16(shape, 0.45, 52)
    s_h = 1.9 / 448
    out = fp8lin.fp8lin_swiglu_2in_quant(g.to(gpu), u.to(gpu), s_h)
    n = check_swiglu_codes(g, u, s_h, u8(out))
    print("near-midpoint differences: %d of %d" % (n, out.numel()))


def test_swiglu_fp8_full_size_sampled(gpu):
    """The gated-MLP SwiGLU at [8192, 16384]: gate/up from the W8A8 projections."""
    announce("swiglu fp8 full size")
    m, inter = 8192, 16384
    g = normal_bf16((m, inter), 0.45, 61)
    u = normal_bf16((m, inter), 0.45, 62)
    s_h = 2.1 / 448
    out = fp8lin.fp8lin_swiglu_2in_quant(g.to(gpu), u.to(gpu), s_h)
    torch.cuda.synchronize()
    rows = sample_rows(m, 64, 3)
    n = check_swiglu_codes(g[rows], u[rows], s_h, u8(out)[rows])
    print("near-midpoint differences: %d of %d" % (n, rows.size * inter))


def test_swiglu_bf16_output(gpu):
    announce("swiglu bf16")
    g = normal_bf16((300, 1040), 0.45, 71)
    u = normal_bf16((300, 1040), 0.45, 72)
    out = fp8lin.fp8lin_swiglu_2in_quant(g.to(gpu), u.to(gpu), out_dtype=fp8lin.DT_BF16)
    h = swiglu.swiglu_2in(f32(g), f32(u))
    got = f32(out).astype(np.float64)
    assert np.all(np.abs(got - h) <= obf16.ulp(h))


def test_swiglu_special_values(gpu):
    announce("swiglu special values")
    g = torch.tensor([0.0, 2.0, -3.0, 30.0, -90.0, 1.0, float("nan"), 0.5] * 2, dtype=torch.bfloat16).reshape(1, 16)
    u = torch.tensor([5.0, 0.0, 0.0, 1.5, 2.0, float("nan"), 1.0, -0.25] * 2, dtype=torch.bfloat16).reshape(1, 16)
    out = u8(fp8lin.fp8lin_swiglu_2in_quant(g.to(gpu), u.to(gpu), 1.0)).ravel()
    assert out[0] & 0x7F == 0 and out[1] & 0x7F == 0 and out[2] & 0x7F == 0
    assert out[3] == 0x63  # silu(30) * 1.5 is just below 45 -> nearest E4M3 value 44 (0x63)
    assert out[4] & 0x7F == 0  # very negative gate: zero, no NaN
    assert out[5] & 0x7F == 0x7F and out[6] & 0x7F == 0x7F  # NaN propagates
    bf = fp8lin.fp8lin_swiglu_2in_quant(g.to(gpu), u.to(gpu), out_dtype=fp8lin.DT_BF16).float().cpu().ravel()
    assert bf[3] == 45.0 and bf[0] == 0 and torch.isnan(bf[5])


def test_swiglu_rejects_non_contiguous(gpu):
    announce("swiglu non-contiguous")
    g = torch.zeros((64, 32), dtype=torch.bfloat16, device=gpu).t()
    with pytest.raises(ValueError):
        fp8lin.fp8lin_swiglu_2in_quant(g, g, 1.0)


# ---------------------------------------------------------------- fused gate/up + SwiGLU


@pytest.mark.parametrize(
    "m,k,inter",
    [(300, 528, 272), (256, 256, 128), (77, 64, 16), (513, 1040, 400), (8192, 4096, 16384),
     # 17 x 17 tiles of 3 K stages: workgroups change tiles at an odd K-stage count
     (4100, 384, 2064)],
)
def test_gate_up_swiglu_fused(gpu, m, k, inter):
    """One launch equals gemm_w8a8(gate), gemm_w8a8(up), swiglu_2in_quant bit for bit, and the oracle's
    SwiGLU codes of those bf16 outputs (midpoint cases aside)."""
    announce("gate_up_swiglu fused m=%d k=%d inter=%d" % (m, k, inter))
    case = config4(m=m, hidden=k, inter=inter, cal_rows=64)
    qg = fp8lin.fp8lin_quantize_static(case.w_gate.to(gpu), case.s_gate)
    qu = fp8lin.fp8lin_quantize_static(case.w_up.to(gpu), case.s_up)
    qx = fp8lin.fp8lin_quantize_static(case.x.to(gpu), case.input_scale)
    c0 = [fp8lin.fp8lin_launch_count(i) for i in range(5)]
    h = fp8lin.fp8lin_gate_up_swiglu_w8a8(qx, qg, qu, case.input_scale, case.s_gate, case.s_up, case.s_h)
    c1 = [fp8lin.fp8lin_launch_count(i) - c for i, c in enumerate(c0)]
    assert c1 == [0, 0, 0, 0, 1]  # one launch, no GEMM or SwiGLU kernel of its own
    g = fp8lin.fp8lin_gemm_w8a8(qx, qg, case.input_scale, case.s_gate)
    u = fp8lin.fp8lin_gemm_w8a8(qx, qu, case.input_scale, case.s_up)
    ref = fp8lin.fp8lin_swiglu_2in_quant(g, u, case.s_h, fp8lin.DT_E4M3)
    torch.cuda.synchronize()
    assert h.shape == (m, inter) and h.dtype == torch.uint8
    mism = int((h != ref).sum())
    assert mism == 0, "%d codes differ from the unfused path" % mism
    rows = sample_rows(m, 64, 21) if m > 1024 else np.arange(m)
    near = check_swiglu_codes(g.cpu()[rows], u.cpu()[rows], case.s_h, u8(h)[rows])
    print("codes at a rounding midpoint: %d" % near)


def test_gate_up_swiglu_writes_only_its_output(gpu):
    announce("gate_up_swiglu guard bytes")
    case = config4(m=40, hidden=128, inter=48, cal_rows=16)
    qg = fp8lin.fp8lin_quantize_static(case.w_gate.to(gpu), case.s_gate)
    qu = fp8lin.fp8lin_quantize_static(case.w_up.to(gpu), case.s_up)
    qx = fp8lin.fp8lin_quantize_static(case.x.to(gpu), case.input_scale)
    buf = torch.full((40 * 48 + 256,), 0xA5, dtype=torch.uint8, device=gpu)
    out = buf[: 40 * 48].view(40, 48)
    fp8lin.fp8lin_gate_up_swiglu_w8a8(qx, qg, qu, case.input_scale, case.s_gate, case.s_up, case.s_h, out=out)
    torch.cuda.synchronize()
    assert torch.all(buf[40 * 48:] == 0xA5)


@pytest.mark.parametrize("m,k,inter", [(300, 528, 272), (77, 64, 16), (513, 1040, 400), (8192, 4096, 16384)])
def test_gate_up_swiglu_fused_w8a16(gpu, m, k, inter):
    """16-bit step: one launch equals gemm_w8a16(gate), gemm_w8a16(up), swiglu_2in_quant(bf16) bit for bit,
    and is within the bf16 rounding of the oracle's SwiGLU of those outputs."""
    announce("gate_up_swiglu fused w8a16 m=%d k=%d inter=%d" % (m, k, inter))
    case = config4(m=m, hidden=k, inter=inter, cal_rows=64)
    qg = fp8lin.fp8lin_quantize_static(case.w_gate.to(gpu), case.s_gate)
    qu = fp8lin.fp8lin_quantize_static(case.w_up.to(gpu), case.s_up)
    x = case.x.to(gpu)
    c0 = [fp8lin.fp8lin_launch_count(i) for i in range(5)]
    h = fp8lin.fp8lin_gate_up_swiglu_w8a16(x, qg, qu, case.s_gate, case.s_up)
    c1 = [fp8lin.fp8lin_launch_count(i) - c for i, c in enumerate(c0)]
    assert c1 == [0, 0, 0, 0, 1]
    g = fp8lin.fp8lin_gemm_w8a16(x, qg, case.s_gate)
    u = fp8lin.fp8lin_gemm_w8a16(x, qu, case.s_up)
    ref = fp8lin.fp8lin_swiglu_2in_quant(g, u, 1.0, fp8lin.DT_BF16)
    torch.cuda.synchronize()
    assert h.shape == (m, inter) and h.dtype == torch.bfloat16
    mism = int((h.view(torch.int16) != ref.view(torch.int16)).sum())
    assert mism == 0, "%d values differ from the unfused path" % mism
    rows = sample_rows(m, 64, 23) if m > 1024 else np.arange(m)
    gr = f32(g.cpu()[rows]).astype(np.float64)
    ur = f32(u.cpu()[rows]).astype(np.float64)
    exact = swiglu.swiglu_2in(gr, ur)
    got = f32(h.cpu()[rows]).astype(np.float64)
    assert np.all(np.abs(got - exact) <= obf16.ulp(exact))


def test_gate_up_swiglu_w8a16_refuses_fp8_activation(gpu):
    qw = torch.zeros((16, 64), dtype=torch.uint8, device=gpu)
    with pytest.raises(fp8lin.Fp8LinError) as e:
        fp8lin.fp8lin_gate_up_swiglu_w8a16(torch.zeros((4, 64), dtype=torch.uint8, device=gpu), qw, qw, 1.0, 1.0)
    assert e.value.status == fp8lin.EDTYPE
