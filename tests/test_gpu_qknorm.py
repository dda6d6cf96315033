"""GPU parity: per-head QK RMSNorm + rotate-half RoPE on contiguous Q / K.

Every output is within oracle.qknorm.qk_norm_rope_bound of the exact
(float64) value: the float32 error budget of the norm and the rotation plus
one bf16 rounding. In-place and out-of-place calls agree bit for bit, the
weight may be omitted, and the op runs on the grouped QKV projection's own
Q and K outputs (the consumer the pages describe).
"""

import numpy as np
import pytest
import torch

import w8a16_linear_layers_amd as fp8lin
from oracle import bf16, qknorm
from tests.helpers import announce, sample_rows
from workloads import config3, norm_weight_bf16, normal_bf16, rope_tables

pytestmark = pytest.mark.gpu

EPS = 1e-6


def f64(t):
    return t.detach().double().cpu().numpy()


def check(x, out, heads, w, c, s, what):
    wv = f64(w) if w is not None else np.ones(x.shape[1] // heads)
    xr, cr, sr = f64(x), c.numpy(), s.numpy()
    ref = qknorm.qk_norm_rope(xr, heads, wv, cr, sr, EPS)
    bound = qknorm.qk_norm_rope_bound(xr, heads, wv, cr, sr, EPS, bf16.ulp)
    got = f64(out)
    ok = np.abs(got - ref) <= bound
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError("%s: %d of %d outside the bound; first at %s: gpu %r ref %r bound %r"
                             % (what, (~ok).sum(), ok.size, i, got[i], ref[i], bound[i]))


@pytest.mark.parametrize("tokens,qh,kh,d", [(37, 3, 2, 128), (1, 1, 0, 128), (300, 4, 4, 64), (129, 32, 8, 128)])
def test_qk_norm_rope(gpu, tokens, qh, kh, d):
    announce("qk_norm_rope t=%d qh=%d kh=%d d=%d" % (tokens, qh, kh, d))
    q = normal_bf16((tokens, qh * d), 0.8, 201)
    k = normal_bf16((tokens, kh * d), 0.8, 202) if kh else None
    wq, wk = norm_weight_bf16(d, 203), norm_weight_bf16(d, 204)
    c, s = rope_tables(tokens, d, offset=5)
    c0 = fp8lin.fp8lin_launch_count(fp8lin.KERNEL_QK_NORM_ROPE)
    qo, ko = fp8lin.fp8lin_qk_norm_rope(q.to(gpu), k.to(gpu) if kh else None, wq.to(gpu), wk.to(gpu), c.to(gpu),
                                        s.to(gpu), d, EPS)
    assert fp8lin.fp8lin_launch_count(fp8lin.KERNEL_QK_NORM_ROPE) - c0 == 1
    check(q, qo, qh, wq, c, s, "q")
    if kh:
        check(k, ko, kh, wk, c, s, "k")
    else:
        assert ko is None


def test_in_place_and_unit_weight(gpu):
    announce("qk_norm_rope in place")
    t, h, d = 200, 8, 128
    q = normal_bf16((t, h * d), 0.5, 211).to(gpu)
    k = normal_bf16((t, h * d), 0.5, 212).to(gpu)
    ones = torch.ones(d, dtype=torch.bfloat16, device=gpu)
    c, s = (v.to(gpu) for v in rope_tables(t, d))
    qo, ko = fp8lin.fp8lin_qk_norm_rope(q, k, ones, ones, c, s, d, EPS)
    qn, kn = fp8lin.fp8lin_qk_norm_rope(q, k, None, None, c, s, d, EPS)  # no weight = unit weight
    assert torch.equal(qo, qn) and torch.equal(ko, kn)
    qi, ki = q.clone(), k.clone()
    fp8lin.fp8lin_qk_norm_rope(qi, ki, ones, ones, c, s, d, EPS, q_out=qi, k_out=ki)
    assert torch.equal(qi, qo) and torch.equal(ki, ko)


def test_special_values(gpu):
    announce("qk_norm_rope special values")
    d = 128
    q = normal_bf16((4, 2 * d), 0.5, 221)
    q[0, :d] = 0.0                       # a zero head stays zero
    q[1, 5] = float("nan")               # a NaN spreads over its head only
    q[2, d:] = 3.0                       # constant head: x / sqrt(x^2 + eps)
    c = torch.ones((4, d // 2), dtype=torch.float32)
    s = torch.zeros((4, d // 2), dtype=torch.float32)  # angle 0: the norm alone
    qo, _ = fp8lin.fp8lin_qk_norm_rope(q.to(gpu), None, None, None, c.to(gpu), s.to(gpu), d, EPS)
    out = f64(qo)
    assert np.all(out[0, :d] == 0)
    assert np.isnan(out[1, :d]).all() and not np.isnan(out[1, d:]).any()
    assert np.all(out[2, d:] == bf16.round_rne(np.array([3.0 / np.sqrt(9.0 + EPS)]))[0])
    fin = ~np.isnan(out)
    ref = qknorm.qk_norm_rope(f64(q), 2, np.ones(d), c.numpy(), s.numpy(), EPS)
    bound = qknorm.qk_norm_rope_bound(f64(q), 2, np.ones(d), c.numpy(), s.numpy(), EPS, bf16.ulp)
    assert np.all(np.abs(out - ref)[fin] <= bound[fin])


def test_full_size_sampled(gpu):
    """Q and K of the 16384-token QKV group: 32 heads of 128 each, one launch."""
    announce("qk_norm_rope 16384 x 32 x 128")
    t, h, d = 16384, 32, 128
    q = normal_bf16((t, h * d), 0.8, 231)
    k = normal_bf16((t, h * d), 0.8, 232)
    wq, wk = norm_weight_bf16(d, 233), norm_weight_bf16(d, 234)
    c, s = rope_tables(t, d)
    qo, ko = fp8lin.fp8lin_qk_norm_rope(q.to(gpu), k.to(gpu), wq.to(gpu), wk.to(gpu), c.to(gpu), s.to(gpu), d, EPS)
    torch.cuda.synchronize()
    rows = sample_rows(t, 64, 11)
    check(q[rows], qo[rows], h, wq, c[rows], s[rows], "q full size")
    check(k[rows], ko[rows], h, wk, c[rows], s[rows], "k full size")


def test_on_the_qkv_group_outputs(gpu):
    """The consumer on the grouped W8A8 projection's contiguous Q and K."""
    announce("qkv_shared -> qk_norm_rope")
    m, kdim, n, d = 600, 1024, 1024, 128
    case = config3(m=m, k=kdim, n=n)
    qws = [fp8lin.fp8lin_quantize_static(w.to(gpu), sw) for w, sw in zip(case.ws, case.weight_scales)]
    outs, _ = fp8lin.fp8lin_qkv_shared(case.x.to(gpu), qws, case.weight_scales, [case.input_scale] * 3,
                                       fp8lin.MODE_W8A8)
    assert outs[0].is_contiguous() and outs[1].is_contiguous()
    wq, wk = norm_weight_bf16(d, 241), norm_weight_bf16(d, 242)
    c, s = rope_tables(m, d)
    qo, ko = fp8lin.fp8lin_qk_norm_rope(outs[0], outs[1], wq.to(gpu), wk.to(gpu), c.to(gpu), s.to(gpu), d, EPS)
    check(outs[0], qo, n // d, wq, c, s, "q of the group")
    check(outs[1], ko, n // d, wk, c, s, "k of the group")


# ------------------------------------------- fused into the QKV GEMM epilogue


@pytest.mark.parametrize("m,kdim,n,nproj", [(600, 1024, 1024, 3), (300, 528, 384, 3), (77, 64, 128, 2),
                                            (16384, 4096, 4096, 3),
                                            # 816 tiles of 3 K stages: 3-4 tile changes per workgroup
                                            (4100, 384, 4096, 3)])
def test_fused_qkv_norm_rope(gpu, m, kdim, n, nproj):
    """Q and K normalized and rotated in the grouped GEMM's epilogue: within the bound of the exact
    norm + RoPE of the plain grouped GEMM's own bf16 outputs; V equal to the plain output bit for bit."""
    announce("qkv_w8a8_norm_rope m=%d k=%d n=%d nproj=%d" % (m, kdim, n, nproj))
    d = 128
    case = config3(m=m, k=kdim, n=n)
    qws = [fp8lin.fp8lin_quantize_static(w.to(gpu), sw) for w, sw in zip(case.ws, case.weight_scales)][:nproj]
    sws = case.weight_scales[:nproj]
    qx = fp8lin.fp8lin_quantize_static(case.x.to(gpu), case.input_scale)
    plain = fp8lin.fp8lin_gemm_w8a8_group(qx, qws, case.input_scale, sws)
    wq, wk = norm_weight_bf16(d, 251), norm_weight_bf16(d, 252)
    c, s = rope_tables(m, d, offset=3)
    c0 = [fp8lin.fp8lin_launch_count(i) for i in (fp8lin.KERNEL_GEMM_W8A8, fp8lin.KERNEL_QK_NORM_ROPE)]
    fused = fp8lin.fp8lin_qkv_w8a8_norm_rope(qx, qws, case.input_scale, sws, wq.to(gpu), wk.to(gpu), c.to(gpu),
                                             s.to(gpu), EPS)
    c1 = [fp8lin.fp8lin_launch_count(i) for i in (fp8lin.KERNEL_GEMM_W8A8, fp8lin.KERNEL_QK_NORM_ROPE)]
    assert [b - a for a, b in zip(c0, c1)] == [1, 0]
    torch.cuda.synchronize()
    if nproj == 3:
        assert torch.equal(fused[2], plain[2])
    rows = sample_rows(m, 64, 12) if m > 4096 else np.arange(m)
    check(plain[0][rows], fused[0][rows], n // d, wq, c[rows], s[rows], "fused q")
    check(plain[1][rows], fused[1][rows], n // d, wk, c[rows], s[rows], "fused k")


def test_fused_qkv_norm_rope_unit_weight_and_standalone_agree(gpu):
    """No weight = unit weight, and the fused and standalone forms differ by at most one bf16 ulp."""
    announce("qkv_w8a8_norm_rope vs qk_norm_rope")
    m, kdim, n, d = 513, 1024, 512, 128
    case = config3(m=m, k=kdim, n=n)
    qws = [fp8lin.fp8lin_quantize_static(w.to(gpu), sw) for w, sw in zip(case.ws, case.weight_scales)]
    qx = fp8lin.fp8lin_quantize_static(case.x.to(gpu), case.input_scale)
    c, s = (v.to(gpu) for v in rope_tables(m, d))
    ones = torch.ones(d, dtype=torch.bfloat16, device=gpu)
    a = fp8lin.fp8lin_qkv_w8a8_norm_rope(qx, qws, case.input_scale, case.weight_scales, ones, ones, c, s, EPS)
    b = fp8lin.fp8lin_qkv_w8a8_norm_rope(qx, qws, case.input_scale, case.weight_scales, None, None, c, s, EPS)
    assert all(torch.equal(x, y) for x, y in zip(a, b))
    plain = fp8lin.fp8lin_gemm_w8a8_group(qx, qws, case.input_scale, case.weight_scales)
    qs, ks = fp8lin.fp8lin_qk_norm_rope(plain[0], plain[1], ones, ones, c, s, d, EPS)
    for fused, sep in ((a[0], qs), (a[1], ks)):
        diff = np.abs(f64(fused) - f64(sep))
        assert np.all(diff <= bf16.ulp(np.abs(f64(sep))))
