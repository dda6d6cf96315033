"""GPU parity: the activation-dtype variants.

* Two-input SwiGLU from binary16 gate/up ([TRT-17476] "What changed": the
  split SwiGLU runs on BF16 and FP16 shapes): E4M3 codes as for bf16 inputs
  (equal to the oracle's except next to a rounding midpoint), binary16
  output within one binary16 ulp of silu(g) u, overflowing to infinity.
* W8A16 with binary16 activations: within the float32-accumulation bound of
  the exact product (oracle.linear.gemm_w8a16_bound, K exact terms, one
  binary16 rounding); bit-exact on identity and scaled-permutation weights.
* W8A16 with float32 activations ([DF-14664] "Tests"): the three-piece split
  in the workspace equals x exactly, the product stays within the bound for
  3 K exact float32 terms, and identity / scaled-permutation weights give
  the exactly scaled activation, bit for bit.
* The fused gate/up + SwiGLU for binary16 activations equals the chain of
  the two binary16 GEMMs and the binary16 SwiGLU bit for bit.
"""

import numpy as np
import pytest
import torch

import w8a16_linear_layers_amd as fp8lin
from oracle import e4m3, f16, linear, swiglu
from tests.helpers import announce, sample_rows, u8
from workloads import max_calibrated_scale, normal_bf16, normal_f16, normal_f32

pytestmark = pytest.mark.gpu


def f64(t):
    return t.detach().double().cpu().numpy()


def check_codes(g, u, s_h, got):
    """E4M3 codes of silu(g) u / s_h: equal to the oracle's, or the other
    neighbour of a rounding midpoint within relative 2^-20."""
    ref, t = swiglu.swiglu_2in_quant(g, u, s_h)
    diff = got != ref
    if diff.any():
        near = swiglu.near_midpoint(t)
        assert not (diff & ~near).any(), "%d codes differ away from a midpoint" % np.count_nonzero(diff & ~near)
        step = (got[diff] & 0x7F).astype(int) - (ref[diff] & 0x7F).astype(int)
        assert np.all(np.abs(step) == 1)
    return int(diff.sum())


def weight(n, k, seed, gpu, std=0.02):
    """E4M3 weight quantized on the GPU and by the oracle (codes must agree)."""
    w = normal_bf16((n, k), std, seed)
    s_w = max_calibrated_scale(w)
    qw = fp8lin.fp8lin_quantize_static(w.to(gpu), s_w)
    qr = linear.quantize_static(w.float().numpy(), s_w)
    assert np.array_equal(u8(qw), qr)
    return qw, qr, s_w


def assert_within(y, ref, bound, what):
    ok = np.abs(y - ref) <= bound
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError("%s: %d of %d outside the bound; first at %s: gpu %r ref %r bound %r"
                             % (what, (~ok).sum(), ok.size, i, y[i], ref[i], bound[i]))


def one_code(v):
    """E4M3 code of a value that is exactly representable."""
    c = e4m3.encode(np.array([v], dtype=np.float64))[0]
    assert e4m3.decode(np.array([c], dtype=np.uint8))[0] == v
    return c


def scaled_permutation(n, seed):
    """qw [n, n] with one power of two per row at column perm[row]."""
    rng = np.random.default_rng(seed)
    perm = rng.permutation(n)
    exps = rng.integers(-4, 5, n)
    qw = np.zeros((n, n), dtype=np.uint8)
    for r in range(n):
        qw[r, perm[r]] = one_code(2.0 ** int(exps[r]))
    return qw, perm, exps


# ------------------------------------------------------------ SwiGLU fp16


@pytest.mark.parametrize("shape", [(1, 16), (37, 208), (1000, 1040)])
def test_swiglu_f16_to_e4m3(gpu, shape):
    announce("swiglu f16 -> e4m3 %s" % (shape,))
    g = normal_f16(shape, 0.45, 81)
    u = normal_f16(shape, 0.45, 82)
    s_h = 1.9 / 448
    c0 = fp8lin.fp8lin_launch_count(fp8lin.KERNEL_SWIGLU)
    out = fp8lin.fp8lin_swiglu_2in(g.to(gpu), u.to(gpu), s_h, fp8lin.DT_E4M3)
    assert fp8lin.fp8lin_launch_count(fp8lin.KERNEL_SWIGLU) - c0 == 1
    assert out.dtype == torch.uint8 and out.shape == shape
    n = check_codes(f64(g), f64(u), s_h, u8(out))
    print("near-midpoint differences: %d of %d" % (n, out.numel()))


def test_swiglu_f16_full_size_sampled(gpu):
    announce("swiglu f16 -> e4m3 full size")
    m, inter = 8192, 16384
    g = normal_f16((m, inter), 0.45, 83)
    u = normal_f16((m, inter), 0.45, 84)
    s_h = 2.1 / 448
    out = fp8lin.fp8lin_swiglu_2in(g.to(gpu), u.to(gpu), s_h, fp8lin.DT_E4M3)
    torch.cuda.synchronize()
    rows = sample_rows(m, 48, 4)
    n = check_codes(f64(g[rows]), f64(u[rows]), s_h, u8(out)[rows])
    print("near-midpoint differences: %d of %d" % (n, rows.size * inter))


def test_swiglu_f16_out(gpu):
    announce("swiglu f16 -> f16")
    g = normal_f16((300, 1040), 2.0, 85)
    u = normal_f16((300, 1040), 2.0, 86)
    g[0, :4] = torch.tensor([300.0, -300.0, 300.0, 65504.0], dtype=torch.float16)
    u[0, :4] = torch.tensor([300.0, 300.0, -300.0, 2.0], dtype=torch.float16)
    out = fp8lin.fp8lin_swiglu_2in(g.to(gpu), u.to(gpu), out_dtype=fp8lin.DT_F16)
    assert out.dtype == torch.float16
    h = swiglu.swiglu_2in(f64(g), f64(u))
    ref = f16.round_rne(h)
    got = f64(out)
    fin = np.isfinite(ref)
    assert np.all(np.abs(got[fin] - h[fin]) <= f16.ulp(h[fin]))
    assert np.array_equal(got[~fin], ref[~fin])  # overflow: same-signed infinity
    assert got[0, 0] == np.inf and got[0, 1] == 0.0 and got[0, 2] == -np.inf and got[0, 3] == np.inf


def test_swiglu_f16_special_values(gpu):
    announce("swiglu f16 special values")
    nan = float("nan")
    g = torch.tensor([0.0, 2.0, -3.0, 30.0, -90.0, 1.0, nan, 0.5] * 2, dtype=torch.float16).reshape(1, 16)
    u = torch.tensor([5.0, 0.0, 0.0, 1.5, 2.0, nan, 1.0, -0.25] * 2, dtype=torch.float16).reshape(1, 16)
    codes = u8(fp8lin.fp8lin_swiglu_2in(g.to(gpu), u.to(gpu), 1.0, fp8lin.DT_E4M3)).ravel()
    assert codes[0] & 0x7F == 0 and codes[1] & 0x7F == 0 and codes[2] & 0x7F == 0
    assert codes[3] == 0x63  # silu(30) * 1.5 just below 45 -> 44
    assert codes[4] & 0x7F == 0
    assert codes[5] & 0x7F == 0x7F and codes[6] & 0x7F == 0x7F
    h = fp8lin.fp8lin_swiglu_2in(g.to(gpu), u.to(gpu), out_dtype=fp8lin.DT_F16).double().cpu().ravel()
    assert h[0] == 0 and h[3] == 45.0 and torch.isnan(h[5]) and torch.isnan(h[6])


def test_swiglu_2in_bf16_equals_the_bf16_entry(gpu):
    announce("swiglu_2in bf16 == swiglu_2in_quant")
    g = normal_bf16((129, 1040), 0.45, 87).to(gpu)
    u = normal_bf16((129, 1040), 0.45, 88).to(gpu)
    for dt in (fp8lin.DT_E4M3, fp8lin.DT_BF16):
        a = fp8lin.fp8lin_swiglu_2in(g, u, 2.0 / 448, dt)
        b = fp8lin.fp8lin_swiglu_2in_quant(g, u, 2.0 / 448, dt)
        assert torch.equal(a, b)


# ------------------------------------------------------------ W8A16 fp16


@pytest.mark.parametrize("m,n,k", [(300, 264, 528), (1, 8, 16), (257, 520, 1040)])
def test_gemm_w8a16_f16(gpu, m, n, k):
    announce("gemm_w8a16 f16 m=%d n=%d k=%d" % (m, n, k))
    x = normal_f16((m, k), 0.35, 91)
    qw, qr, s_w = weight(n, k, 92, gpu)
    y = fp8lin.fp8lin_gemm_w8a16(x.to(gpu), qw, s_w)
    assert y.dtype == torch.float16 and y.shape == (m, n)
    ref = linear.gemm_w8a16(f64(x), qr, s_w)
    bound = linear.gemm_w8a16_bound(f64(x), qr, s_w, k, f16.ulp)
    assert_within(f64(y), ref, bound, "w8a16 f16")


def test_gemm_w8a16_f16_full_size_sampled(gpu):
    announce("gemm_w8a16 f16 16384x4096x4096")
    m, n, k = 16384, 4096, 4096
    x = normal_f16((m, k), 0.35, 93)
    qw, qr, s_w = weight(n, k, 94, gpu)
    y = fp8lin.fp8lin_gemm_w8a16(x.to(gpu), qw, s_w)
    torch.cuda.synchronize()
    rows = sample_rows(m, 96, 6)
    xr = f64(x[rows])
    assert_within(f64(y)[rows], linear.gemm_w8a16(xr, qr, s_w), linear.gemm_w8a16_bound(xr, qr, s_w, k, f16.ulp),
                  "w8a16 f16 full size")


def test_gemm_w8a16_f16_big_tiles_k_tail_sampled(gpu):
    """256 x 256 tiles (187 of them) with K not a whole number of 64-element stages: the form whose copies test
    each lane's chunk against K."""
    announce("gemm_w8a16 f16 2600x4104x528 (256x256 tiles, K tail)")
    m, n, k = 2600, 4104, 528
    x = normal_f16((m, k), 0.35, 97)
    qw, qr, s_w = weight(n, k, 98, gpu)
    y = fp8lin.fp8lin_gemm_w8a16(x.to(gpu), qw, s_w)
    torch.cuda.synchronize()
    rows = sample_rows(m, 96, 7)
    xr = f64(x[rows])
    assert_within(f64(y)[rows], linear.gemm_w8a16(xr, qr, s_w), linear.gemm_w8a16_bound(xr, qr, s_w, k, f16.ulp),
                  "w8a16 f16 K tail")


def test_gemm_w8a16_f16_exact_on_scaled_permutations(gpu):
    announce("gemm_w8a16 f16 permutation")
    n = 528
    x = normal_f16((300, n), 0.35, 95)
    qw, perm, exps = scaled_permutation(n, 96)
    y = f64(fp8lin.fp8lin_gemm_w8a16(x.to(gpu), torch.from_numpy(qw).to(gpu), 0.5))
    expect = f64(x)[:, perm] * np.ldexp(1.0, exps - 1)[None, :]
    assert np.array_equal(y, f16.round_rne(expect))  # one rounding, of the exact value


# ------------------------------------------------------------ W8A16 fp32


def split3_ref(x, kp):
    """Expected workspace rows: per 64-value block, hi / mid / lo bf16 bits
    (truncation split), padding zero. Integer bit manipulation only."""
    m, k = x.shape
    xb = np.zeros((m, kp), dtype=np.float32)
    xb[:, :k] = x
    bits = xb.view(np.uint32)
    hi = bits & 0xFFFF0000
    r = (xb - hi.view(np.float32)).astype(np.float32)
    mid = r.view(np.uint32) & 0xFFFF0000
    lo = (r - mid.view(np.float32)).astype(np.float32).view(np.uint32)
    out = np.zeros((m, kp // 64, 3, 64), dtype=np.uint16)
    for p, v in enumerate((hi, mid, lo)):
        out[:, :, p, :] = (v >> 16).astype(np.uint16).reshape(m, kp // 64, 64)
    return out.reshape(m, 3 * kp), hi.view(np.float32), mid.view(np.float32), lo.view(np.float32)


@pytest.mark.parametrize("m,n,k", [(300, 264, 528), (1, 8, 16), (257, 520, 1040), (64, 64, 80)])
def test_gemm_w8a16_f32(gpu, m, n, k):
    announce("gemm_w8a16 f32 m=%d n=%d k=%d" % (m, n, k))
    x = normal_f32((m, k), 0.35, 101)
    qw, qr, s_w = weight(n, k, 102, gpu)
    kp = (k + 63) // 64 * 64
    need = fp8lin.fp8lin_w8a16_f32_workspace_bytes(m, k)
    assert need == m * 3 * kp * 2
    ws = torch.full((need + 64,), 0xAB, dtype=torch.uint8, device=gpu)  # guard bytes past the end
    c0 = [fp8lin.fp8lin_launch_count(i) for i in (fp8lin.KERNEL_SPLIT, fp8lin.KERNEL_GEMM_W8A16)]
    y = fp8lin.fp8lin_gemm_w8a16_f32(x.to(gpu), qw, s_w, workspace=ws)
    c1 = [fp8lin.fp8lin_launch_count(i) for i in (fp8lin.KERNEL_SPLIT, fp8lin.KERNEL_GEMM_W8A16)]
    assert [b - a for a, b in zip(c0, c1)] == [1, 1]
    torch.cuda.synchronize()
    assert y.dtype == torch.float32 and y.shape == (m, n)
    # the workspace holds the exact three-piece split, padding zero
    exp_ws, hi, mid, lo = split3_ref(x.numpy(), kp)
    got_ws = ws[:need].cpu().numpy().view(np.uint16).reshape(m, 3 * kp)
    assert np.array_equal(got_ws, exp_ws)
    assert np.all(ws[need:].cpu().numpy() == 0xAB)
    assert np.array_equal(hi.astype(np.float64) + mid + lo, np.pad(x.numpy(), ((0, 0), (0, kp - k))).astype(np.float64))
    ref = linear.gemm_w8a16(x.numpy(), qr, s_w)
    bound = linear.gemm_w8a16_bound(x.numpy(), qr, s_w, 3 * k, linear.f32_ulp)
    assert_within(f64(y), ref, bound, "w8a16 f32")


def test_gemm_w8a16_f32_is_float32_accurate(gpu):
    """Far closer to the exact product than the bf16-activation path (which
    would pass the GEMM tolerance but not this)."""
    announce("gemm_w8a16 f32 accuracy")
    m, n, k = 256, 256, 1024
    x = normal_f32((m, k), 0.35, 103)
    qw, qr, s_w = weight(n, k, 104, gpu)
    ref = linear.gemm_w8a16(x.numpy(), qr, s_w)
    y32 = f64(fp8lin.fp8lin_gemm_w8a16_f32(x.to(gpu), qw, s_w))
    y16 = f64(fp8lin.fp8lin_gemm_w8a16(x.to(torch.bfloat16).to(gpu), qw, s_w))
    e32 = np.sqrt(np.mean((y32 - ref) ** 2))
    e16 = np.sqrt(np.mean((y16 - ref) ** 2))
    rms = np.sqrt(np.mean(ref ** 2))
    print("rms rel error: f32 %.3g, bf16 %.3g" % (e32 / rms, e16 / rms))
    assert e32 / rms < 2.0**-18 and e16 / rms > 2.0**-12


def test_gemm_w8a16_f32_exact_on_identity_and_permutations(gpu):
    announce("gemm_w8a16 f32 identity / permutation")
    n = 528
    rng = np.random.default_rng(105)
    # values over a wide range, all 24 significand bits in use; every piece
    # stays a normal bf16 (|x| >= 2^-60)
    x = (rng.uniform(1, 2, (77, n)) * np.ldexp(1.0, rng.integers(-60, 60, (77, n)))).astype(np.float32)
    x *= np.where(rng.random((77, n)) < 0.5, -1, 1).astype(np.float32)
    eye = np.where(np.eye(n, dtype=bool), np.uint8(0x38), np.uint8(0))
    y = fp8lin.fp8lin_gemm_w8a16_f32(torch.from_numpy(x).to(gpu), torch.from_numpy(eye).to(gpu), 1.0)
    assert np.array_equal(y.cpu().numpy().view(np.uint32), x.view(np.uint32))
    qw, perm, exps = scaled_permutation(n, 106)
    xs = (rng.normal(0, 0.35, (77, n))).astype(np.float32)
    y = fp8lin.fp8lin_gemm_w8a16_f32(torch.from_numpy(xs).to(gpu), torch.from_numpy(qw).to(gpu), 0.125)
    expect = xs.astype(np.float64)[:, perm] * np.ldexp(1.0, exps - 3)[None, :]
    assert np.array_equal(y.cpu().numpy().astype(np.float64), expect)


def test_gemm_w8a16_f32_non_finite(gpu):
    announce("gemm_w8a16 f32 non-finite")
    n = 64
    x = np.full((2, n), 0.5, dtype=np.float32)
    x[0, 5] = np.inf
    x[1, 9] = np.nan
    eye = np.where(np.eye(n, dtype=bool), np.uint8(0x38), np.uint8(0))
    y = fp8lin.fp8lin_gemm_w8a16_f32(torch.from_numpy(x).to(gpu), torch.from_numpy(eye).to(gpu), 1.0).cpu().numpy()
    # inf * 0 is NaN in every other column of row 0; a NaN spreads over row 1
    assert y[0, 5] == np.inf and np.isnan(np.delete(y[0], 5)).all()
    assert np.isnan(y[1]).all()


def test_gemm_w8a16_f32_full_size_sampled(gpu):
    announce("gemm_w8a16 f32 16384x4096x4096")
    m, n, k = 16384, 4096, 4096
    x = normal_f32((m, k), 0.35, 107)
    qw, qr, s_w = weight(n, k, 108, gpu)
    y = fp8lin.fp8lin_gemm_w8a16_f32(x.to(gpu), qw, s_w)
    torch.cuda.synchronize()
    rows = sample_rows(m, 64, 7)
    xr = x.numpy()[rows]
    assert_within(f64(y)[rows], linear.gemm_w8a16(xr, qr, s_w),
                  linear.gemm_w8a16_bound(xr, qr, s_w, 3 * k, linear.f32_ulp), "w8a16 f32 full size")


def test_gemm_w8a16_refuses_f32_without_workspace(gpu):
    announce("gemm_w8a16 f32 refused")
    x = torch.zeros((4, 64), dtype=torch.float32, device=gpu)
    qw = torch.zeros((64, 64), dtype=torch.uint8, device=gpu)
    with pytest.raises(fp8lin.Fp8LinError) as e:
        fp8lin.fp8lin_gemm_w8a16(x, qw, 1.0)
    assert e.value.status == fp8lin.EDTYPE


# ------------------------------------------------- fused gate/up + SwiGLU fp16


@pytest.mark.parametrize("m,k,inter", [(300, 528, 272), (77, 64, 16), (8192, 4096, 16384)])
def test_gate_up_swiglu_w8a16_f16_equals_chain(gpu, m, k, inter):
    announce("gate_up_swiglu w8a16 f16 m=%d k=%d i=%d" % (m, k, inter))
    x = normal_f16((m, k), 0.35, 111).to(gpu)
    qg, _, sg = weight(inter, k, 112, gpu)
    qu, _, su = weight(inter, k, 113, gpu)
    h = fp8lin.fp8lin_gate_up_swiglu_w8a16(x, qg, qu, sg, su)
    assert h.dtype == torch.float16 and h.shape == (m, inter)
    g = fp8lin.fp8lin_gemm_w8a16(x, qg, sg)
    u = fp8lin.fp8lin_gemm_w8a16(x, qu, su)
    chain = fp8lin.fp8lin_swiglu_2in(g, u, out_dtype=fp8lin.DT_F16)
    assert torch.equal(h, chain)
