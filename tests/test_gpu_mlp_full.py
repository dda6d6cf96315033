"""GPU parity of the split gated MLP at its full size, element by element against the oracle.

The chain of [TRT-17476] "What changed" (gate and up on one shared quantization of x, the two-input
SwiGLU emitting FP8 for the down projection) and its 16-bit form of "Denoising-step activation
precision" (every stage on the 16-bit activation, the FP8 weights kept), at x [8192, 4096], gate/up
4096 -> 16384 and down 16384 -> 4096 (K = 16384, 128 K stages of the W8A8 kernel).

Each stage is compared on sampled rows (every column) with the oracle applied to inputs that the test
has already validated: the gate/up outputs must lie within the GEMM tolerance of the exact products,
the SwiGLU output of those bf16 values must match the oracle's codes (both neighbours of an E4M3
rounding midpoint are correct) or lie within one bf16 ulp of the exact product, and the down
projection of those validated values must lie within the GEMM tolerance of its exact product. Rows
are independent, so a row subset of every stage is exact for those rows.
"""

import numpy as np
import pytest
import torch

import w8a16_linear_layers_amd as fp8lin
from oracle import bf16 as obf16
from oracle import linear, swiglu
from tests.helpers import announce, assert_gemm_close, f32, sample_rows, u8
from workloads import config4

pytestmark = pytest.mark.gpu

M, HIDDEN, INTER = 8192, 4096, 16384


@pytest.fixture(scope="module")
def mlp(gpu):
    announce("split gated MLP 8192x4096->16384->4096: weights and oracle codes")
    case = config4(m=M, hidden=HIDDEN, inter=INTER, device=gpu)
    qw_gpu, qw_ref = [], []
    for w, s in ((case.w_gate, case.s_gate), (case.w_up, case.s_up), (case.w_down, case.s_down)):
        g = fp8lin.fp8lin_quantize_static(w.to(gpu), s)
        r = linear.quantize_static(f32(w), s)
        assert np.array_equal(u8(g), r), "weight codes differ from the oracle's"
        qw_gpu.append(g)
        qw_ref.append(r)
    rows = sample_rows(M, 64, 4)
    return case, qw_gpu, qw_ref, rows


def _rows_of(t, rows):
    return t[torch.from_numpy(rows).to(t.device)]


def test_gated_mlp_w8a8_full_size(gpu, mlp):
    case, (qg, qu, qd), (qg_r, qu_r, qd_r), rows = mlp
    announce("gated MLP W8A8: gate/up 8192x4096->16384 (nproj = 2), SwiGLU E4M3, down K = 16384")
    x = case.x.to(gpu)
    (g, u), qx = fp8lin.fp8lin_qkv_shared(x, [qg, qu], [case.s_gate, case.s_up], [case.input_scale] * 2,
                                          fp8lin.MODE_W8A8)
    h = fp8lin.fp8lin_swiglu_2in_quant(g, u, case.s_h)
    y = fp8lin.fp8lin_gemm_w8a8(h, qd, case.s_h, case.s_down)
    torch.cuda.synchronize()
    assert g.shape == u.shape == (M, INTER) and h.shape == (M, INTER) and y.shape == (M, HIDDEN)

    qx_r = linear.quantize_static(f32(case.x[rows]), case.input_scale)
    assert np.array_equal(u8(_rows_of(qx, rows)), qx_r)
    g_s, u_s = f32(_rows_of(g, rows)).astype(np.float64), f32(_rows_of(u, rows)).astype(np.float64)
    assert_gemm_close(g_s, linear.gemm_w8a8(qx_r, qg_r, case.input_scale, case.s_gate), "gate 8192x4096->16384")
    assert_gemm_close(u_s, linear.gemm_w8a8(qx_r, qu_r, case.input_scale, case.s_up), "up 8192x4096->16384")

    # SwiGLU of the validated bf16 g and u: the oracle's codes, or the other neighbour of a midpoint
    h_s = u8(_rows_of(h, rows))
    ref_codes, t = swiglu.swiglu_2in_quant(g_s, u_s, case.s_h)
    diff = h_s != ref_codes
    assert not (diff & ~swiglu.near_midpoint(t)).any(), "SwiGLU codes differ away from a rounding midpoint"
    assert np.all(np.abs((h_s[diff] & 0x7F).astype(int) - (ref_codes[diff] & 0x7F).astype(int)) == 1)
    print("SwiGLU codes at a rounding midpoint: %d of %d" % (int(diff.sum()), diff.size))

    # down projection, K = 16384, on the validated codes
    assert_gemm_close(_rows_of(y, rows), linear.gemm_w8a8(h_s, qd_r, case.s_h, case.s_down),
                      "down 8192x16384->4096 W8A8")


def test_gated_mlp_w8a16_full_size(gpu, mlp):
    case, (qg, qu, qd), (qg_r, qu_r, qd_r), rows = mlp
    announce("gated MLP W8A16: gate/up 8192x4096->16384 (nproj = 2), SwiGLU bf16, down K = 16384")
    x = case.x.to(gpu)
    c0 = fp8lin.fp8lin_launch_count(fp8lin.KERNEL_QUANTIZE)
    (g, u), _ = fp8lin.fp8lin_qkv_shared(x, [qg, qu], [case.s_gate, case.s_up], [case.input_scale] * 2,
                                         fp8lin.MODE_W8A16)
    assert fp8lin.fp8lin_launch_count(fp8lin.KERNEL_QUANTIZE) == c0  # no activation quantization on 16-bit steps
    h = fp8lin.fp8lin_swiglu_2in_quant(g, u, out_dtype=fp8lin.DT_BF16)
    y = fp8lin.fp8lin_gemm_w8a16(h, qd, case.s_down)
    torch.cuda.synchronize()
    assert h.dtype == torch.bfloat16 and y.shape == (M, HIDDEN)

    xr = f32(case.x[rows])
    g_s, u_s = f32(_rows_of(g, rows)).astype(np.float64), f32(_rows_of(u, rows)).astype(np.float64)
    assert_gemm_close(g_s, linear.gemm_w8a16(xr, qg_r, case.s_gate), "gate 8192x4096->16384 W8A16")
    assert_gemm_close(u_s, linear.gemm_w8a16(xr, qu_r, case.s_up), "up 8192x4096->16384 W8A16")

    h_s = f32(_rows_of(h, rows)).astype(np.float64)
    exact = swiglu.swiglu_2in(g_s, u_s)
    assert np.all(np.abs(h_s - exact) <= obf16.ulp(exact)), "bf16 SwiGLU beyond one ulp of the exact product"

    assert_gemm_close(_rows_of(y, rows), linear.gemm_w8a16(h_s, qd_r, case.s_down), "down 8192x16384->4096 W8A16")
