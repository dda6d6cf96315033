"""GPU: fp8lin_gemm_w8a8_splitk_noalloc (the split-K W8A8 GEMM with its float32 partials in the library's
static scratch array) against fp8lin_gemm_w8a8_splitk (the same kernels with a caller workspace) and the
oracle, on two calls in a row, the second on a smaller input.

The two entry points run the same kernels over the same slices, so their outputs must agree bit for bit;
both must meet the GEMM tolerance against the exact product. The caller workspace is filled with a pattern
first and the scratch array still holds the first call's partials during the second call: neither may
leak into a result.
"""

import numpy as np
import pytest
import torch

import w8a16_linear_layers_amd as fp8lin
from oracle import linear
from tests.helpers import announce, assert_gemm_close, f32, sample_rows, u8
from workloads import max_calibrated_scale, normal_bf16

pytestmark = pytest.mark.gpu


def _case(m, n, k, seed):
    x = normal_bf16((m, k), 0.35, seed)
    w = normal_bf16((n, k), 0.02, seed + 1)
    return x, w, max_calibrated_scale(x), max_calibrated_scale(w)


def test_splitk_noalloc_matches_workspace_entry_twice(gpu):
    for (m, n, k, splits, seed) in ((1024, 4096, 4096, 2, 81), (300, 528, 1024, 4, 83)):
        announce("gemm_w8a8_splitk_noalloc m=%d n=%d k=%d splits=%d" % (m, n, k, splits))
        assert splits * m * n * 4 <= fp8lin.SCRATCH_BYTES
        x, w, s_in, s_w = _case(m, n, k, seed)
        qx = fp8lin.fp8lin_quantize_static(x.to(gpu), s_in)
        qw = fp8lin.fp8lin_quantize_static(w.to(gpu), s_w)
        y_na = torch.full((m, n), 3.0, dtype=torch.bfloat16, device=gpu)
        c0 = [fp8lin.fp8lin_launch_count(i) for i in (fp8lin.KERNEL_GEMM_W8A8, fp8lin.KERNEL_SPLITK_REDUCE)]
        fp8lin.fp8lin_gemm_w8a8_splitk_noalloc(qx, qw, s_in, s_w, splits=splits, out=y_na)
        c1 = [fp8lin.fp8lin_launch_count(i) for i in (fp8lin.KERNEL_GEMM_W8A8, fp8lin.KERNEL_SPLITK_REDUCE)]
        assert [b - a for a, b in zip(c0, c1)] == [1, 1]
        ws = torch.full((splits * m * n * 4,), 0x5A, dtype=torch.uint8, device=gpu)
        y_ws = fp8lin.fp8lin_gemm_w8a8_splitk(qx, qw, s_in, s_w, splits=splits, workspace=ws)
        torch.cuda.synchronize()
        assert torch.equal(y_na.view(torch.int16), y_ws.view(torch.int16)), "no-alloc and workspace entries differ"
        rows = sample_rows(m, 96, seed) if m > 512 else np.arange(m)
        qr = linear.quantize_static(f32(x)[rows], s_in)
        qwr = linear.quantize_static(f32(w), s_w)
        assert np.array_equal(u8(qx)[rows], qr) and np.array_equal(u8(qw), qwr)
        assert_gemm_close(f32(y_na)[rows], linear.gemm_w8a8(qr, qwr, s_in, s_w), "split-K no-alloc")
