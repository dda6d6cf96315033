"""The split-vs-fused re-quantization identity ([TRT-17476] "Description").

Split projections keep s_i * qW_i exactly; a fused loader that stores one
scale max(s) re-rounds the others to FP8-round(s_i qW_i / max s). The check
first asserts the scales genuinely differ (else fusion is lossless and the
test cannot discriminate), as the pages' own checkpoint test does.
"""

import numpy as np

from oracle import bf16, e4m3, linear
from workloads import QKV_RATIOS, config3


def small_group():
    case = config3(m=64, k=512, n=192)
    x = case.x.float().numpy()
    qws = [linear.quantize_static(w.float().numpy(), s) for w, s in zip(case.ws, case.weight_scales)]
    return case, x, qws


def test_scales_differ_and_keep_ratios():
    case, _, _ = small_group()
    s = case.weight_scales
    assert len(set(s)) == 3
    for r, si in zip(QKV_RATIOS, s):
        assert abs(si / s[0] - r) < 1e-6


def test_fused_requant_keeps_max_shard_and_rerounds_the_others():
    case, _, qws = small_group()
    s_max = max(case.weight_scales)
    changed = []
    for qw, s in zip(qws, case.weight_scales):
        fq = linear.fused_requant(qw, s, s_max)
        changed.append(np.mean(fq != qw))
        if s == s_max:
            assert np.array_equal(fq, qw)
    assert changed[1] > 0.2 and changed[2] > 0.2, changed


def test_separate_path_meets_tolerance_fused_path_does_not():
    case, x, qws = small_group()
    s_max = max(case.weight_scales)
    q = linear.quantize_static(x, case.input_scale)
    ratios = []
    for qw, s in zip(qws, case.weight_scales):
        y_ref = linear.gemm_w8a8(q, qw, case.input_scale, s)  # s_i * qW_i kept exactly
        y_sep = bf16.round_rne(y_ref)  # what a split projection returns (bf16 output)
        assert linear.within_gemm_tolerance(y_sep, y_ref).all()
        fq = linear.fused_requant(qw, s, s_max)
        y_fused = bf16.round_rne(linear.gemm_w8a8(q, fq, case.input_scale, s_max))
        ok = linear.within_gemm_tolerance(y_fused, y_ref)
        if s == s_max:
            assert ok.all()
        else:
            assert np.mean(ok) < 0.5, np.mean(ok)
            err_fused = np.sqrt(np.mean((y_fused - y_ref) ** 2))
            err_sep = np.sqrt(np.mean((y_sep - y_ref) ** 2))
            ratios.append(err_fused / err_sep)
    # analogue of the pages' "7-18x the numerical floor": context, loosely bounded
    assert all(r > 3 for r in ratios), ratios


def test_requant_of_equal_scale_is_identity_on_every_code():
    allc = np.arange(256, dtype=np.uint8)
    finite = allc[(allc & 0x7F) != 0x7F]
    assert np.array_equal(linear.fused_requant(finite, 0.37, 0.37), finite)
    assert np.array_equal(e4m3.encode(e4m3.decode(finite)), finite)
