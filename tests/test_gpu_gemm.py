"""GPU parity: fp8lin_gemm_w8a8 and fp8lin_gemm_w8a16 against the oracle.

Tolerance (elementwise): |y - y_ref| <= 2^-7 |y_ref| + 1e-3 rms(y_ref), with
y_ref the exact float64 result. Small cases are compared in full; the
full-size 4096 x 4096 projections on sampled rows (every column).
Weights are quantized on each side by its own quantizer from the same bf16
weights, and the codes are checked equal first.
"""

import numpy as np
import pytest
import torch

import w8a16_linear_layers_amd as fp8lin
from oracle import bf16 as obf16
from oracle import linear
from tests.helpers import announce, assert_gemm_close, f32, sample_rows, u8
from workloads import config1, config2, config3, max_calibrated_scale, normal_bf16, random_e4m3_codes

pytestmark = pytest.mark.gpu


def both_weights(w, s_w, gpu):
    """The weight's E4M3 codes on the GPU (library) and on the host (oracle)."""
    qw_gpu = fp8lin.fp8lin_quantize_static(w.to(gpu), s_w)
    qw_ref = linear.quantize_static(f32(w), s_w)
    assert np.array_equal(u8(qw_gpu), qw_ref)
    return qw_gpu, qw_ref


@pytest.mark.parametrize(
    "m,n,k",
    # K = 128, 256, 384, 512: exactly 1, 2, 3 and 4 K stages of 128 bytes (every stage kind of the pipeline)
    [(1, 8, 16), (7, 24, 48), (33, 40, 80), (64, 64, 64), (300, 520, 1040), (257, 264, 4096 + 16), (513, 1032, 272),
     (31, 48, 128), (200, 256, 256), (65, 136, 384), (129, 264, 512),
     # more tiles than compute units at 1 and 2 K stages: workgroups change tiles inside the last stage
     (4100, 4104, 128), (2100, 8200, 256),
     # the down projection's K = 16384 (128 stages), and with a K tail
     (300, 264, 16384), (513, 136, 16384 + 16),
     # 128 x 128 tiles (256 x 256 tiles would keep at most 60% of the CUs busy): 5 and 6 stages (the
     # stage loop runs in pairs), ragged M and N
     (77, 520, 640), (130, 136, 768)],
)
def test_w8a8_random_codes(gpu, m, n, k):
    announce("w8a8 random codes m=%d n=%d k=%d" % (m, n, k))
    q = random_e4m3_codes((m, k), 1000 + m)
    qw = random_e4m3_codes((n, k), 2000 + n)
    s_in, s_w = 1.7e-3, 3.1e-5
    y = fp8lin.fp8lin_gemm_w8a8(q.to(gpu), qw.to(gpu), s_in, s_w)
    torch.cuda.synchronize()
    assert_gemm_close(y, linear.gemm_w8a8(q.numpy(), qw.numpy(), s_in, s_w), "w8a8 %dx%dx%d" % (m, n, k))


@pytest.mark.parametrize("m,n,k", [(1, 8, 16), (33, 40, 80), (300, 520, 1040), (257, 264, 4096 + 16), (65, 136, 64),
                                   (129, 264, 128), (40, 256, 192), (4100, 4104, 64), (2100, 8200, 128),
                                   (300, 264, 16384), (129, 520, 16384 + 16),
                                   # 128 x 128 tiles: 4 and 5 stages of 64 K values
                                   (77, 520, 256), (130, 136, 320)])
def test_w8a16_random_codes(gpu, m, n, k):
    announce("w8a16 random codes m=%d n=%d k=%d" % (m, n, k))
    x = normal_bf16((m, k), 0.35, 3000 + m)
    qw = random_e4m3_codes((n, k), 4000 + n)
    s_w = 2.3e-4
    y = fp8lin.fp8lin_gemm_w8a16(x.to(gpu), qw.to(gpu), s_w)
    torch.cuda.synchronize()
    assert_gemm_close(y, linear.gemm_w8a16(f32(x), qw.numpy(), s_w), "w8a16 %dx%dx%d" % (m, n, k))


def _random_shape(seed):
    """A seeded GEMM shape: M from one of three ranges (up to one 256-row tile, up to ~4 of them, and 2600-5999
    rows with N of at least 2048, where 256 x 256 tiles fill the device), N a multiple of 8 up to 5592, K a
    multiple of 16 up to 4784, and an output row pitch up to 16 elements past N."""
    rng = np.random.default_rng(5000 + seed)
    lo, hi, nlo = [(1, 300, 1), (300, 1100, 1), (2600, 6000, 256)][seed % 3]
    m = int(rng.integers(lo, hi))
    n = 8 * int(rng.integers(nlo, 700))
    k = 16 * int(rng.integers(1, 300))
    pad = 8 * int(rng.integers(0, 3))
    return m, n, k, pad


@pytest.mark.parametrize("seed", range(24))
def test_random_shapes(gpu, seed):
    """Both GEMMs at seeded random shapes (every tile path, K-stage count and ragged edge the draws land
    on), against the oracle on every row of the smaller products and on sampled rows of the larger ones; the
    output's padding columns are left untouched."""
    m, n, k, pad = _random_shape(seed)
    announce("random shape m=%d n=%d k=%d ldy=%d" % (m, n, k, n + pad))
    q = random_e4m3_codes((m, k), 7000 + seed)
    qw = random_e4m3_codes((n, k), 7100 + seed)
    x = normal_bf16((m, k), 0.35, 7200 + seed)
    s_in, s_w, s_w16 = 1.7e-3, 3.1e-5, 2.3e-4
    qwg = qw.to(gpu)
    buf8 = torch.full((m, n + pad), 7.0, dtype=torch.bfloat16, device=gpu)
    buf16 = torch.full((m, n + pad), 7.0, dtype=torch.bfloat16, device=gpu)
    fp8lin.fp8lin_gemm_w8a8(q.to(gpu), qwg, s_in, s_w, out=buf8[:, :n])
    fp8lin.fp8lin_gemm_w8a16(x.to(gpu), qwg, s_w16, out=buf16[:, :n])
    torch.cuda.synchronize()
    if pad:
        assert torch.all(buf8[:, n:] == 7.0) and torch.all(buf16[:, n:] == 7.0)
    rows = np.arange(m) if m * n * k <= 4e8 else sample_rows(m, 64, seed)
    assert_gemm_close(f32(buf8[:, :n])[rows], linear.gemm_w8a8(q.numpy()[rows], qw.numpy(), s_in, s_w), "w8a8")
    assert_gemm_close(f32(buf16[:, :n])[rows], linear.gemm_w8a16(f32(x)[rows], qw.numpy(), s_w16), "w8a16")


def test_config1_both_modes(gpu):
    announce("config1 w8a8 + w8a16")
    case = config1()
    qw_gpu, qw_ref = both_weights(case.w, case.weight_scale, gpu)
    x = case.x.to(gpu)
    q = fp8lin.fp8lin_quantize_static(x, case.input_scale)
    y8 = fp8lin.fp8lin_gemm_w8a8(q, qw_gpu, case.input_scale, case.weight_scale)
    y16 = fp8lin.fp8lin_gemm_w8a16(x, qw_gpu, case.weight_scale)
    torch.cuda.synchronize()
    xr = f32(case.x)
    qr = linear.quantize_static(xr, case.input_scale)
    ref8 = linear.gemm_w8a8(qr, qw_ref, case.input_scale, case.weight_scale)
    ref16 = linear.gemm_w8a16(xr, qw_ref, case.weight_scale)
    assert_gemm_close(y8, ref8, "config1 w8a8")
    assert_gemm_close(y16, ref16, "config1 w8a16")
    # the two paths differ, and 16-bit activations land closer to the unquantized product
    unq = xr.astype(np.float64) @ f32(case.w).astype(np.float64).T
    e8 = np.sqrt(np.mean((f32(y8) - unq) ** 2))
    e16 = np.sqrt(np.mean((f32(y16) - unq) ** 2))
    assert not torch.equal(y8, y16)
    assert e16 < e8


@pytest.mark.parametrize("m", [1024, 8192])
def test_config2_projection(gpu, m):
    announce("config2 m=%d" % m)
    case = config2(m)
    qw_gpu, qw_ref = both_weights(case.w, case.weight_scale, gpu)
    x = case.x.to(gpu)
    q = fp8lin.fp8lin_quantize_static(x, case.input_scale)
    y8 = fp8lin.fp8lin_gemm_w8a8(q, qw_gpu, case.input_scale, case.weight_scale)
    y16 = fp8lin.fp8lin_gemm_w8a16(x, qw_gpu, case.weight_scale)
    torch.cuda.synchronize()
    rows = sample_rows(m, 192, m)
    xr = f32(case.x[rows])
    qr = linear.quantize_static(xr, case.input_scale)
    assert np.array_equal(u8(q[torch.from_numpy(rows).to(gpu)]), qr)
    assert_gemm_close(f32(y8)[rows], linear.gemm_w8a8(qr, qw_ref, case.input_scale, case.weight_scale), "w8a8")
    assert_gemm_close(f32(y16)[rows], linear.gemm_w8a16(xr, qw_ref, case.weight_scale), "w8a16")


def test_headline_shape_sampled(gpu):
    """M=16384, K=N=4096: the Q projection of the shared-QKV workload."""
    announce("headline 16384x4096x4096")
    case = config3()
    qw_gpu, qw_ref = both_weights(case.ws[0], case.weight_scales[0], gpu)
    x = case.x.to(gpu)
    q = fp8lin.fp8lin_quantize_static(x, case.input_scale)
    y8 = fp8lin.fp8lin_gemm_w8a8(q, qw_gpu, case.input_scale, case.weight_scales[0])
    y16 = fp8lin.fp8lin_gemm_w8a16(x, qw_gpu, case.weight_scales[0])
    torch.cuda.synchronize()
    rows = sample_rows(16384, 160, 77)
    xr = f32(case.x[rows])
    qr = linear.quantize_static(xr, case.input_scale)
    assert_gemm_close(f32(y8)[rows], linear.gemm_w8a8(qr, qw_ref, case.input_scale, case.weight_scales[0]), "w8a8")
    assert_gemm_close(f32(y16)[rows], linear.gemm_w8a16(xr, qw_ref, case.weight_scales[0]), "w8a16")


@pytest.mark.parametrize(
    "m,n,k",
    # 256 x 256 tiles (enough of them to fill the device), ragged M and N, 1-4 stages and a K tail
    [(4100, 4104, 4096 + 16), (3100, 3080, 384), (3100, 3080, 512)],
)
def test_big_tiles_ragged_sampled(gpu, m, n, k):
    """The 256 x 256 kernels on shapes with ragged edges and every K-stage kind, on sampled rows (the last
    M-tile's rows included)."""
    announce("big tiles m=%d n=%d k=%d" % (m, n, k))
    q = random_e4m3_codes((m, k), 5000 + m)
    qw = random_e4m3_codes((n, k), 6000 + n)
    x = normal_bf16((m, k), 0.35, 7000 + m)
    y8 = fp8lin.fp8lin_gemm_w8a8(q.to(gpu), qw.to(gpu), 1.7e-3, 3.1e-5)
    y16 = fp8lin.fp8lin_gemm_w8a16(x.to(gpu), qw.to(gpu), 2.3e-4)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([sample_rows(m, 48, m), np.arange(m - 8, m)]))
    assert_gemm_close(f32(y8)[rows], linear.gemm_w8a8(q.numpy()[rows], qw.numpy(), 1.7e-3, 3.1e-5), "w8a8")
    assert_gemm_close(f32(y16)[rows], linear.gemm_w8a16(f32(x)[rows], qw.numpy(), 2.3e-4), "w8a16")


@pytest.mark.parametrize("k", [384, 640, 4096 + 16])
def test_w8a8_tile_changes_odd_stage_counts(gpu, k):
    """Workgroups that walk 2-3 tiles of an odd number of K stages (3, 5, 33; 33 x 17 = 561 tiles of 256 x 256
    for 256 compute units): a tile starts on the LDS buffer the previous tile's last stage left, so the buffer
    parity alternates from tile to tile, and stage KT - 2 already copies the next tile's stage 0. Rows from
    every M-tile (each row crosses all 17 N-tiles) against the oracle, and a second launch bit-identical."""
    m, n = 8200, 4104
    announce("w8a8 tile changes m=%d n=%d k=%d" % (m, n, k))
    q = random_e4m3_codes((m, k), 8000 + k)
    qw = random_e4m3_codes((n, k), 9000 + k)
    qg, qwg = q.to(gpu), qw.to(gpu)
    y = fp8lin.fp8lin_gemm_w8a8(qg, qwg, 1.7e-3, 3.1e-5)
    y2 = fp8lin.fp8lin_gemm_w8a8(qg, qwg, 1.7e-3, 3.1e-5)
    torch.cuda.synchronize()
    assert torch.equal(y, y2)
    rows = np.unique(np.concatenate([sample_rows(m, 64, k), np.arange(k % 256, m, 256), [m - 1]]))
    assert_gemm_close(f32(y)[rows], linear.gemm_w8a8(q.numpy()[rows], qw.numpy(), 1.7e-3, 3.1e-5), "w8a8")


@pytest.mark.parametrize("m", [1024, 2048])
def test_small_tiles_full_rows_sampled(gpu, m):
    """128 x 128 tiles at the small-batch sizes: one tile per CU (1024 rows), several per CU (2048), and the
    shared-QKV group at 1024 rows (three projections in one launch), on sampled rows."""
    announce("small tiles m=%d" % m)
    case = config2(8192)
    x = case.x[:m].contiguous()
    qw_gpu, qw_ref = both_weights(case.w, case.weight_scale, gpu)
    xg = x.to(gpu)
    q = fp8lin.fp8lin_quantize_static(xg, case.input_scale)
    y8 = fp8lin.fp8lin_gemm_w8a8(q, qw_gpu, case.input_scale, case.weight_scale)
    y16 = fp8lin.fp8lin_gemm_w8a16(xg, qw_gpu, case.weight_scale)
    outs, _ = fp8lin.fp8lin_qkv_shared(xg, [qw_gpu] * 3, [case.weight_scale] * 3, [case.input_scale] * 3,
                                       fp8lin.MODE_W8A8)
    torch.cuda.synchronize()
    rows = sample_rows(m, 96, m + 1)
    xr = f32(x[rows])
    qr = linear.quantize_static(xr, case.input_scale)
    ref8 = linear.gemm_w8a8(qr, qw_ref, case.input_scale, case.weight_scale)
    assert_gemm_close(f32(y8)[rows], ref8, "w8a8")
    assert_gemm_close(f32(y16)[rows], linear.gemm_w8a16(xr, qw_ref, case.weight_scale), "w8a16")
    for o in outs:
        assert torch.equal(o, y8)  # the same projection three times in one grouped launch
    # Rows are independent: the first m rows of the 8192-row product (256 x 256 tiles) are the same
    # numbers, K summed in the same order per element.
    xb = case.x.to(gpu)
    qb = fp8lin.fp8lin_quantize_static(xb, case.input_scale)
    assert torch.equal(qb[:m], q)
    big8 = fp8lin.fp8lin_gemm_w8a8(qb, qw_gpu, case.input_scale, case.weight_scale)
    big16 = fp8lin.fp8lin_gemm_w8a16(xb, qw_gpu, case.weight_scale)
    torch.cuda.synchronize()
    assert torch.equal(big8[:m], y8), "128x128 and 256x256 W8A8 tiles differ"
    assert torch.equal(big16[:m].view(torch.int16), y16.view(torch.int16)), "128x128 and 256x256 W8A16 tiles differ"


def test_w8a16_identity_weight_is_exact(gpu):
    announce("w8a16 identity weight")
    k = 512
    x = normal_bf16((300, k), 0.35, 9)
    ident = torch.where(torch.eye(k, dtype=torch.bool), 0x38, 0x00).to(torch.uint8)
    y = fp8lin.fp8lin_gemm_w8a16(x.to(gpu), ident.to(gpu), 1.0)
    assert torch.equal(y.cpu(), x)


def test_w8a8_identity_weight(gpu):
    announce("w8a8 identity weight")
    k = 256
    q = random_e4m3_codes((130, k), 21)
    ident = torch.where(torch.eye(k, dtype=torch.bool), 0x38, 0x00).to(torch.uint8)
    s_in = 0.01
    y = fp8lin.fp8lin_gemm_w8a8(q.to(gpu), ident.to(gpu), s_in, 1.0)
    ref = linear.gemm_w8a8(q.numpy(), ident.numpy(), s_in, 1.0)
    assert_gemm_close(y, ref, "identity")


def test_output_stride_and_guard(gpu):
    """ldy > N: only columns [0, N) of each row are written."""
    announce("w8a8 ldy > n")
    m, n, k, ldy = 70, 136, 128, 200
    q = random_e4m3_codes((m, k), 31).to(gpu)
    qw = random_e4m3_codes((n, k), 32).to(gpu)
    buf = torch.full((m, ldy), 7.0, dtype=torch.bfloat16, device=gpu)
    fp8lin.fp8lin_gemm_w8a8(q, qw, 0.01, 0.02, out=buf, ldy=ldy)
    fp8lin.fp8lin_gemm_w8a16(torch.zeros((m, k), dtype=torch.bfloat16, device=gpu), qw, 0.02, out=buf[:, 8:], ldy=ldy)
    torch.cuda.synchronize()
    assert torch.all(buf[:, n + 8 :] == 7.0)
    assert torch.all(buf[:, 8 : n + 8] == 0)
    ref = linear.gemm_w8a8(u8(q), u8(qw), 0.01, 0.02)
    assert_gemm_close(f32(buf[:, :8]), ref[:, :8], "ldy columns")


def test_rank3_activation_and_empty(gpu):
    announce("w8a8 rank-3 input and M=0")
    q = random_e4m3_codes((2, 3, 64), 41).to(gpu)
    qw = random_e4m3_codes((16, 64), 42).to(gpu)
    y = fp8lin.fp8lin_gemm_w8a8(q, qw, 0.5, 0.25)
    assert y.shape == (2, 3, 16)
    ref = linear.gemm_w8a8(u8(q).reshape(6, 64), u8(qw), 0.5, 0.25)
    assert_gemm_close(f32(y).reshape(6, 16), ref, "rank3")
    empty = fp8lin.fp8lin_gemm_w8a8(q[:0], qw, 0.5, 0.25)
    assert empty.shape == (0, 3, 16)


def test_w8a16_refuses_fp8_activation(gpu):
    announce("w8a16 refuses fp8")
    q = torch.zeros((4, 64), dtype=torch.uint8, device=gpu)
    qw = torch.zeros((16, 64), dtype=torch.uint8, device=gpu)
    with pytest.raises(fp8lin.Fp8LinError) as e:
        fp8lin.fp8lin_gemm_w8a16(q, qw, 1.0)
    assert e.value.status == fp8lin.EDTYPE


@pytest.mark.parametrize("kind", ["w8a8", "w8a16", "gate_up_w8a8", "gate_up_w8a16", "w8a8_small", "w8a16_small"])
def test_repeated_launches_are_bit_identical(gpu, kind):
    """Several tiles per workgroup (persistent kernels): every launch gives the same bits. A wave that
    reuses LDS another wave still reads (tile changes, staging areas) would show up as run-to-run
    differences. The small kinds run 2048 rows: 128 x 128 tiles, two per workgroup."""
    announce("repeatability %s" % kind)
    m, k, n = (2048 if kind.endswith("small") else 8192), 4096, 4096
    kind = kind.replace("_small", "")
    x = normal_bf16((m, k), 0.35, 61).to(gpu)
    qw = random_e4m3_codes((n, k), 62).to(gpu)
    qw2 = random_e4m3_codes((n, k), 63).to(gpu)
    qx = fp8lin.fp8lin_quantize_static(x, 0.35 * 4 / 448)
    if kind == "w8a8":
        run = lambda: fp8lin.fp8lin_gemm_w8a8(qx, qw, 0.35 * 4 / 448, 1e-3)  # noqa: E731
    elif kind == "w8a16":
        run = lambda: fp8lin.fp8lin_gemm_w8a16(x, qw, 1e-3)  # noqa: E731
    elif kind == "gate_up_w8a8":
        run = lambda: fp8lin.fp8lin_gate_up_swiglu_w8a8(qx, qw, qw2, 0.35 * 4 / 448, 1e-3, 1e-3, 0.05)  # noqa: E731
    else:
        run = lambda: fp8lin.fp8lin_gate_up_swiglu_w8a16(x, qw, qw2, 1e-3, 1e-3)  # noqa: E731
    first = run()
    for _ in range(4):
        again = run()
        torch.cuda.synchronize()
        assert torch.equal(first.view(torch.uint8), again.view(torch.uint8))


# ---------------------------------------------------------------- split-K


@pytest.mark.parametrize("m,n,k,splits", [(1024, 4096, 4096, 4), (1024, 4096, 4096, 2), (300, 528, 1024, 4),
                                          (77, 64, 128, 2),
                                          # 306 tiles of 3-stage slices: workgroups change tiles at an odd K count
                                          (2100, 4104, 768, 2)])
def test_gemm_w8a8_splitk(gpu, m, n, k, splits):
    """K split into float32 partials, summed in slice order: the oracle's tolerance, within one bf16 ulp of
    the unsplit GEMM, and nothing written past the partials."""
    announce("gemm_w8a8_splitk m=%d n=%d k=%d splits=%d" % (m, n, k, splits))
    x = normal_bf16((m, k), 0.35, 61)
    w = normal_bf16((n, k), 0.02, 62)
    s_in, s_w = max_calibrated_scale(x), max_calibrated_scale(w)
    qx = fp8lin.fp8lin_quantize_static(x.to(gpu), s_in)
    qw = fp8lin.fp8lin_quantize_static(w.to(gpu), s_w)
    need = splits * m * n * 4
    ws = torch.full((need + 256,), 0x5A, dtype=torch.uint8, device=gpu)
    c0 = [fp8lin.fp8lin_launch_count(i) for i in (fp8lin.KERNEL_GEMM_W8A8, fp8lin.KERNEL_SPLITK_REDUCE)]
    y = fp8lin.fp8lin_gemm_w8a8_splitk(qx, qw, s_in, s_w, splits=splits, workspace=ws)
    c1 = [fp8lin.fp8lin_launch_count(i) for i in (fp8lin.KERNEL_GEMM_W8A8, fp8lin.KERNEL_SPLITK_REDUCE)]
    assert [b - a for a, b in zip(c0, c1)] == [1, 1]
    y_plain = fp8lin.fp8lin_gemm_w8a8(qx, qw, s_in, s_w)
    torch.cuda.synchronize()
    assert torch.all(ws[need:] == 0x5A)
    rows = sample_rows(m, 96, 21) if m > 512 else np.arange(m)
    qr = linear.quantize_static(f32(x)[rows], s_in)
    qwr = linear.quantize_static(f32(w), s_w)
    assert np.array_equal(u8(qx)[rows], qr)
    ref = linear.gemm_w8a8(qr, qwr, s_in, s_w)
    assert_gemm_close(f32(y)[rows], ref, "split-K")
    a, b = f32(y).astype(np.float64), f32(y_plain).astype(np.float64)
    assert np.all(np.abs(a - b) <= obf16.ulp(np.maximum(np.abs(a), np.abs(b))))


@pytest.mark.parametrize("m,n,k,splits", [(1024, 4096, 4096, 2), (1024, 4096, 4096, 4), (300, 528, 1024, 4),
                                          (77, 64, 128, 2), (77, 64, 160, 2)])
def test_gemm_w8a16_splitk(gpu, m, n, k, splits):
    """W8A16 with K split into float32 partials, summed in slice order: the oracle's tolerance, both the split
    and the unsplit GEMM within the float32-summation bound of the exact product (their summation orders
    differ, and bf16 x E4M3 products carry more bits than one bf16 ulp can absorb under cancellation), and
    nothing written past the partials."""
    announce("gemm_w8a16_splitk m=%d n=%d k=%d splits=%d" % (m, n, k, splits))
    x = normal_bf16((m, k), 0.35, 63)
    w = normal_bf16((n, k), 0.02, 64)
    s_w = max_calibrated_scale(w)
    qw = fp8lin.fp8lin_quantize_static(w.to(gpu), s_w)
    xg = x.to(gpu)
    need = splits * m * n * 4
    ws = torch.full((need + 256,), 0x5A, dtype=torch.uint8, device=gpu)
    c0 = [fp8lin.fp8lin_launch_count(i) for i in (fp8lin.KERNEL_GEMM_W8A16, fp8lin.KERNEL_SPLITK_REDUCE)]
    y = fp8lin.fp8lin_gemm_w8a16_splitk(xg, qw, s_w, splits=splits, workspace=ws)
    c1 = [fp8lin.fp8lin_launch_count(i) for i in (fp8lin.KERNEL_GEMM_W8A16, fp8lin.KERNEL_SPLITK_REDUCE)]
    assert [b - a for a, b in zip(c0, c1)] == [1, 1]
    y_plain = fp8lin.fp8lin_gemm_w8a16(xg, qw, s_w)
    torch.cuda.synchronize()
    assert torch.all(ws[need:] == 0x5A)
    rows = sample_rows(m, 96, 23) if m > 512 else np.arange(m)
    qwr = linear.quantize_static(f32(w), s_w)
    assert np.array_equal(u8(qw), qwr)
    ref = linear.gemm_w8a16(f32(x)[rows], qwr, s_w)
    assert_gemm_close(f32(y)[rows], ref, "W8A16 split-K")
    bound = linear.gemm_w8a16_bound(f32(x)[rows].astype(np.float64), qwr, s_w, k, obf16.ulp)
    for got, what in ((y, "split"), (y_plain, "unsplit")):
        err = np.abs(f32(got)[rows].astype(np.float64) - ref)
        assert np.all(err <= bound), "%s: %d elements outside the float32 bound" % (what, int((err > bound).sum()))


def test_gemm_splitk_choice():
    """No split where the unsplit call runs on 128 x 128 tiles (which beat the splits) or fills the device."""
    for choice in (fp8lin.fp8lin_gemm_w8a8_splitk_choice, fp8lin.fp8lin_gemm_w8a16_splitk_choice):
        assert choice(16384, 4096, 4096) == 1
        assert choice(1024, 4096, 4096) == 1
        assert choice(128, 512, 512) == 1
