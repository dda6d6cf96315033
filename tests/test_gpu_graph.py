"""GPU: the entry points are safe under HIP graph capture.

The header promises that no call allocates, synchronizes or reads device
memory from the host, so a whole step can be captured once and replayed.
The captured step (static quantization, the grouped QKV GEMM, the QK norm +
RoPE consumer, the fused gate/up + SwiGLU, the dynamic quantization with its
device-scale GEMM) is replayed several times, with eager work and
synchronizations in between, and every replay must equal the eager step bit
for bit.
"""

import pytest
import torch

import w8a16_linear_layers_amd as fp8lin
from tests.helpers import announce
from workloads import config3, config4, norm_weight_bf16, rope_tables

pytestmark = pytest.mark.gpu


def test_captured_step_replays_bit_exactly(gpu):
    announce("hip graph capture of a step")
    m, k, n, inter, d = 512, 1024, 1024, 2048, 128
    case = config3(m=m, k=k, n=n)
    mlp = config4(m=m, hidden=k, inter=inter, cal_rows=64)
    x = case.x.to(gpu)
    qws = [fp8lin.fp8lin_quantize_static(w.to(gpu), s) for w, s in zip(case.ws, case.weight_scales)]
    qg = fp8lin.fp8lin_quantize_static(mlp.w_gate.to(gpu), mlp.s_gate)
    qu = fp8lin.fp8lin_quantize_static(mlp.w_up.to(gpu), mlp.s_up)
    wq, wk = norm_weight_bf16(d, 301).to(gpu), norm_weight_bf16(d, 302).to(gpu)
    c, s = (v.to(gpu) for v in rope_tables(m, d))
    s_in, sw = case.input_scale, case.weight_scales
    # every buffer the step writes, allocated before capture
    qx = torch.empty((m, k), dtype=torch.uint8, device=gpu)
    ys = [torch.empty((m, n), dtype=torch.bfloat16, device=gpu) for _ in range(3)]
    qo, ko = torch.empty_like(ys[0]), torch.empty_like(ys[1])
    h = torch.empty((m, inter), dtype=torch.uint8, device=gpu)
    qd = torch.empty((m, k), dtype=torch.uint8, device=gpu)
    sd = torch.empty(1, dtype=torch.float32, device=gpu)
    wsd = torch.empty(1, dtype=torch.int32, device=gpu)
    yd = torch.empty((m, n), dtype=torch.bfloat16, device=gpu)
    outs = [qx, *ys, qo, ko, h, qd, sd, yd]

    def step():
        fp8lin.fp8lin_quantize_static(x, s_in, out=qx)
        fp8lin.fp8lin_gemm_w8a8_group(qx, qws, s_in, sw, outs=ys)
        fp8lin.fp8lin_qk_norm_rope(ys[0], ys[1], wq, wk, c, s, d, 1e-6, q_out=qo, k_out=ko)
        fp8lin.fp8lin_gate_up_swiglu_w8a8(qx, qg, qu, s_in, mlp.s_gate, mlp.s_up, mlp.s_h,
                                          out=h)
        fp8lin.fp8lin_quantize_dynamic(x, out=qd, scale=sd, workspace=wsd)
        fp8lin.fp8lin_gemm_w8a8_dev_scale(qd, qws[0], sd, sw[0], out=yd)

    step()
    torch.cuda.synchronize()
    eager = [t.clone() for t in outs]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # warm the side stream before capture
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    graph = torch.cuda.CUDAGraph()
    for t in outs:
        t.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for t in outs:  # eager work between replays: clobber every output
            t.fill_(7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, (got, ref) in enumerate(zip(outs, eager)):
            assert torch.equal(got, ref), "replay %d: output %d differs from the eager step" % (rep, i)
