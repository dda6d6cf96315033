"""Step-policy driver: a stack of static-FP8 transformer-style blocks.

Each denoising step asks fp8lin_step_policy for the mode of the generation
tower ([DF-14664] "Behavior": the choice is made once per scheduler step, so
the CFG cond and uncond passes of a step run the same mode) and runs every
block in it. A block is the linear-layer skeleton of a decoder layer:
shared-QKV projections, an output projection, a split gated MLP (gate/up on a
shared quantization, two-input SwiGLU, down projection) -- [TRT-17476]
"What changed". On W8A8 steps activations are quantized (once per shared
group, and SwiGLU emits E4M3 straight into the down projection); on W8A16
steps every sharing site stands down and all GEMMs take bf16 activations
("Denoising-step activation precision").

The attention between the projections is not part of the layer and is
replaced by the identity on V; q and k are computed for their cost and left
unused. Only C-ABI calls are made here; buffers are allocated once.
"""

from dataclasses import dataclass, field
from typing import List

import torch

from . import (
    DT_BF16,
    DT_E4M3,
    MODE_W8A8,
    MODE_W8A16,
    TOWER_GENERATION,
    fp8lin_gate_up_swiglu_w8a8,
    fp8lin_gate_up_swiglu_w8a16,
    fp8lin_gemm_w8a8,
    fp8lin_gemm_w8a16,
    fp8lin_qkv_shared,
    fp8lin_quantize_static,
    fp8lin_step_policy,
    fp8lin_swiglu_2in_quant,
)


@dataclass
class BlockWeights:
    """E4M3 weights (uint8 on the device) and static scales of one block."""

    qkv: List[torch.Tensor]
    s_qkv: List[float]
    s_in_qkv: float
    out: torch.Tensor
    s_out: float
    s_in_out: float
    gate: torch.Tensor
    up: torch.Tensor
    s_gate: float
    s_up: float
    s_in_mlp: float
    down: torch.Tensor
    s_down: float
    s_h: float  # the down projection's input scale (SwiGLU output scale)


@dataclass
class Buffers:
    m: int
    hidden: int
    inter: int
    device: torch.device
    q: torch.Tensor = field(init=False)
    k: torch.Tensor = field(init=False)
    v: torch.Tensor = field(init=False)
    o: torch.Tensor = field(init=False)
    g: torch.Tensor = field(init=False)
    u: torch.Tensor = field(init=False)
    h8: torch.Tensor = field(init=False)
    h16: torch.Tensor = field(init=False)
    xq: torch.Tensor = field(init=False)
    out: List[torch.Tensor] = field(init=False)

    def __post_init__(self):
        bf, u8 = torch.bfloat16, torch.uint8
        m, d, i, dev = self.m, self.hidden, self.inter, self.device
        self.q, self.k, self.v, self.o = (torch.empty((m, d), dtype=bf, device=dev) for _ in range(4))
        self.g, self.u = (torch.empty((m, i), dtype=bf, device=dev) for _ in range(2))
        self.h8 = torch.empty((m, i), dtype=u8, device=dev)
        self.h16 = torch.empty((m, i), dtype=bf, device=dev)
        self.xq = torch.empty((m, max(d, i)), dtype=u8, device=dev)
        self.out = [torch.empty((m, d), dtype=bf, device=dev) for _ in range(2)]


def block_forward(w: BlockWeights, x: torch.Tensor, mode: int, buf: Buffers, out: torch.Tensor, fused_mlp=False):
    """One block in `mode`; writes the block output into `out` (bf16 [m, hidden]).

    fused_mlp: gate/up and the SwiGLU run as one fused launch
    (fp8lin_gate_up_swiglu_w8a8 on the once-quantized MLP input on W8A8
    steps, fp8lin_gate_up_swiglu_w8a16 on 16-bit steps); the output equals
    the split path's bit for bit.
    """
    m, d = x.shape
    xq = buf.xq.view(-1)[: m * d].view(m, d)
    if mode == MODE_W8A8:
        fp8lin_qkv_shared(x, w.qkv, w.s_qkv, [w.s_in_qkv] * 3, MODE_W8A8, outs=[buf.q, buf.k, buf.v], workspace=xq)
        fp8lin_quantize_static(buf.v, w.s_in_out, out=xq)
        fp8lin_gemm_w8a8(xq, w.out, w.s_in_out, w.s_out, out=buf.o)
        if fused_mlp:
            fp8lin_quantize_static(buf.o, w.s_in_mlp, out=xq)
            fp8lin_gate_up_swiglu_w8a8(xq, w.gate, w.up, w.s_in_mlp, w.s_gate, w.s_up, w.s_h, out=buf.h8)
        else:
            fp8lin_qkv_shared(buf.o, [w.gate, w.up], [w.s_gate, w.s_up], [w.s_in_mlp] * 2, MODE_W8A8,
                              outs=[buf.g, buf.u], workspace=xq)
            fp8lin_swiglu_2in_quant(buf.g, buf.u, w.s_h, DT_E4M3, out=buf.h8)
        fp8lin_gemm_w8a8(buf.h8, w.down, w.s_h, w.s_down, out=out)
    elif mode == MODE_W8A16:
        fp8lin_qkv_shared(x, w.qkv, w.s_qkv, [w.s_in_qkv] * 3, MODE_W8A16, outs=[buf.q, buf.k, buf.v])
        fp8lin_gemm_w8a16(buf.v, w.out, w.s_out, out=buf.o)
        if fused_mlp:
            fp8lin_gate_up_swiglu_w8a16(buf.o, w.gate, w.up, w.s_gate, w.s_up, out=buf.h16)
        else:
            fp8lin_qkv_shared(buf.o, [w.gate, w.up], [w.s_gate, w.s_up], [w.s_in_mlp] * 2, MODE_W8A16,
                              outs=[buf.g, buf.u])
            fp8lin_swiglu_2in_quant(buf.g, buf.u, 1.0, DT_BF16, out=buf.h16)
        fp8lin_gemm_w8a16(buf.h16, w.down, w.s_down, out=out)
    else:
        raise ValueError("mode must be MODE_W8A8 or MODE_W8A16")
    return out


def stack_forward(blocks: List[BlockWeights], x: torch.Tensor, mode: int, buf: Buffers, fused_mlp=False):
    """All blocks in one mode; returns the buffer holding the last output."""
    h = x
    for b, w in enumerate(blocks):
        h = block_forward(w, h, mode, buf, buf.out[b % 2], fused_mlp)
    return h


def run_schedule(blocks, policy, num_steps, step_inputs, buf, branches=2, fused_mlp=False, step_hook=None):
    """Run `num_steps` denoising steps of `branches` CFG passes each.

    step_inputs(step, branch) returns the bf16 input of that pass. Returns
    the per-step mode trace (the policy is asked once per step).
    step_hook(step, mode, done), if given, is called before (done = False)
    and after (done = True) the passes of each step are enqueued, e.g. to
    record events that time the step kinds apart.
    """
    trace = []
    for step in range(num_steps):
        mode = fp8lin_step_policy(policy, TOWER_GENERATION, step, num_steps)
        trace.append(mode)
        if step_hook is not None:
            step_hook(step, mode, False)
        for branch in range(branches):
            stack_forward(blocks, step_inputs(step, branch), mode, buf, fused_mlp)
        if step_hook is not None:
            step_hook(step, mode, True)
    return trace
