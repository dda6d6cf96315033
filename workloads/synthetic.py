"""Seeded synthetic workloads for the static per-tensor FP8 linear layer.

The pages measure on Cosmos3 checkpoints and prompts that are not available
here; these generators stand in for them with the shapes, scales and value
distributions of the layer ([DF-15170] "Logs": a 4096 -> 4096 projection,
bias=False, input amax 0.5430 and weight amax 0.5039 under a max calibrator).

Recipe: every tensor is drawn on the CPU with torch.Generator().manual_seed
(seed) as float32 N(0, 1) times its standard deviation, then cast to bf16
with torch's round-to-nearest-even cast. Static scales are "calibrated" the
way a max calibrator does it: amax / 448 in float32 over a separately seeded
calibration batch (activations) or over the tensor itself (weights).

Nothing here performs the layer's own arithmetic (no quantization, no FP8
GEMM); that is done separately by the HIP library and by the oracle.
"""

from dataclasses import dataclass, field
from typing import List

import numpy as np
import torch

E4M3_MAX = 448.0  # largest finite E4M3 magnitude: the calibrator's target

__all__ = [
    "E4M3_MAX",
    "normal_bf16",
    "normal_f16",
    "normal_f32",
    "rope_tables",
    "norm_weight_bf16",
    "max_calibrated_scale",
    "random_e4m3_codes",
    "all_bf16_patterns",
    "LinearCase",
    "GroupCase",
    "MlpCase",
    "linear_case",
    "config1",
    "config2",
    "config3",
    "config4",
    "QKV_RATIOS",
    "BlockCase",
    "config5",
    "config5_step_input",
]

QKV_RATIOS = (1.0, 0.7, 0.45)


def normal_bf16(shape, std, seed, device="cpu"):
    """bf16 tensor of N(0, std^2) draws, reproducible from `seed`."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=gen, dtype=torch.float32) * float(std)
    return t.to(torch.bfloat16).to(device)


def normal_f16(shape, std, seed, device="cpu"):
    """IEEE binary16 tensor of N(0, std^2) draws (torch's round-to-nearest-even cast)."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=gen, dtype=torch.float32) * float(std)
    return t.to(torch.float16).to(device)


def normal_f32(shape, std, seed, device="cpu"):
    """float32 tensor of N(0, std^2) draws, reproducible from `seed`."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    t = torch.randn(tuple(shape), generator=gen, dtype=torch.float32) * float(std)
    return t.to(device)


def rope_tables(tokens, head_dim, base=10000.0, offset=0):
    """float32 cos / sin tables [tokens, head_dim / 2] of the usual rotary angles
    (position p, frequency base^(-2 i / head_dim)), as a caller precomputes them."""
    half = head_dim // 2
    pos = np.arange(offset, offset + tokens, dtype=np.float64)[:, None]
    inv = base ** (-np.arange(half, dtype=np.float64) * 2.0 / head_dim)
    ang = pos * inv
    return torch.from_numpy(np.cos(ang).astype(np.float32)), torch.from_numpy(np.sin(ang).astype(np.float32))


def norm_weight_bf16(d, seed, std=0.1):
    """bf16 RMSNorm weight [d]: 1 + N(0, std^2), reproducible from `seed`."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    return (1.0 + torch.randn((d,), generator=gen, dtype=torch.float32) * float(std)).to(torch.bfloat16)


def max_calibrated_scale(t):
    """float32(amax(|t|)) / float32(448): the max-calibrator scale of `t`."""
    amax = np.float32(t.detach().abs().max().float().cpu().item())
    return float(amax / np.float32(E4M3_MAX))


def random_e4m3_codes(shape, seed):
    """uint8 tensor of uniformly drawn finite E4M3 codes (NaN codes excluded)."""
    gen = torch.Generator(device="cpu").manual_seed(int(seed))
    r = torch.randint(0, 254, tuple(shape), generator=gen, dtype=torch.int32)
    r = torch.where(r >= 0x7F, r + 1, r)  # skip 0x7F; 253 -> 0xFE
    return r.to(torch.uint8)


def all_bf16_patterns():
    """All 65,536 bf16 bit patterns in order, as a bf16 tensor [65536]."""
    bits = torch.arange(65536, dtype=torch.int32).to(torch.int16)
    return bits.view(torch.bfloat16)


@dataclass
class LinearCase:
    """One projection: activation x [M, K], unquantized weight w [N, K]."""

    x: torch.Tensor
    w: torch.Tensor
    input_scale: float
    weight_scale: float


@dataclass
class GroupCase:
    """Projections sharing one activation and one input scale (Q/K/V)."""

    x: torch.Tensor
    ws: List[torch.Tensor]
    input_scale: float
    weight_scales: List[float]
    ratios: tuple = field(default=())


@dataclass
class MlpCase:
    """Split gated MLP: gate/up on a shared input, SwiGLU, then down."""

    x: torch.Tensor
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor
    input_scale: float
    s_gate: float
    s_up: float
    s_down: float
    s_h: float


def linear_case(m, n, k, x_std, w_std, seed_x, seed_w, seed_cal, cal_rows):
    x = normal_bf16((m, k), x_std, seed_x)
    w = normal_bf16((n, k), w_std, seed_w)
    cal = normal_bf16((cal_rows, k), x_std, seed_cal)
    return LinearCase(x, w, max_calibrated_scale(cal), max_calibrated_scale(w))


def config1():
    """x [128, 512] ~ N(0, 0.5), W [512, 512] ~ N(0, 0.02).

    The input scale comes from a 64-element calibration draw, so about 1% of
    x exceeds 448 * s_in and saturates.
    """
    x = normal_bf16((128, 512), 0.5, 123)
    w = normal_bf16((512, 512), 0.02, 124)
    cal = normal_bf16((64,), 0.5, 125)
    return LinearCase(x, w, max_calibrated_scale(cal), max_calibrated_scale(w))


def config2(m=8192):
    """4096 -> 4096 projection, x [m, 4096] ~ N(0, 0.35) (m in {1024, 8192})."""
    x = normal_bf16((8192, 4096), 0.35, 223)[:m].contiguous()
    w = normal_bf16((4096, 4096), 0.02, 224)
    cal = normal_bf16((1024, 4096), 0.35, 225)
    return LinearCase(x, w, max_calibrated_scale(cal), max_calibrated_scale(w))


def config3(m=16384, k=4096, n=4096):
    """Shared QKV: x [m, k] ~ N(0, 0.35); W_q, W_k, W_v ~ N(0, (0.02 r_i)^2).

    Weight scales keep the exact ratios r = (1, 0.7, 0.45):
    s_i = float32(r_i * s0) with s0 = max_i(amax(W_i) / r_i) / 448, so the
    three scales genuinely differ and no weight saturates.
    """
    x = normal_bf16((m, k), 0.35, 323)
    ws = [normal_bf16((n, k), 0.02 * r, 324 + i) for i, r in enumerate(QKV_RATIOS)]
    amax = [float(w.abs().max().float()) for w in ws]
    s0 = np.float32(max(a / r for a, r in zip(amax, QKV_RATIOS))) / np.float32(E4M3_MAX)
    scales = [float(np.float32(r) * s0) for r in QKV_RATIOS]
    cal = normal_bf16((1024, k), 0.35, 327)
    return GroupCase(x, ws, max_calibrated_scale(cal), scales, QKV_RATIOS)


def config4(m=8192, hidden=4096, inter=16384, cal_rows=1024, device="cpu"):
    """Split gated MLP on x [m, hidden] ~ N(0, 0.35).

    W_gate, W_up [inter, hidden] and W_down [hidden, inter] ~ N(0, 0.02).
    s_h, the down projection's input scale, is calibrated on an unquantized
    float32 forward of `cal_rows` calibration rows (what an offline max
    calibrator observes at the SwiGLU output); `device` only selects where
    that float32 calibration forward runs.
    """
    x = normal_bf16((m, hidden), 0.35, 423)
    w_gate = normal_bf16((inter, hidden), 0.02, 424)
    w_up = normal_bf16((inter, hidden), 0.02, 425)
    w_down = normal_bf16((hidden, inter), 0.02, 426)
    cal = normal_bf16((cal_rows, hidden), 0.35, 427)
    with torch.no_grad():
        c = cal.to(device).float()
        g = c @ w_gate.to(device).float().t()
        u = c @ w_up.to(device).float().t()
        h = torch.nn.functional.silu(g) * u
        s_h = max_calibrated_scale(h)
        del c, g, u, h
    return MlpCase(
        x,
        w_gate,
        w_up,
        w_down,
        max_calibrated_scale(cal),
        max_calibrated_scale(w_gate),
        max_calibrated_scale(w_up),
        max_calibrated_scale(w_down),
        s_h,
    )


@dataclass
class BlockCase:
    """Unquantized bf16 weights and calibrated static scales of one block."""

    w_qkv: List[torch.Tensor]
    w_out: torch.Tensor
    w_gate: torch.Tensor
    w_up: torch.Tensor
    w_down: torch.Tensor
    s_qkv: List[float]
    s_out: float
    s_gate: float
    s_up: float
    s_down: float
    s_in_qkv: float
    s_in_out: float
    s_in_mlp: float
    s_h: float


def config5(num_blocks=4, hidden=4096, inter=16384, cal_rows=256, device="cpu"):
    """A stack of synthetic blocks for the denoising-schedule workload.

    Block b: QKV (3 x hidden^2), output projection (hidden^2), gate/up
    (inter x hidden each), down (hidden x inter), all ~ N(0, 0.02) with seeds
    5000 + 10 b + i. The down weight is rescaled once so that a calibration
    pass leaves the block output with standard deviation 0.35, like its
    input. Input scales are max-calibrated on an unquantized float32 forward
    of `cal_rows` fresh N(0, 0.35) rows (seed 700) -- the calibration
    trajectory of a sampler without latent feedback; `device` only selects
    where that float32 forward runs. Attention is the identity on V.
    """
    cal = normal_bf16((cal_rows, hidden), 0.35, 700).to(device).float()
    blocks = []
    for b in range(num_blocks):
        seed = 5000 + 10 * b
        w_qkv = [normal_bf16((hidden, hidden), 0.02, seed + i) for i in range(3)]
        w_out = normal_bf16((hidden, hidden), 0.02, seed + 3)
        w_gate = normal_bf16((inter, hidden), 0.02, seed + 4)
        w_up = normal_bf16((inter, hidden), 0.02, seed + 5)
        w_down = normal_bf16((hidden, inter), 0.02, seed + 6)
        with torch.no_grad():
            s_in_qkv = max_calibrated_scale(cal)
            v = cal @ w_qkv[2].to(device).float().t()
            s_in_out = max_calibrated_scale(v)
            o = v @ w_out.to(device).float().t()
            s_in_mlp = max_calibrated_scale(o)
            g = o @ w_gate.to(device).float().t()
            u = o @ w_up.to(device).float().t()
            h = torch.nn.functional.silu(g) * u
            s_h = max_calibrated_scale(h)
            y = h @ w_down.to(device).float().t()
            gain = 0.35 / float(y.std())
            w_down = (w_down.float() * gain).to(torch.bfloat16)
            cal = (h @ w_down.to(device).float().t())
            del v, o, g, u, h, y
        blocks.append(
            BlockCase(
                w_qkv, w_out, w_gate, w_up, w_down,
                [max_calibrated_scale(w) for w in w_qkv],
                max_calibrated_scale(w_out),
                max_calibrated_scale(w_gate),
                max_calibrated_scale(w_up),
                max_calibrated_scale(w_down),
                s_in_qkv, s_in_out, s_in_mlp, s_h,
            )
        )
    return blocks


def config5_step_input(step, branch, m=16384, hidden=4096):
    """Fresh input of one CFG pass of one denoising step: N(0, 0.35), seed 600 + 2 step + branch."""
    return normal_bf16((m, hidden), 0.35, 600 + 2 * step + branch)
