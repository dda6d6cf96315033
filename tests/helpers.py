"""Small shared helpers for the GPU parity tests (conversion and reporting)."""

import sys

import numpy as np
import torch

from oracle import linear, swiglu


def announce(what):
    """Print the case name before a GPU step (flushed, so a crash still names it)."""
    print("\n[case] %s" % what, flush=True)
    sys.stdout.flush()


def f32(t):
    """bf16 torch tensor (any device) -> float32 numpy array with the same values."""
    return t.detach().float().cpu().numpy()


def u8(t):
    return t.detach().cpu().numpy().astype(np.uint8)


def bf16_weight(w):
    return f32(w)


def assert_gemm_close(y_gpu, y_ref, what):
    """GEMM acceptance rule: |y - y_ref| <= 2^-7 |y_ref| + 1e-3 rms(y_ref), elementwise."""
    y = f32(y_gpu).astype(np.float64) if isinstance(y_gpu, torch.Tensor) else np.asarray(y_gpu, np.float64)
    ok = linear.within_gemm_tolerance(y, y_ref)
    if not ok.all():
        bad = np.argwhere(~ok)
        i = tuple(bad[0])
        raise AssertionError(
            "%s: %d of %d outside tolerance; first at %s: gpu %r ref %r"
            % (what, (~ok).sum(), ok.size, i, y[i], y_ref[i])
        )


def sample_rows(m, count, seed):
    rng = np.random.default_rng(seed)
    rows = np.unique(np.concatenate([rng.choice(m, size=min(count, m), replace=False), [0, m - 1]]))
    return rows


def check_swiglu_codes(g, u, s_h, got):
    """SwiGLU E4M3 codes of bf16 g, u against the oracle's: equal, except where the exact value lies within
    relative 2^-20 of an E4M3 rounding midpoint, where the other neighbour (one code step away) is accepted.
    Returns the number of such differences."""
    ref, t = swiglu.swiglu_2in_quant(f32(g).astype(np.float64), f32(u).astype(np.float64), s_h)
    diff = got != ref
    if diff.any():
        near = swiglu.near_midpoint(t)
        assert not (diff & ~near).any(), "%d codes differ away from a midpoint" % np.count_nonzero(diff & ~near)
        # where they differ, the GPU chose the other neighbour of the midpoint
        step = (got[diff] & 0x7F).astype(int) - (ref[diff] & 0x7F).astype(int)
        assert np.all(np.abs(step) == 1)
    return int(diff.sum())
