"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This package holds none of the layer's arithmetic: it draws random tensors
and plays the part of the offline calibration that produces a checkpoint's
static scales (amax / 448, the max-calibrator rule). Weights are handed out
unquantized, in bf16; each side (the HIP library and the CPU oracle)
quantizes them to E4M3 with its own code.
"""

from .synthetic import *  # noqa: F401,F403
