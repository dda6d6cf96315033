"""Plain, slow CPU oracle for the static per-tensor FP8 linear layer.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this package: only the test suite (``tests/``), the smoke check in
``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` use it.
It shares no code, constant table or helper with the HIP library in
``w8a16_linear_layers_amd/``; both sides only consume the seeded synthetic
inputs of ``workloads/``, which hold none of the method's arithmetic.

Everything here is NumPy on the host, in float64 unless the pages fix a
precision (the activation quotient is an fp32 division because the
reference's quantizer divides fp32 values by an fp32 scale).

Sources (web pages; cited by title and section):
  [CF-157]  NVIDIA/cosmos-framework PR #157, "feat: load ModelOpt static-FP8
            checkpoints via TorchAO" -- sections "Commits", "Verification".
  [DF-14664] huggingface/diffusers PR #14664, "[Cosmos3] Mixed W8A8/W8A16
            denoising for ModelOpt FP8 checkpoints" -- "Behavior", "Tests".
  [TRT-17476] NVIDIA/TensorRT-LLM PR #17476, "Load static FP8 Cosmos3
            Nano/Super checkpoints without re-quantizing them" --
            "Description", "What changed", "Test Coverage",
            "Denoising-step activation precision".
  [DF-15170] huggingface/diffusers issue #15170, "Cosmos 3 docs: FP8 snippet
            fails at the first W8A8 step ..." -- "Describe the bug", "Logs".

Modules:
  e4m3      -- OCP E4M3 ("FN") decode / saturating round-to-nearest-even encode
  bf16      -- bfloat16 bit conversion and round-to-nearest-even
  f16       -- IEEE binary16 decode and round-to-nearest-even
  linear    -- static activation quantization, W8A8 and W8A16 GEMMs,
               shared-QKV, the fused max-scale re-quantization identity,
               and the float32-accumulation bound of W8A16 outputs
  dynamic   -- dynamic per-tensor quantization: the scale from a runtime amax
  swiglu    -- two-input SwiGLU with E4M3, bf16 or fp16 output
  qknorm    -- per-head QK RMSNorm followed by rotate-half RoPE
  policy    -- diffusion_step_policy validation and per-step mode selection

Parity pins: every function is pinned by tests in ``tests/test_oracle_*.py``
against closed forms, brute force, an independent library routine (torch's
CPU float8_e4m3fn cast) or the traces printed on the pages. The SwiGLU
E4M3 path near rounding midpoints is pinned only up to the documented
near-tie rule (see ``swiglu``).
"""

from . import bf16, dynamic, e4m3, f16, linear, policy, qknorm, swiglu  # noqa: F401
