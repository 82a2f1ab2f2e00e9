"""CPU oracle for the ConvRot-rotated low-bit quantized linear layer.

TEST INFRASTRUCTURE ONLY. This package is a plain, slow, deliberately
unoptimised numpy statement of what the GPU path computes. Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import it.
The GPU library never calls, links or falls back to anything here, and this
package imports nothing from the GPU path (it shares no code, table or
constant generator with it).

Sources (the five web pages this work follows; cited by title and section):
  [P1] "Qwen-Image-Edit-2511 - INT4 tensorwise W4A4 (+ConvRot, mixed int8 fallback)"
  [P2] "Qwen-Image-Edit-2511-W4A8-ConvRot" (model card mirror)
  [P3] "Qwen-Image-Edit-2511 INT4 (ComfyUI Optimized)" (SVDQuant W4A4)
  [P4] "Qwen Image 2.1 - Hybrid W4A8 / INT8 ConvRot for ComfyUI"
  [P5] "Qwen3-4B - ConvRot W4A4 (ComfyUI text encoder)"

Modules, in the order the path runs:
  hadamard  - the group-wise regular Hadamard rotation (ConvRot)
  quant     - dynamic symmetric / unsigned-shift / asymmetric quantizers
  pack      - int4 packing (natural and tile-packed layouts)
  gemm      - exact integer GEMM and per-group partial sums
  linear    - epilogues and the composed reference linears

Every function states the passage it follows, or, where the pages are silent,
the reading taken and why. The pins that tie this oracle to the mathematics
and to the pages (closed forms, invariants, brute force on tiny inputs,
constructed rounding ties) live in tests/test_oracle_*.py.
"""
from . import hadamard, quant, pack, gemm, linear  # noqa: F401
