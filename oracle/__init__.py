"""CPU oracle for the fused dequantize-and-multiply of block-quantized weights.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path imports this package:
only the test suite, the smoke check and the benchmark's CPU-baseline leg do.
It shares no code with the HIP library (no headers, helpers or tables) and
never reads anything the HIP path produced, except where a test hands it a
packed buffer to unpack for the round-trip check.

What it computes, and where the pages define it:

* The weights are blocks of small integers plus a per-block fp16 scale (and a
  min or zero), multiplied against f32/f16 activations without forming the
  dense matrix (llmopt README, "Current compiler and runtime": packed
  group-64 W4A16 linear kernels; aot-llm README, feature list "Static code
  generation" and "SIMD kernels": matvec_q4_k, matvec_q6_k, Q8_0, and the
  Metal backend notes on on-the-fly dequantization with f32 activations).
* The correctness baseline is the packed-block -> dense conversion followed by
  a plain product (pytensor-ml issue 53, PR 15 "GGUF loading", item F-41),
  compared against an f64 reference (aot-llm README, Metal backend notes:
  kernel error against an f64 reference).

Modules:
  fp         exact fp16 / bf16 decoding from the IEEE-754 field definitions
  dequantize per-format dequantization to f32, in the normative order
  reference  f64 matvec / GEMM, the per-output tolerance bound, and the fused
             decode epilogues (bias / residual add, SwiGLU) with their bounds
  layout     reference packer / unpacker of the library's packed layout v1
  q8act      activations quantized to 8-bit blocks (the integer-dot variant)

Parity status: every function here is pinned by `-m "not gpu"` tests against
hand-worked blocks, library routines and exact rational arithmetic.
"""
from .fp import f16_to_f32, f16_to_f64, bf16_to_f32, bf16_to_f64  # noqa: F401
from .dequantize import dequant, dequant_rows  # noqa: F401
from .reference import matvec_ref, gemm_ref, tolerance_bound, check_within  # noqa: F401
from .reference import silu_ref, swiglu_ref, swiglu_bound, epilogue_ref, epilogue_bound  # noqa: F401
from .layout import pack_ref, unpack_ref, packed_bytes_ref  # noqa: F401
from .q8act import quantize_q8x, dequant_q8x, pack_q8x, q8x_record_bytes  # noqa: F401
