"""CPU oracle for the QLoRA NF4 linear layer.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously
correct definition that the HIP library is checked against.  Only the test
suite, the ``smoke()`` entry point and the benchmark's CPU-baseline leg may
import it; the product path (``bit_nf4_quantized_13_amd``) never does, and
this package imports nothing from it.

Sources (the pages are cited by title and section):
  * chkda.github.io, "Why do we need LoRA and QLoRA?" -- sections
    "First, how does k-bit quantization work?", "NF4: Choose the codebook to
    fit the distribution", "Building the NF4 codebook", "Quantizing and
    dequantizing with the codebook", "Double quantization and double
    dequantization", "How does it work?", "How does alpha/r control adapter
    strength?", "Merging LoRA weights for inference".
  * fromzero2ai.dev, "LoRA and QLoRA" -- "Linear Layer Deconstruction",
    "Low-Rank Matrix Factorization", "Why Does This Save Memory?".

Modules:
  nf4    -- codebook, blockwise NF4 quantize/dequantize, Int8 absmax,
            double quantization and doubleDequant (bit-exact contracts).
  qlora  -- the linear layer forward and backward in float64.
"""
from . import nf4, qlora  # noqa: F401
