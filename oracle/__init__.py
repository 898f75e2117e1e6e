"""CPU oracle for the QLoRA frozen-base NF4 linear layer.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously correct
definition of what the GPU library computes.  Only the test-suite, the smoke
check and the CPU-baseline leg of the benchmark may import it; the product path
(the HIP library and its Python binding) never does, and shares no code,
table or constant generator with it.

Sources are the pages on QLoRA: "DL0087 QLoRA: 4-bit Quantized LoRA"
(numbered list items (1)-(4), Figure 1, Mathematical Formulation),
"QLoRA: Finetuning 65B Models on a Single GPU with 4-Bit Quantization"
(sections "4-bit NormalFloat" and "Double Quantization and Paged Optimizers";
the INT4 / FP4 codebooks and fp32 constants it sets NF4 against live in
oracle.codebooks),
"QLoRA: Quantized Low Rank Adaptation at Extreme Scale" (The Quantization
Layer) and "QLoRA (Quantized Low-Rank Adaptation)" (The Efficient Symphony
of the QLoRA Workflow).

Every function states the passage it follows.  Where the pages are silent the
reading taken is stated in the function's docstring.

Pin status: every function here is pinned by a CPU test against something
other than itself (closed forms printed on the pages, exact rational brute
force, independent library routines, finite differences); none is
"parity unpinned" except that the NF4 level *values* cannot be compared with
the original paper's table, which the pages do not print (the construction
itself is pinned).
"""
from .nf4 import (BLOCK, GROUP, normal_quantile, nf4_levels_f64, nf4_levels,
                  bf16_rne_bits, bf16_bits_to_f64, encode, quantize,
                  unpack_codes, dequantize, dequantize_at, code_boundaries,
                  storage_bytes, bits_per_param)
from . import adamw, codebooks
from .linear import (linear_fwd_f64, linear_bwd_f64, linear_fwd, linear_bwd, block_fwd_f64,
                     block_bwd_f64, block_fwd, block_bwd)

__all__ = [
    "BLOCK", "GROUP", "normal_quantile", "nf4_levels_f64", "nf4_levels",
    "bf16_rne_bits", "bf16_bits_to_f64", "encode", "quantize", "unpack_codes",
    "dequantize", "dequantize_at", "code_boundaries", "storage_bytes",
    "bits_per_param", "linear_fwd_f64", "linear_bwd_f64", "linear_fwd",
    "linear_bwd", "block_fwd_f64", "block_bwd_f64", "block_fwd", "block_bwd", "adamw", "codebooks",
]
