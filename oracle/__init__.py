"""CPU oracle for the W8A8 FP8 linear path — TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct NumPy definition of what
the GPU library computes. Only the test suite, the smoke check and the
benchmark's CPU-baseline leg may import it; the product path never does,
and this package imports nothing from the product.

What it defines, and where the pages state it:

* E4M3 codec (``e4m3``): the FP8 format the checkpoints store
  (Lernex/Metis-1.6-Logos-FP8, "What is in FP8": E4M3 weights;
  Lernex/Metis-1.6-Praxis-NVFP4, hub sidebar: tensor type F8_E4M3).
* Per-row dynamic quantisation (``quant``): one scale per token for
  activations and one per output row for weights (Lernex/Metis-1.6-Logos-
  FP8, "What is in FP8"; sglang-metis 0.1.0, "Serve", memory paragraph).
* The W8A8 linear (``linear``): the per-token FP8 version of a layer's
  input times the FP8 weights (Lernex/Metis-1.6-Logos-FP8, "What
  --fast-math does"); the weights are decoded exactly and the product is
  carried out in high precision, the emulation the same page's
  "Benchmarks" section describes for its FP8 scores.
* The default-maths linear (``linear.w8a16_linear``): without the fast-math
  flag the FP8 weights are widened to 16 bits and the product is taken in
  BF16 on unquantised activations (Lernex/Metis-1.6-Logos-FP8, "What
  --fast-math does").
* MXFP4 (``mxfp4``): the 4-bit E2M1 expert format with one power-of-two
  scale per 32 inputs, the GPU-native analogue of the NVFP4 experts
  (Lernex/Metis-1.6-Praxis-NVFP4, "What is in NVFP4": E2M1 values with a
  scale per small block; "What --fast-math does": expert inputs rounded to
  FP4), its block quantiser, linear layer and routed-expert pass.
* The routed-expert chain (``moe``): routed experts in FP8 with the same
  scheme, top-k routing, the stack run twice with shared weights
  (Lernex/Metis-1.6-Praxis, "Architecture"; sglang-metis 0.1.0, "How the
  model maps onto SGLang"); a token's output is the router-weighted sum of
  its routed copies' outputs at full precision, rounded once to BF16.

Floating point is carried in float64; where a step is defined at float32
precision (the scale and the scaled value fed to the E4M3 encoder) the
oracle rounds to float32 explicitly. BF16 outputs are rounded once, from
float64, to nearest even.
"""
from .e4m3 import (E4M3_MAX, decode, decode_table, encode, encode_bits,
                   finite_codes, magnitudes)
from .bf16 import bf16_bits_to_f64, round_to_bf16_bits
from .quant import bf16_bits_to_f32, quantize_rows
from .linear import w8a8_linear, w8a8_linear_int, w8a16_linear
from .moe import (route, grouped_gate_up, moe_pass, moe_two_pass, swiglu_f32, bf16_values, combine_copies)
from .mxfp4 import (e2m1_decode, e2m1_encode, e8m0_value, mx_dequant, mx_quantize_rows, mx_unpack, mxfp4_linear,
                    moe_mxfp4_pass, moe_mxfp4_two_pass)

__all__ = [
    "E4M3_MAX", "decode", "decode_table", "encode", "encode_bits", "finite_codes", "magnitudes",
    "bf16_bits_to_f64", "round_to_bf16_bits", "bf16_bits_to_f32", "quantize_rows",
    "w8a8_linear", "w8a8_linear_int", "w8a16_linear", "route", "grouped_gate_up", "moe_pass", "moe_two_pass",
    "swiglu_f32", "bf16_values", "combine_copies", "e2m1_decode", "e2m1_encode", "e8m0_value", "mx_dequant", "mx_quantize_rows", "mx_unpack",
    "mxfp4_linear", "moe_mxfp4_pass", "moe_mxfp4_two_pass",
]
