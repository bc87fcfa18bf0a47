"""Per-tensor BF16 -> E4M3 quantisation (oracle; test only).

vLLM-Omni "Quantized KV Cache", "Overview": Q, K and V are quantised to FP8 on the fly,
right before the attention operator. vLLM docs "FP8 ViT Encoder Attention" (first
paragraph) says the same for the ViT encoder.

Rule: q8 = E4M3( binary32( x * inv ) ), where x is the bf16 value and inv the tensor's
binary32 quantisation multiplier (448 / A). The product of a bf16 (8 significant bits)
and a binary32 (24 bits) is exact in float64, so rounding it once to binary32 is exactly
an IEEE single-precision multiply. Then E4M3 encode (RNE, saturating).
"""

import numpy as np

from .e4m3 import e4m3_encode
from .numerics import bf16_bits_to_f64, round_f32


def quantize_bf16(bits, inv):
    """E4M3 codes (uint8, same shape) of bf16 bit patterns under multiplier inv."""
    x = bf16_bits_to_f64(bits)
    y = round_f32(x * float(inv))
    return e4m3_encode(y)
