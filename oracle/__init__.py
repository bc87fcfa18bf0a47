"""CPU oracle for online per-tensor FP8 attention.

TEST INFRASTRUCTURE ONLY. This package is the plain, slow, obviously-correct statement of
what the GPU path computes. Only the test suite, the smoke check and the CPU-baseline leg
of the benchmark may import it; the product path (the HIP library and its Python
binding) never does, and shares no code, table or constant with it.

Everything is numpy in float64 (or exact integers). Each function cites the passage of
the source pages it follows:
  * vLLM-Omni user guide "Quantized KV Cache" ("Overview", "Parameters"),
  * vLLM docs "FP8 ViT Encoder Attention" ("Usage", "Scale file format"),
  * the Korean wiki rewrite "FP8 ViT 인코더 어텐션" ("Requirements"),
  * the Ascend chapter "5.4 昇腾量化与 KV Cache 优化", section 4 (names E4M3),
and, for the number format, the OCP 8-bit floating point specification (E4M3).

Parity status: every function here is pinned by CPU tests (tests/test_oracle_*.py)
against closed forms, exhaustive brute force, a library codec or the pages' worked
values. No page prints an attention output, so the attention functions are pinned by a
two-key case worked out by hand (its weights 320 and 128 and sum 448), a pure-Python
brute force of the rule on tiny batches, invariants (a zero query gives the mean of V, a
constant V comes out unchanged, key order does not matter, the largest weight lies in
[224, 448]) and a mutation check that each plausible slip fails one of these.
"""

from .e4m3 import (E4M3_MAX, e4m3_decode, e4m3_encode, e4m3_decode_table,
                   e4m3_finite_values)
from .numerics import bf16_bits_to_f64, f64_to_bf16_bits, round_f32
from .scaling import (AmaxRing, RING_SLOTS, SCALE_FLOOR, amax_bf16, amax_bf16_bits, scale_pair,
                      static_amax)
from .quant import quantize_bf16
from .attention import (attention_f64, fp8_attention, fp8_attention_head,
                        bf16_reference_attention, varlen_rows)

__all__ = [
    "E4M3_MAX", "e4m3_decode", "e4m3_encode", "e4m3_decode_table", "e4m3_finite_values",
    "bf16_bits_to_f64", "f64_to_bf16_bits", "round_f32",
    "AmaxRing", "RING_SLOTS", "SCALE_FLOOR", "amax_bf16", "amax_bf16_bits", "scale_pair",
    "static_amax",
    "quantize_bf16",
    "attention_f64", "fp8_attention", "fp8_attention_head", "bf16_reference_attention",
    "varlen_rows",
]
