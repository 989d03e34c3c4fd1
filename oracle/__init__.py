"""CPU oracle for causal prefill attention (test infrastructure only).

This package is the checker, not the product. Only the test suite, the
smoke check of the package entry point and the CPU-baseline leg of the
benchmark may import it. The GPU library neither imports nor links
anything here, and nothing here imports the GPU library.

Everything is plain numpy in float64 (attention) or exact integer/bit
arithmetic (the bf16 and e4m3fn codecs, the power-of-two quantizer).

Sources (cited by page title and section):
- "ZYFA" README (GitHub page of Zyphra/zyfa): Usage (LSE, descales,
  padding), Supported configurations (formats, head dims, GQA), Accuracy
  (fp64 attention on the same quantized inputs), Kernel design (every
  conversion rounds to nearest even).
- flash-attention RDNA3 extension page, kernel notes (partial results over
  key splits merged by an LSE reduction), with the README's Accuracy note on
  merging results over key ranges: partial.py.
- "ZYFA" README, "Using FP8 attention in a model" (Hadamard rotation of q
  and k before quantization): rotation.py.

Parity pins for every function live in tests/test_oracle_*.py and
tests/golden/. No function here is "parity unpinned".
"""
from .codecs import (bf16_round, bf16_decode, bf16_encode_bits, e4m3fn_decode,
                     e4m3fn_encode, E4M3FN_MAX)
from .quantize import fp8_quantize_ref
from .attention import causal_attention_ref, causal_probs_ref, causal_attention_rows_ref
from .partial import range_attention_ref, range_attention_rows_ref, lse_merge_ref, lse_merge_layout_ref
from .rotation import (hadamard, rotation_matrix, rotate_ref, quantize_rotated_ref, key_mean_ref,
                       quantize_shifted_rotated_ref)

__all__ = [
    "bf16_round", "bf16_decode", "bf16_encode_bits", "e4m3fn_decode", "e4m3fn_encode",
    "E4M3FN_MAX", "fp8_quantize_ref", "causal_attention_ref", "causal_probs_ref",
    "causal_attention_rows_ref", "range_attention_ref",
    "range_attention_rows_ref", "lse_merge_ref", "lse_merge_layout_ref", "hadamard",
    "rotation_matrix", "rotate_ref", "quantize_rotated_ref", "key_mean_ref", "quantize_shifted_rotated_ref",
]
