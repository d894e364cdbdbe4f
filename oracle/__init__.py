"""CPU oracle (float64) for attention forward and gradients -- test infrastructure only.

Only tests, the smoke check and the bench's CPU-baseline leg may use it.
"""
from .softmax_attention import (attention, attention_backward, attention_fp8, attention_two_pass,
                                attention_from_storage, decode, decode_bf16,
                                decode_f16, decode_fp8_e4m3, scale_value)

from .ffn import ffn, ffn_chunked, gelu_tanh

__all__ = ["ffn", "ffn_chunked", "gelu_tanh", "attention", "attention_backward", "attention_fp8",
           "attention_two_pass", "attention_from_storage",
           "decode", "decode_bf16", "decode_f16", "decode_fp8_e4m3", "scale_value"]
