"""fp64 CPU oracle for attention forward, and the NVFP4 quantisation of its
output.  Test infrastructure only: the product path (the HIP library and its
Python binding) never imports it."""

from .nvfp4 import attention_nvfp4_ref, nvfp4_dequantize, nvfp4_quantize
from .reference import (attended_pairs, attention_ref, attention_varlen_ref, effective_scale, valid_lengths,
                        varlen_spans)

__all__ = ["attention_ref", "attention_varlen_ref", "attended_pairs", "effective_scale", "valid_lengths",
           "varlen_spans", "attention_nvfp4_ref", "nvfp4_quantize", "nvfp4_dequantize"]
