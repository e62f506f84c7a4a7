"""fp64 CPU oracle for attention forward.  Test infrastructure only: the
product path (the HIP library and its Python binding) never imports it."""

from .reference import (attended_pairs, attention_ref, attention_varlen_ref, effective_scale, valid_lengths,
                        varlen_spans)

__all__ = ["attention_ref", "attention_varlen_ref", "attended_pairs", "effective_scale", "valid_lengths",
           "varlen_spans"]
