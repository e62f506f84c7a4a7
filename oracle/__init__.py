"""fp64 CPU oracle for attention forward.  Test infrastructure only: the
product path (the HIP library and its Python binding) never imports it."""

from .reference import attention_ref, attended_pairs, effective_scale, valid_lengths

__all__ = ["attention_ref", "attended_pairs", "effective_scale", "valid_lengths"]
