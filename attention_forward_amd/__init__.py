"""Fused attention forward for AMD Instinct MI355X (gfx950).

The compute path is the HIP library built from ``csrc/`` (C ABI in
``include/fa.h``); ``attention_forward_amd.fa`` is its ctypes binding.  The
library is loaded on first use and its absence is an error.
"""

from .fa import (  # noqa: F401
    FA_BF16,
    FA_FP16,
    FA_OK,
    FAError,
    attention,
    attention_nvfp4,
    attention_varlen,
    fa_abi_version,
    fa_fwd,
    fa_fwd_nvfp4,
    fa_fwd_plan,
    fa_fwd_static,
    fa_fwd_strided,
    fa_fwd_variant,
    fa_fwd_variant_workspace_bytes,
    fa_fwd_varlen,
    fa_fwd_workspace_bytes,
    fa_set_workspace,
    fa_status_string,
    load_library,
    reserve_workspace,
)

__all__ = [
    "FA_BF16",
    "FA_FP16",
    "FA_OK",
    "FAError",
    "attention",
    "attention_nvfp4",
    "attention_varlen",
    "fa_abi_version",
    "fa_fwd",
    "fa_fwd_nvfp4",
    "fa_fwd_plan",
    "fa_fwd_static",
    "fa_fwd_strided",
    "fa_fwd_variant",
    "fa_fwd_variant_workspace_bytes",
    "fa_fwd_varlen",
    "fa_fwd_workspace_bytes",
    "fa_set_workspace",
    "fa_status_string",
    "load_library",
    "reserve_workspace",
]
