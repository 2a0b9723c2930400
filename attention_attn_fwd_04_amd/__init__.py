"""MI355X (gfx950) fused causal RoPE attention forward.

The compute lives in the HIP library libattn_mi355x.so (C ABI in
include/attn.h); `binding` marshals torch tensors into it.  Build with
`python -m attention_attn_fwd_04_amd.build`.
"""
from .binding import (AttnError, attn_check_args, attn_fwd, attn_pruned_terms,  # noqa: F401
                      attn_release, attn_rope_apply, attn_window_table, strerror)

__all__ = ["AttnError", "attn_fwd", "attn_rope_apply", "attn_window_table", "attn_pruned_terms",
           "attn_check_args", "attn_release", "strerror"]
