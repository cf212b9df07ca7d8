"""MFA decode attention for MI355X (gfx950): a C-ABI HIP library plus a thin
PyTorch binding.  Importing this package does not load the library; the first
call does, and fails loudly if it has not been built."""

from .binding import (
    decode_desc,
    mfa_decode_attention,
    mfa_decode_attention_gqa,
    mfa_decode_attention_mtp,
    mfa_decode_attention_phase,
    mfa_decode_attention_noalloc,
    mfa_decode_plan_splits,
    mfa_decode_workspace_size,
    mfa_kv_append,
    mfa_query_proj,
    mfa_sparse_attention,
    mfa_sparse_select,
    mfa_sparse_summarize,
    mfa_sparse_summarize_new,
    mfa_stream_read,
    V_LAYOUTS,
)

__all__ = [
    "decode_desc",
    "mfa_decode_attention",
    "mfa_decode_attention_gqa",
    "mfa_decode_attention_mtp",
    "mfa_decode_attention_phase",
    "mfa_decode_attention_noalloc",
    "mfa_decode_plan_splits",
    "mfa_decode_workspace_size",
    "mfa_kv_append",
    "mfa_query_proj",
    "mfa_sparse_attention",
    "mfa_sparse_select",
    "mfa_sparse_summarize",
    "mfa_sparse_summarize_new",
    "mfa_stream_read",
    "V_LAYOUTS",
]
