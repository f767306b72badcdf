"""MI355X (gfx950) multi-row speculative-verification decode attention.

The compute runs in the HIP library lib/libverify_attn.so; this package only
marshals arguments to its C ABI (include/verify_attn.h).  Loading happens on
first use and raises if the library has not been built.
"""
from ._binding import (  # noqa: F401
    VAError, Plan, verify_attn_plan, verify_attn_plan_query, verify_attn_plan_split_range,
    verify_attn_split, verify_attn_combine, verify_attn_split_state, verify_attn_combine_state, pack_state,
    verify_attn_split_append, verify_attn_split_append_state, verify_attn_noalloc,
    NOALLOC_WORKSPACE_BYTES,
    swa_ring_write, verify_kv_write, verify_attn, workspace_for,
    library_path, load_library, MASKS, KV_FORMATS,
    sample_params, sample_workspace_bytes, sample_workspace_for, va_sample, va_accept, va_sample_accept,
    PURPOSE_TARGET, PURPOSE_ACCEPT, PURPOSE_RESIDUAL, va_read_probe,
)
