"""MI355X (gfx950) tree-verify MLA attention: a C-ABI HIP library plus a thin binding.

The library (csrc/verify_attn.hip, declared in include/verify_attn.h) does all
of the work; ``binding`` only marshals torch tensors into its C calls.
"""
from .binding import (  # noqa: F401
    VaPlan,
    VerifyAttnError,
    load_library,
    verify_attn,
    verify_attn_build_tree,
    verify_attn_build_tree_rows,
    verify_attn_check_tree,
    verify_attn_compact,
    verify_attn_error_string,
    verify_attn_forward_static,
    verify_attn_gather_rows,
    verify_attn_permute_rows,
    verify_attn_stream_read,
    verify_attn_plan,
    verify_attn_read_status,
    verify_attn_reduce,
    verify_attn_run,
    workspace_for,
)
