"""MI355X-native causal sparse-attention prefill (block gating, sliding
window, token top-k, GQA, sink) behind the C ABI of include/sparse_attn.h.

Importing this package does not load the shared library; the first call of
an entry point does, and raises if it has not been built.
"""
from .binding import (  # noqa: F401
    EXPORTS, SA_BF16, SA_F32, SA_FP8, Params, SparseAttnCfg, SparseAttnError, Workspace, backward,
    block_pool, forward, load_library, params_for, sparse_attn_block_pool, sparse_attn_fwd,
    sparse_attn_fwd_noalloc,
    sparse_attn_bwd_workspace_bytes,
    sparse_attn_check_far_lists, sparse_attn_set_checks,
    sparse_attn_set_timing, sparse_attn_stage_times, sparse_attn_strerror,
    sparse_attn_workspace_bytes,
)
