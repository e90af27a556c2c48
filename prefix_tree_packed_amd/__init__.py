"""Prefix-tree-packed attention and the Basal decision for AMD MI355X (gfx950).

The compute lives in libtreeattn.so (C ABI: include/tree_attn.h): a host plan
builder and hand-written HIP kernels. ``prefix_tree_packed_amd.binding`` is the
thin Python binding with the same function names; importing this package does
not load the library, the first binding call does (and raises if it is missing).
"""

from .binding import (  # noqa: F401
    Plan,
    TreeAttnError,
    decision_readout,
    letter_logits,
    load_library,
    readout_mlp,
    readout_mlp_noalloc,
    readout_mlp_workspace_size,
    readout_pack_gate_up,
    readout_workspace_views,
    tree_attn_cache_write,
    tree_attn_forward,
    tree_attn_forward_cached,
    tree_attn_forward_chunked,
    tree_attn_last_error,
    tree_attn_mfma_peak_probe,
    tree_attn_plan,
    tree_attn_plan_destroy,
    tree_attn_plan_export,
    tree_attn_plan_info,
    tree_attn_plan_masks,
    tree_attn_plan_schedule,
    tree_attn_plan_set_max_workgroups,
    tree_attn_plan_upload,
    tree_attn_plan_workgroups,
    tree_attn_rope_cache_write,
    tree_form_batches,
    tree_pack,
    tree_request_cost,
)
