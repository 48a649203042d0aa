"""MI355X (gfx950) tree-verify MLA-absorb attention, greedy tree acceptance and race-free KV
compaction.

The compute lives in ``libddtree.so`` (C ABI, ``include/ddtree.h``); this package only binds it::

    from tree_verify_mla_absorb_amd import verify_attn, verify_attn_ex, tree_accept, accept_compact, compact_kv
"""
from ._lib import (  # noqa: F401
    NOALLOC_SCRATCH_BYTES,
    DDTreeError,
    accept_compact,
    accept_compact_layers,
    accept_compact_ragged,
    append_tree_kv,
    compact_kv,
    compact_kv_layers,
    compact_kv_ragged,
    num_splits,
    status_string,
    tree_accept,
    tree_build,
    verify_attn,
    verify_attn_ex,
    verify_attn_noalloc,
    verify_attn_ragged,
    version,
    workspace_size,
)
