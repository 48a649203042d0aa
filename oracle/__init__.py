"""Plain fp64 CPU oracle for tree-verify MLA-absorb attention and post-accept KV compaction.

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the tests, the smoke check and the benchmark's CPU
baseline may import this package.  It shares no code with the HIP library and imports nothing
from it; the two meet only in the seeded arrays of the ``synth`` module.

Everything is written out from its definition, in float64, with no blocking or fusion:

* ``verify_attn``   -- masked softmax attention in the absorbed MLA form.
* ``compact_kv``    -- the out-of-place gather of the kept tree rows into the prefix.
* ``tree_accept``   -- the greedy walk that picks the accepted path (the rows to keep).
* ``tree_build``    -- the best-first expansion of the drafter's top-k into the draft tree.
* ``append_tree_kv`` -- the tree's cache rows: RMSNorm of the latent part, NeoX rotation of the
  rotary part at each node's position, rounded to bf16, written at the tree's offset.

Every function is pinned by the CPU tests (brute force over all small trees, causal attention
for a chain, per-path causal attention, closed forms, lse merge, equivariances, the absorb
identity, the race example, and for acceptance: a chain closed form, the deepest-consistent-node
formulation, and token-for-token agreement with autoregressive greedy decoding).
"""
from .verify import (  # noqa: F401
    DEFAULT_SCALE,
    ancestor_or_self,
    bf16_bits_to_f64,
    masked_softmax_attention,
    scores_absorbed,
    verify_attn,
    verify_attn_f64,
    verify_attn_ragged,
    verify_attn_stream,
    visibility,
)
from .compact import compact_kv, compact_kv_ragged, validate_keep  # noqa: F401
from .accept import tree_accept, tree_accept_streams, validate_parents  # noqa: F401
from .build import tree_build  # noqa: F401
from .append import append_tree_kv, bf16_round_bits, rms_norm, rope_neox, tree_depths, tree_rows  # noqa: F401
