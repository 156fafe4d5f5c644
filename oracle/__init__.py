"""fp64 CPU oracle for layout-grounded tree attention.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and
the CPU-baseline leg of ``bench.py`` may import anything from here.  The
library (``tree_structured_attention_amd``) never calls it and shares no code
with it.
"""
from .tree_attn_oracle import (  # noqa: F401
    ancestor_mask_page,
    masked_attention,
    masked_attention_backward,
    prefill,
    prefill_backward,
    prefill_backward_sampled,
    decode,
    verify,
    plan_prefill,
    plan_decode,
    plan_verify,
    depth,
    tree_ancestor_mask,
    lse_merge,
)
from .draft_oracle import (  # noqa: F401,E402
    draft_candidates,
    prefix_tree,
    draft_tree,
    tree_accept,
    chain_accept,
)
from .kv_pool_oracle import KVPool, PoolError, gather as gather_paged  # noqa: F401,E402
