"""treeverify: EAGLE-style draft-tree verification on AMD MI355X (gfx950).

The product is libtreeverify.so (C ABI in include/treeverify.h) with the calls of
the verification pass -- tree_build, tree_expand_rerank, tree_verify_attn,
tree_accept -- plus tree_accept_stochastic (rejection-sampling acceptance),
tree_kv_compact (the accepted continuation into the KV cache), tree_draft_continue
(the per-level stop of drafting) and tree_candidate_logits (the draft model's
low-rank candidate head),
and this thin binding that passes torch tensors' device pointers and torch's current
stream to it.
"""

from ._lib import TreeVerifyError, lib, EXPORTS, LIB_PATH
from .ops import (abi_version, tree_build, expand_workspace, ExpandOutputs, tree_expand_rerank,
                  attn_workspace, attn_plan, tree_verify_attn, tree_verify_attn_noalloc,
                  tree_accept, tree_kv_compact,
                  tree_accept_stochastic, tree_draft_continue, tree_candidate_logits,
                  budget_thresholds, cost_lookup)

__all__ = ["TreeVerifyError", "lib", "EXPORTS", "LIB_PATH", "abi_version", "tree_build",
           "expand_workspace", "ExpandOutputs", "tree_expand_rerank", "attn_workspace", "attn_plan",
           "tree_verify_attn", "tree_verify_attn_noalloc", "tree_accept", "tree_kv_compact", "tree_accept_stochastic",
           "tree_draft_continue", "tree_candidate_logits", "budget_thresholds",
           "cost_lookup"]
