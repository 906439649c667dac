"""Plain, slow CPU oracle for draft-tree verification. TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  The product path (the HIP
library and its Python binding) never imports, calls or falls back to it, and this
package imports nothing from the product path: the two share no code.  The one
thing both sides consume is the seeded input generators in ``synth/``, which hold
none of the method's arithmetic.

Pages this oracle follows (cited by title and section throughout):

* "EAGLE" -- study notes on EAGLE-1/2/3 (s1mplewind astro-blog).  Sections used:
  "1. EAGLE pipeline / Draft Model" (a draft tree of depth m holding more than m
  tokens, built in m draft passes; the depth-3, 10-token example; static trees are
  left-heavy), "3. Verify" (tree attention), "Well-Calibrated Draft Model"
  (confidence is the softmax of the draft logits; greedy acceptance is agreement
  of the most likely tokens), "Expansion of tree" (a node's value is the product
  of the confidences on its root path; keep the top-k), "Reranking Nodes" (keep
  the m nodes of largest value over the whole tree).
* "What is EAGLE-3 and how does it differ from standard speculative decoding?"
  (aivaro.ru Q&A), section 3 "Evolution" (tree attention checks all branches and
  takes the longest accepted sequence) and section 4 "How EAGLE-3 works", step 4
  "Accepting the sequence".
* "Technical analysis of EAGLE-4" (dev48.org translation), section "EAGLE-4
  verification trees and the harness": the attention mask lets every token see
  the shared prefix, its ancestors and itself, hiding siblings and other
  branches; verification follows the accepted path and then continues with the
  target's own token; the harness then keeps the accepted continuation and frees
  the rejected KV-cache entries.

Precision: attention is computed in float64 from the exact float32 upcast of the
inputs (the pages fix no precision).  The tree-expansion scores are the one place
where floating point decides integers (which nodes are kept); there the oracle
takes the decision in the precision the kernel uses, stated in ``expand.py``.

Parity pins: every function here is pinned by ``tests/test_oracle_*.py`` against
closed forms, library routines, brute force or the pages' structural facts; the
pages print no numeric worked example, so no pin compares against printed values.
"""

from .tree import tree_build, validate_parents, path_to_root, STATUS_OK, STATUS_BAD_PARENT, \
    STATUS_SECOND_ROOT, STATUS_BAD_N, STATUS_NONFINITE
from .attention import tree_verify_attn, tree_mask
from .expand import expand_rerank, ExpandResult
from .accept import tree_accept
from .compact import kv_compact, kept_nodes
from .stochastic import tree_accept_stochastic
from .candidates import candidate_logits

__all__ = [
    "tree_build", "validate_parents", "path_to_root", "tree_verify_attn", "tree_mask",
    "expand_rerank", "ExpandResult", "tree_accept", "kv_compact", "kept_nodes",
    "tree_accept_stochastic", "candidate_logits",
    "STATUS_OK", "STATUS_BAD_PARENT", "STATUS_SECOND_ROOT", "STATUS_BAD_N", "STATUS_NONFINITE",
]
