"""Oracle for greedy longest-accepted-path acceptance (test infrastructure only).

"EAGLE" study notes, section "Well-Calibrated Draft Model": under greedy decoding a
draft token is accepted when it is the target's most likely token at that place.
"What is EAGLE-3 ...", section 4 step 4 "Accepting the sequence", and section 3
("Tree attention" term): the target keeps the longest prefix of the tree whose
tokens all pass.  "Technical analysis of EAGLE-4", section "EAGLE-4 verification
trees and the harness": verification follows the accepted path and then goes on
with the target's own token where the draft stops matching.

Readings: ``target_next[b][i]`` is the target's greedy token after node i (its
prediction for i's children).  Node i >= 1 passes when token[i] equals
target_next[parent[i]]; a node is reachable when every node on its root path
passes (the root always is).  The chosen node is the reachable node of largest
depth, ties to the lowest index.  accept_len is its depth, the path lists its root
path without the root in index order (-1 padded), and the bonus token is the
target's token after it.  An invalid parent array or n_nodes gives -1 everywhere.
"""

import numpy as np

from .tree import validate_parents, path_to_root, STATUS_OK


def node_passes(parent_row, token_row, target_row, j):
    """Greedy test of node j >= 1: its draft token is the target's token after its parent."""
    return int(token_row[j]) == int(target_row[int(parent_row[j])])


def tree_accept(parent, token, target_next, n_nodes):
    """Returns (accept_len int32 [B], best int32 [B], bonus int32 [B], path int32 [B][n_max])."""
    parent = np.asarray(parent)
    B, n_max = parent.shape
    accept_len = np.full(B, -1, dtype=np.int32)
    best = np.full(B, -1, dtype=np.int32)
    bonus = np.full(B, -1, dtype=np.int32)
    path = np.full((B, n_max), -1, dtype=np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        if validate_parents(parent[b], n, n_max) != STATUS_OK:
            continue
        chosen, chosen_depth = 0, 0
        for i in range(n):
            walk = path_to_root(parent[b], i)          # i ... root
            passes = all(node_passes(parent[b], token[b], target_next[b], j) for j in walk[:-1])
            d = len(walk) - 1
            if passes and d > chosen_depth:            # strict: equal depth keeps the lower index
                chosen, chosen_depth = i, d
        walk = sorted(path_to_root(parent[b], chosen))[1:]
        accept_len[b] = chosen_depth
        best[b] = chosen
        bonus[b] = int(target_next[b, chosen])
        path[b, :len(walk)] = walk
    return accept_len, best, bonus, path
