"""Oracle for the draft-tree structure (test infrastructure; see the package docstring).

A draft tree is a parent array: node 0 is the root (the target's last token, which
verification also queries), ``parent[0] == -1`` and ``0 <= parent[i] < i`` for
every other node.  "EAGLE" study notes, section "1. EAGLE pipeline / Draft Model",
describe the draft as a tree of depth m with more than m tokens; "Technical
analysis of EAGLE-4", section "EAGLE-4 verification trees and the harness", says
what a node may see: the shared prefix, its ancestors and itself.  The ancestor
set of node i is therefore the set of nodes on the walk i -> parent[i] -> ... -> 0,
computed here by literally walking the parent pointers.
"""

import numpy as np

STATUS_OK = 0
STATUS_BAD_PARENT = 1     # parent[0] != -1, or parent[i] < -1, or parent[i] >= i
STATUS_SECOND_ROOT = 2    # parent[i] == -1 for some i >= 1
STATUS_BAD_N = 3          # n_nodes outside [1, n_max]
STATUS_NONFINITE = 4      # a draft-logit row holds NaN or +-Inf (expansion only)


def validate_parents(parent_row, n, n_max):
    """Status of one sequence's parent array (0 = valid).

    The first offending node in index order decides the code, so the result is
    unique.  ``n`` outside [1, n_max] is reported before anything else.
    """
    if n < 1 or n > n_max:
        return STATUS_BAD_N
    for i in range(n):
        p = int(parent_row[i])
        if i == 0:
            if p != -1:
                return STATUS_BAD_PARENT
            continue
        if p == -1:
            return STATUS_SECOND_ROOT
        if p < -1 or p >= i:
            return STATUS_BAD_PARENT
    return STATUS_OK


def path_to_root(parent_row, i):
    """Nodes on the walk from node i up to the root, i first, root last."""
    path = []
    j = int(i)
    while j != -1:
        path.append(j)
        j = int(parent_row[j])
    return path


def tree_build(parent, n_nodes, prefix_len=None):
    """Depth, ancestor bitset and position of every node of every sequence.

    parent     int [B][n_max]
    n_nodes    int [B]
    prefix_len int [B] or None (None means a prefix of length 0)

    Returns (anc uint64 [B][n_max], depth int32 [B][n_max], pos int32 [B][n_max],
    status int32 [B]).  For node i < n_nodes[b]: depth = number of parent steps to
    the root; bit j of anc is set iff j is on the walk from i to the root (i and
    the root included); pos = prefix length + depth, the position the caller gives
    the node when it applies its position encoding.  Padding entries and every
    entry of a sequence with a nonzero status hold anc 0, depth -1, pos -1.
    """
    parent = np.asarray(parent)
    B, n_max = parent.shape
    anc = np.zeros((B, n_max), dtype=np.uint64)
    depth = np.full((B, n_max), -1, dtype=np.int32)
    pos = np.full((B, n_max), -1, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    for b in range(B):
        n = int(n_nodes[b])
        st = validate_parents(parent[b], n, n_max)
        status[b] = st
        if st != STATUS_OK:
            continue
        L = 0 if prefix_len is None else int(prefix_len[b])
        for i in range(n):
            walk = path_to_root(parent[b], i)
            bits = 0
            for j in walk:
                bits |= 1 << j
            anc[b, i] = np.uint64(bits)
            depth[b, i] = len(walk) - 1
            pos[b, i] = L + len(walk) - 1
    return anc, depth, pos, status
