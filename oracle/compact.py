"""Oracle for KV compaction after acceptance (test infrastructure only).

"Technical analysis of EAGLE-4", section "EAGLE-4 verification trees and the
harness": after verification the harness keeps the accepted continuation, frees the
draft's rejected KV-cache entries and starts the next round.

Readings: the continuation the next round attends to is the root (node 0: the
target's last token, queried in this pass but not yet cached) followed by the
accepted path, root to leaf.  Row j of a sequence's destination receives the K and
V of node 0 for j = 0 and of path[j-1] for 1 <= j <= accept_len, for every KV head;
the rest of the tree is simply not copied (that is the freeing: the tree buffers are
reused by the next round).  A sequence whose accept_len is negative (a tree that
tree_accept rejected) copies nothing.  Destination rows outside the destination
buffer are skipped.
"""

import numpy as np


def kept_nodes(path_row, accept_len):
    """Node indices of the continuation, in destination order: the root, then the path."""
    if accept_len < 0:
        return []
    return [0] + [int(path_row[j]) for j in range(accept_len)]


def kv_compact(k_tree, v_tree, path, accept_len, k_dst, v_dst, dst_row):
    """Returns copies of (k_dst, v_dst) with each sequence's continuation written.

    k_tree, v_tree: [B][n_max][Hkv][D]; path int32 [B][n_max]; accept_len int32 [B];
    k_dst, v_dst: [rows][Hkv][D]; dst_row int64 [B] (first destination row)."""
    k_out, v_out = np.array(k_dst, copy=True), np.array(v_dst, copy=True)
    rows = k_out.shape[0]
    n_max = k_tree.shape[1]
    for b in range(k_tree.shape[0]):
        for j, node in enumerate(kept_nodes(path[b], int(accept_len[b]))):
            r = int(dst_row[b]) + j
            if not (0 <= node < n_max) or not (0 <= r < rows):
                continue
            k_out[r] = k_tree[b, node]
            v_out[r] = v_tree[b, node]
    return k_out, v_out
