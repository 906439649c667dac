"""Oracle for tree-masked verification attention (test infrastructure only).

"Technical analysis of EAGLE-4", section "EAGLE-4 verification trees and the
harness": to score all branches in one target pass, a custom attention mask lets
every token attend to the shared prefix, to its ancestors and to itself, while
siblings and tokens of other branches stay hidden.  "EAGLE" study notes, section
"3. Verify", name the same Medusa-style tree attention.

What is computed, for sequence b, query head h and tree node i < n_nodes[b]
(readings: scale 1/sqrt(D) with the natural exponential; query head h reads KV
head h // (Hq // Hkv); tree K/V are per-node tensors separate from the prefix):

    keys   = prefix keys 0..L_b-1  ++  tree keys of the nodes on i's root path
    s_j    = (q . k_j) * scale
    p_j    = exp(s_j - max s) / sum_j exp(s_j - max s)
    out    = sum_j p_j v_j,     lse = max s + log sum_j exp(s_j - max s)

The mask is built explicitly, row by row, from parent-pointer walks; the softmax
is the naive two-pass one.  Everything is float64 on the exact upcast of the
inputs.
"""

import numpy as np

from .tree import path_to_root


def tree_mask(parent_row, n, L):
    """Boolean visibility matrix [n][L + n]: prefix columns first, then tree nodes.

    Row i sees every prefix column and the tree columns of the nodes met when
    walking from i up to the root (i itself and the root included).
    """
    mask = np.zeros((n, L + n), dtype=bool)
    mask[:, :L] = True
    for i in range(n):
        for j in path_to_root(parent_row, i):
            mask[i, L + j] = True
    return mask


def _attend(qrows, keys, values, mask_rows, scale):
    """Masked softmax attention of each query row over all key rows, in float64."""
    s = (qrows @ keys.T) * scale
    s = np.where(mask_rows, s, -np.inf)
    mx = s.max(axis=1, keepdims=True)
    e = np.exp(s - mx)
    tot = e.sum(axis=1, keepdims=True)
    out = (e / tot) @ values
    lse = mx[:, 0] + np.log(tot[:, 0])
    return out, lse


def tree_verify_attn(q, k_tree, v_tree, k_prefix, v_prefix, prefix_offsets, parent, n_nodes,
                     scale=None, batches=None):
    """Tree verification attention for every (sequence, head, node).

    q         [B][n_max][Hq][D]      k_tree, v_tree   [B][n_max][Hkv][D]
    k_prefix, v_prefix [sum_b L_b][Hkv][D] packed, sequence b at rows
    prefix_offsets[b] .. prefix_offsets[b+1]-1.   parent [B][n_max], n_nodes [B].

    Returns (out float64 [B][n_max][Hq][D], lse float64 [B][n_max][Hq]); padding
    nodes hold 0.  ``batches`` restricts the work to a subset of sequences.
    """
    q = np.asarray(q)
    B, n_max, Hq, D = q.shape
    Hkv = k_tree.shape[2]
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    out = np.zeros((B, n_max, Hq, D), dtype=np.float64)
    lse = np.zeros((B, n_max, Hq), dtype=np.float64)
    for b in (range(B) if batches is None else batches):
        n = int(n_nodes[b])
        off0, off1 = int(prefix_offsets[b]), int(prefix_offsets[b + 1])
        L = off1 - off0
        mask = tree_mask(parent[b], n, L)
        for g in range(Hkv):
            keys = np.concatenate([k_prefix[off0:off1, g, :], k_tree[b, :n, g, :]]).astype(np.float64)
            vals = np.concatenate([v_prefix[off0:off1, g, :], v_tree[b, :n, g, :]]).astype(np.float64)
            for hh in range(G):
                h = g * G + hh
                o, l = _attend(q[b, :n, h, :].astype(np.float64), keys, vals, mask, scale)
                out[b, :n, h, :] = o
                lse[b, :n, h] = l
    return out, lse


def tree_verify_attn_one(q, k_tree, v_tree, k_prefix, v_prefix, prefix_offsets, parent, b, h, i,
                         scale=None):
    """One output row (sequence b, query head h, node i); same arithmetic as above.

    Used to check sampled outputs of workloads too large to recompute in full.
    """
    D = q.shape[3]
    G = q.shape[2] // k_tree.shape[2]
    g = h // G
    if scale is None:
        scale = 1.0 / np.sqrt(D)
    off0, off1 = int(prefix_offsets[b]), int(prefix_offsets[b + 1])
    path = sorted(path_to_root(parent[b], i))
    keys = np.concatenate([k_prefix[off0:off1, g, :], k_tree[b, path, g, :]]).astype(np.float64)
    vals = np.concatenate([v_prefix[off0:off1, g, :], v_tree[b, path, g, :]]).astype(np.float64)
    mask = np.ones((1, keys.shape[0]), dtype=bool)
    o, l = _attend(q[b, i, h, :][None, :].astype(np.float64), keys, vals, mask, scale)
    return o[0], l[0]
