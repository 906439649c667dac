"""Oracle for stochastic (rejection-sampling) tree acceptance (test infrastructure only).

"EAGLE" study notes, section "Well-Calibrated Draft Model": a draft token x is
accepted with rate min(1, P_target(x) / P_draft(x)) under random sampling (always
when the target finds it at least as likely as the draft did, else in proportion).
"What is EAGLE-3 ...", section 4 steps 3-4: a rejected token is replaced by the
target's own token, sampled from a corrected distribution, and the longest prefix
of the tree whose tokens all pass is kept.  "Technical analysis of EAGLE-4", section
"EAGLE-4 verification trees and the harness": rejection sampling accepts the longest
matching prefix, so the output distribution does not change.

The pages give the single-candidate rule only.  Readings for a tree (each one stated
so that the GPU path can take the same decisions in the same precision):
* p_target[b][i] (float32 [V]) is the target's next-token distribution after node
  i's root path; q_draft[b][i] the draft's distribution that proposed i's children.
* The walk starts at the root.  At the current node u the target weights r start as
  p_target[u] and S = sum(r) (float64).  u's children are tried in index order (the
  order expansion created them).  Child c with token x passes when
      u_accept[c] * S * q(x) < r(x)        (float64, left to right)
  i.e. with probability min(1, (r(x)/S) / q(x)); with q(x) == 0 it passes when
  r(x) > 0.  A passing child becomes the current node (fresh r and S from its own
  row).  A failing child turns r into the residual
      r <- max(r - fl32(S) * q, 0)         (float32: product, then difference)
  and S into its float64 sum; the next sibling is tried against that.
* When no child passes (or u is a leaf) the bonus token is the first v whose float64
  running sum of r passes u_bonus * S (the last v of positive weight if rounding
  leaves none); u is the chosen node.
* accept_len, best node, bonus token and path are reported as by greedy acceptance.
  An invalid tree (n_nodes out of range, or anc[0] != 1) gives -1 everywhere.
Sums depend on their order in the last bits; the oracle reports a sequence as
indeterminate when some decision lies within 1e-9 (relative) of its threshold.
"""

import numpy as np

from .tree import validate_parents, STATUS_OK

_EPS = 1e-9


def _sum64(r):
    return float(np.sum(r.astype(np.float64)))


def child_passes(u, S, qx, rx):
    """The acceptance test of one candidate; returns (passes, margin relative to rx)."""
    if qx == 0.0:
        return rx > 0.0, 1.0
    lhs = float(u) * S * float(qx)
    return lhs < float(rx), abs(lhs - float(rx)) / max(abs(float(rx)), 1e-300)


def residual(r, S, q):
    """r <- max(r - fl32(S) * q, 0) in float32, product then difference."""
    prod = np.float32(S) * q.astype(np.float32)
    return np.maximum(r.astype(np.float32) - prod, np.float32(0))


def sample(r, S, u):
    """First index whose float64 running sum passes u * S (the last index of positive
    weight when rounding leaves none); returns (index, margin)."""
    target = float(u) * S
    cum = np.cumsum(r.astype(np.float64))
    idx = int(np.searchsorted(cum, target, side="right"))
    if idx >= len(r):
        pos = np.nonzero(r > 0)[0]
        return (int(pos[-1]) if len(pos) else len(r) - 1), 0.0
    margin = abs(cum[idx] - target) / max(S, 1e-300)
    if idx > 0:
        margin = min(margin, abs(cum[idx - 1] - target) / max(S, 1e-300))
    return idx, margin


def children_of(parent_row, n, u):
    return [c for c in range(1, n) if int(parent_row[c]) == u]


def tree_accept_stochastic(parent, token, n_nodes, p_target, q_draft, u_accept, u_bonus):
    """Returns (accept_len, best, bonus, path, indeterminate) as int32 arrays + bool [B]."""
    parent = np.asarray(parent)
    B, n_max = parent.shape
    accept_len = np.full(B, -1, np.int32)
    best = np.full(B, -1, np.int32)
    bonus = np.full(B, -1, np.int32)
    path = np.full((B, n_max), -1, np.int32)
    indet = np.zeros(B, bool)
    for b in range(B):
        n = int(n_nodes[b])
        if validate_parents(parent[b], n, n_max) != STATUS_OK:
            continue
        u, depth, chain = 0, 0, []
        r = p_target[b, 0].astype(np.float32)
        S = _sum64(r)
        while True:
            moved = False
            for c in children_of(parent[b], n, u):
                x = int(token[b, c])
                ok, margin = child_passes(u_accept[b, c], S, q_draft[b, u][x], r[x])
                if margin < _EPS:
                    indet[b] = True
                if ok:
                    u, depth, moved = c, depth + 1, True
                    chain.append(c)
                    r = p_target[b, c].astype(np.float32)
                    S = _sum64(r)
                    break
                r = residual(r, S, q_draft[b, u])
                S = _sum64(r)
            if not moved:
                break
        v, margin = sample(r, S, u_bonus[b])
        if margin < _EPS:
            indet[b] = True
        accept_len[b], best[b], bonus[b] = depth, u, v
        for j, c in enumerate(sorted(chain)):
            path[b, j] = c
    return accept_len, best, bonus, path, indet
