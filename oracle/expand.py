"""Oracle for EAGLE-2 dynamic draft-tree expansion and reranking (test infrastructure only).

"EAGLE" study notes:
* section "Well-Calibrated Draft Model": a draft token's confidence is the softmax of
  the draft logits, and it tracks the token's acceptance rate well;
* section "Expansion of tree": rejecting a token cuts its whole path, so a node's
  value is its global acceptance, the product of the confidences along its path from
  the root; expansion keeps the top-k;
* section "Reranking Nodes": after expanding, keep the m nodes of largest global
  acceptance over all nodes generated.

Readings taken where the pages leave a step open:
* Values are ranked through their logarithm (log is monotone): a node's score is
  the sum of the log-confidences on its path.  The log-sum-exp of a logit row is
  computed in float64 (max-shifted), rounded once to float32; a child's score is
  fl32(parent_score + fl32(logit - lse32)).  This fixes every score bit, so the
  kept set is reproducible exactly by any implementation doing the same float32
  operations.  Summation order can move lse64 only in its last bits; a row whose
  lse64 lies within 1e-12 (relative) of a float32 rounding midpoint is flagged
  ``indeterminate`` instead of trusted.
* Each expanded node gets the k tokens of largest logit, ties to the lower id.
* The frontier of each level is the k best children of that level by (score
  descending, creation ascending); logit row r of the next level belongs to the
  frontier node of rank r.  Children are created in the order (frontier rank,
  top-k rank).
* Rerank keeps the m-1 best of all generated children by the same order, plus the
  root (m counts the root).  Scores never increase along a path and ties favour
  the earlier-created parent, so the kept set always contains its ancestors.
* Output order: the root, then the kept nodes by (depth, creation), parents remapped.
* Errors surface at the level where they occur, as a caller calling level by level
  sees them: a non-finite logit row fails its sequence at that level (earlier levels
  keep their reported frontier), a kept count m outside [1, n_max] at the last level.
"""

from typing import NamedTuple

import numpy as np

from .tree import STATUS_OK, STATUS_BAD_N, STATUS_NONFINITE


class ExpandResult(NamedTuple):
    parent: np.ndarray           # int32 [B][n_max]
    token: np.ndarray            # int32 [B][n_max]
    score: np.ndarray            # float32 [B][n_max]
    n_nodes: np.ndarray          # int32 [B]
    status: np.ndarray           # int32 [B]
    frontier_tokens: list        # per level: int32 [B][k], tokens of the frontier by rank
    indeterminate: np.ndarray    # bool [B]


def _near_fp32_midpoint(x64):
    """True when float64 x lies within 1e-12 (relative) of a float32 rounding midpoint."""
    f = np.float32(x64)
    lo = np.nextafter(f, np.float32(-np.inf))
    hi = np.nextafter(f, np.float32(np.inf))
    mids = ((np.float64(f) + np.float64(lo)) / 2.0, (np.float64(f) + np.float64(hi)) / 2.0)
    return min(abs(x64 - mm) for mm in mids) <= 1e-12 * abs(x64)


def row_log_normaliser(row):
    """(lse32, lse64) of one float32 logit row: max-shifted log-sum-exp in float64."""
    M = np.float64(row.max())
    lse64 = M + np.log(np.sum(np.exp(row.astype(np.float64) - M)))
    return np.float32(lse64), lse64


def rank_key(score, creation):
    """Sort key putting the better node first: larger score, then earlier creation."""
    return (-float(score), int(creation))


def row_topk(row, k):
    """Ids of the k largest logits, ties to the lower id, best first."""
    return np.argsort(-row, kind="stable")[:k]


def budget_cut(ranked_scores, budget_log):
    """Candidates kept by the verify budget: the leading run of the best-first ranked
    candidates whose score (log value) exceeds the bar for their place: candidate j
    (1-based) passes when score_j > budget_log[j] (float32), and the first failure
    ends the run.  "Technical analysis of EAGLE-4", section "EAGLE-4 verification
    trees and the harness": candidates are added while the gain in cumulative
    probability per unit of measured verification cost stays above a threshold."""
    n = 0
    for j, sc in enumerate(ranked_scores, start=1):
        if not np.float32(sc) > np.float32(budget_log[j]):
            break
        n = j
    return n


def expand_rerank(logits_steps, k, m, root_token, n_max=64, budget_log=None):
    """Build each sequence's dynamic draft tree level by level, then rerank it.

    logits_steps  list of S float32 arrays; level s (1-based) has shape
                  [B][1 if s == 1 else k][V]; row r is the frontier node of rank r.
    k             children per expanded node and frontier width.
    m             nodes kept including the root: int, or int array [B].
    root_token    int [B], the token of each root.
    budget_log    optional float32 [n_max]: after the best m-1 are chosen, only the
                  leading run passing budget_cut is kept.
    """
    S = len(logits_steps)
    B = logits_steps[0].shape[0]
    m_arr = np.broadcast_to(np.asarray(m, dtype=np.int64), (B,))
    parent = np.full((B, n_max), -1, dtype=np.int32)
    token = np.full((B, n_max), -1, dtype=np.int32)
    score = np.zeros((B, n_max), dtype=np.float32)
    n_nodes = np.zeros(B, dtype=np.int32)
    status = np.zeros(B, dtype=np.int32)
    indeterminate = np.zeros(B, dtype=bool)
    frontier_tokens = [np.full((B, k), -1, dtype=np.int32) for _ in range(S)]

    for b in range(B):
        # pool entries: (parent pool index or -1 for the root, token, score, depth)
        pool = []
        frontier = [(-1, np.float32(0.0), 0)]      # (pool index, score, depth) of the root
        bad = False
        for s in range(S):
            rows = logits_steps[s][b]
            children = []
            for f, (fidx, fscore, fdepth) in enumerate(frontier):
                row = np.asarray(rows[f], dtype=np.float32)
                if not np.all(np.isfinite(row)):
                    bad = True
                    break
                lse32, lse64 = row_log_normaliser(row)
                if _near_fp32_midpoint(lse64):
                    indeterminate[b] = True
                for t in row_topk(row, k):
                    logp = np.float32(row[t] - lse32)
                    sc = np.float32(fscore + logp)
                    children.append((fidx, int(t), sc, fdepth + 1, len(pool) + len(children)))
            if bad:
                break                                # this level and later report no frontier
            if s == S - 1 and not 1 <= int(m_arr[b]) <= n_max:
                break                                # the kept count is checked at the last level
            pool.extend(c[:4] for c in children)
            ranked = sorted(children, key=lambda c: rank_key(c[2], c[4]))[:k]
            frontier = [(c[4], c[2], c[3]) for c in ranked]
            frontier_tokens[s][b, :len(ranked)] = [c[1] for c in ranked]
        if bad:
            status[b] = STATUS_NONFINITE
            continue
        mb = int(m_arr[b])
        if not 1 <= mb <= n_max:
            status[b] = STATUS_BAD_N
            continue
        order = sorted(range(len(pool)), key=lambda i: rank_key(pool[i][2], i))
        kept = order[:mb - 1]
        if budget_log is not None:
            kept = kept[:budget_cut([pool[i][2] for i in kept], budget_log)]
        kept.sort(key=lambda i: (pool[i][3], i))
        where = {i: j + 1 for j, i in enumerate(kept)}
        parent[b, 0] = -1
        token[b, 0] = int(root_token[b])
        score[b, 0] = np.float32(0.0)
        for j, i in enumerate(kept):
            pidx, tok, sc, _ = pool[i]
            parent[b, j + 1] = 0 if pidx == -1 else where[pidx]
            token[b, j + 1] = tok
            score[b, j + 1] = sc
        n_nodes[b] = 1 + len(kept)
        status[b] = STATUS_OK
    return ExpandResult(parent, token, score, n_nodes, status, frontier_tokens, indeterminate)


def draft_continue(logits_steps, k, m, budget_log=None, n_max=64):
    """The harness's per-level stop.  "Technical analysis of EAGLE-4", section "EAGLE-4
    verification trees and the harness": at each draft level the gain in cumulative
    probability per unit of measured marginal verification cost decides whether the
    tree is drafted further; drafting stops once it falls below the threshold.

    Reading: after level s, let c be the best child that level created (its
    frontier node of rank 0) and p its place in the whole pool ranked best first by
    (score descending, creation ascending).  Drafting goes on when c
    would be kept by the final rerank if drafting stopped now: p <= m - 1 and the
    places 1..p all pass the verify budget (budget_cut).  A deeper node scores no
    better than its parent and is created after it, so it ranks after c; when c is
    not kept no later level can add a kept node, and stopping leaves the final tree
    unchanged.

    Returns int32 [S][B]: more[s][b] after level s + 1 (0 for a failed sequence and
    for every level from the failing one on).  The levels are expanded with the same
    arithmetic as expand_rerank."""
    S = len(logits_steps)
    B = logits_steps[0].shape[0]
    m_arr = np.broadcast_to(np.asarray(m, dtype=np.int64), (B,))
    more = np.zeros((S, B), dtype=np.int32)
    for b in range(B):
        mb = int(m_arr[b])
        pool = []                                  # (score, creation) of every child
        frontier = [(np.float32(0.0),)]            # scores of the frontier, best first
        for s in range(S):
            rows = logits_steps[s][b]
            children = []
            bad = False
            for f, (fscore,) in enumerate(frontier):
                row = np.asarray(rows[f], dtype=np.float32)
                if not np.all(np.isfinite(row)):
                    bad = True
                    break
                lse32, _ = row_log_normaliser(row)
                for t in row_topk(row, k):
                    sc = np.float32(fscore + np.float32(row[t] - lse32))
                    children.append((sc, len(pool) + len(children)))
            if bad:
                break
            pool.extend(children)
            ranked = sorted(children, key=lambda c: rank_key(c[0], c[1]))
            frontier = [(c[0],) for c in ranked[:k]]
            best = ranked[0]
            order = sorted(pool, key=lambda c: rank_key(c[0], c[1]))
            p = 1 + order.index(best)
            run = p
            if budget_log is not None:
                # one bar per place up to n_max - 1; a place past them is never kept (m <= n_max)
                run = budget_cut([c[0] for c in order[:p]], budget_log) if p < len(budget_log) else 0
            more[s, b] = int(1 <= mb <= n_max and best_child_kept(p, mb, run))
    return more


def best_child_kept(place, m, run):
    """The level's best child, at `place` (1-based) in the best-first pool, is kept by
    the final rerank: it is among the m - 1 candidates and the budget's leading run of
    passing places (`run` long, counted over places 1..place) reaches it."""
    return place <= m - 1 and run == place
