"""Oracle for the low-rank candidate head (test infrastructure only).

"Technical analysis of EAGLE-4", section "EAGLE-4 architecture": a low-rank candidate
head first scores the vocabulary in a smaller representation and then computes full
logits only for the selected candidates, to cut the cost of next-token prediction.

Readings taken where the page leaves a step open:
* The smaller representation is a rank-r factorisation of the LM head: z = A h
  (A: [r][d]) and a low-rank score s_v = Bm[v] . z for every token (Bm: [V][r]); the
  full logit is l_v = W[v] . h (W: [V][d]).  h, A, Bm, W are bf16.
* The selected candidates are the C tokens of largest s, ties to the lower id.
* The head's output is one logit row per draft row: the exact logit at the C
  candidates, the low-rank score everywhere else.  It feeds the dynamic-tree expansion
  unchanged (its log-sum-exp, top-k and scores), so the confidence of a candidate is
  normalised over the whole vocabulary with low-rank scores standing in for the rest.
* Every dot product is summed in float64 from the exact bf16 values and rounded once
  to float32 (z too, before it is used): selection and output bits are then fixed.
  A float64 sum depends on its order only in its last bits, so a result within 1e-12
  (relative) of a float32 rounding midpoint, but not on it, is flagged indeterminate
  instead of trusted.  A sum exactly on a midpoint is one the float64 sum carried
  exactly (its terms have at most 32 significant bits), so both sides round it to
  even.
"""

import numpy as np


def _fp32_near_midpoint(x64):
    """Elementwise: float64 values within 1e-12 (relative) of a float32 rounding midpoint,
    and not exactly on it."""
    x64 = np.asarray(x64, dtype=np.float64)
    f = x64.astype(np.float32)
    lo = np.nextafter(f, np.float32(-np.inf)).astype(np.float64)
    hi = np.nextafter(f, np.float32(np.inf)).astype(np.float64)
    f64 = f.astype(np.float64)
    d = np.minimum(np.abs(x64 - (f64 + lo) / 2), np.abs(x64 - (f64 + hi) / 2))
    return (d > 0) & (d <= 1e-12 * np.abs(x64))


def dot_rows(M, x):
    """float64 M @ x for float32-exact inputs (bf16 upcast): float64 result."""
    return np.asarray(M, dtype=np.float64) @ np.asarray(x, dtype=np.float64)


def top_candidates(scores, C):
    """Ids of the C largest float32 scores, ties to the lower id, best first."""
    return np.argsort(-np.asarray(scores, dtype=np.float32), kind="stable")[:C]


def candidate_logits(h, A, Bm, W, C):
    """h [rows][d], A [r][d], Bm [V][r], W [V][d] (float32 arrays holding bf16 values).

    Returns (logits float32 [rows][V], cand int32 [rows][C], indeterminate bool
    [rows][V], cand_indeterminate bool [rows]): an entry is indeterminate when its own
    float32 value is (a candidate's exact logit or a low-rank score), and every entry
    of a row whose z is; a row's candidate list is indeterminate when a low-rank score
    among its C + 1 best is (or its z)."""
    h = np.asarray(h, dtype=np.float32)
    rows = h.shape[0]
    V = W.shape[0]
    logits = np.empty((rows, V), dtype=np.float32)
    cand = np.empty((rows, C), dtype=np.int32)
    indet = np.zeros((rows, V), dtype=bool)
    cand_indet = np.zeros(rows, dtype=bool)
    for i in range(rows):
        z64 = dot_rows(A, h[i])
        z = z64.astype(np.float32)
        s64 = dot_rows(Bm, z)
        s = s64.astype(np.float32)
        c = top_candidates(s, C)
        l64 = dot_rows(W[c], h[i])
        row = s.copy()
        row[c] = l64.astype(np.float32)
        logits[i] = row
        cand[i] = c
        sflag = _fp32_near_midpoint(s64)
        zflag = bool(_fp32_near_midpoint(z64).any())
        cand_indet[i] = zflag or bool(sflag[top_candidates(s, min(C + 1, V))].any())
        flag = sflag.copy()
        flag[c] = _fp32_near_midpoint(l64)
        indet[i] = True if zflag else flag
    return logits, cand, indet, cand_indet
