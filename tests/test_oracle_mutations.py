"""Plant plausible mistakes in the oracle (on the CPU) and check that a pin notices.

Each mutation replaces one helper of the oracle through monkeypatch; the pins in
``oracle_pins`` must then fail.  This is what makes the pins worth trusting: a
dropped term, a wrong index, a transposed operand or a flipped tie-break anywhere
in the oracle is caught by at least one of them.
"""

import numpy as np
import pytest

import oracle
import oracle.accept
import oracle.attention
import oracle.candidates
import oracle.compact
import oracle.stochastic
import oracle.expand
import oracle.tree
import oracle_pins


_ORIG_WALK = oracle.tree.path_to_root


def _walk_without_self(parent_row, i):
    return _ORIG_WALK(parent_row, i)[1:]


def _walk_without_root(parent_row, i):
    w = _ORIG_WALK(parent_row, i)
    return w[:-1] if len(w) > 1 else w


def _walk_off_by_one(parent_row, i):
    w = _ORIG_WALK(parent_row, i)
    return [j + 1 if j + 1 < len(parent_row) and j != 0 else j for j in w]


def _mask_with_siblings(parent_row, n, L):
    mask = np.zeros((n, L + n), dtype=bool)
    mask[:, :L] = True
    for i in range(n):
        for j in _ORIG_WALK(parent_row, i):
            mask[i, L + j] = True
            for s in range(1, n):
                if parent_row[s] == parent_row[j] and j != 0:
                    mask[i, L + s] = True
    return mask


def _attend_transposed(qrows, keys, values, mask_rows, scale):
    return _ORIG_ATTEND(qrows, values, keys, mask_rows, scale)


def _attend_no_scale(qrows, keys, values, mask_rows, scale):
    return _ORIG_ATTEND(qrows, keys, values, mask_rows, 1.0)


def _attend_lse_without_max(qrows, keys, values, mask_rows, scale):
    out, lse = _ORIG_ATTEND(qrows, keys, values, mask_rows, scale)
    s = np.where(mask_rows, (qrows @ keys.T) * scale, -np.inf)
    return out, lse - s.max(axis=1)


_ORIG_ATTEND = oracle.attention._attend


def _midpoint_dist(x64):
    """Distance of float64 x to the nearest float32 rounding midpoint."""
    f = np.float32(x64)
    lo = np.float64(np.nextafter(f, np.float32(-np.inf)))
    hi = np.float64(np.nextafter(f, np.float32(np.inf)))
    return min(abs(x64 - (np.float64(f) + lo) / 2), abs(x64 - (np.float64(f) + hi) / 2))

MUTATIONS = {
    "tree: walk drops the node itself": [(oracle.tree, "path_to_root", _walk_without_self)],
    "tree: walk index off by one": [(oracle.tree, "path_to_root", _walk_off_by_one)],
    "attention: root missing from the path": [(oracle.attention, "path_to_root", _walk_without_root)],
    "attention: self missing from the path": [(oracle.attention, "path_to_root", _walk_without_self)],
    "attention: siblings leak into the mask": [(oracle.attention, "tree_mask", _mask_with_siblings)],
    "attention: K and V transposed": [(oracle.attention, "_attend", _attend_transposed)],
    "attention: 1/sqrt(D) scale dropped": [(oracle.attention, "_attend", _attend_no_scale)],
    "attention: lse without the max term": [(oracle.attention, "_attend", _attend_lse_without_max)],
    "expand: top-k ties to the higher id": [
        (oracle.expand, "row_topk", lambda row, k: (len(row) - 1 - np.argsort(-row[::-1], kind="stable"))[:k])],
    "expand: ranking ties to the later node": [
        (oracle.expand, "rank_key", lambda score, creation: (-float(score), -int(creation)))],
    "expand: scores not normalised": [
        (oracle.expand, "row_log_normaliser", lambda row: (np.float32(0.0), 0.0))],
    "expand: ascending score order": [
        (oracle.expand, "rank_key", lambda score, creation: (float(score), int(creation)))],
    "accept: compares with the node's own target": [
        (oracle.accept, "node_passes", lambda par, tok, tgt, j: int(tok[j]) == int(tgt[j]))],
    "accept: walk drops the node itself": [(oracle.accept, "path_to_root", _walk_without_self)],
    "compact: root not kept": [
        (oracle.compact, "kept_nodes", lambda row, n: [] if n < 0 else [int(row[j]) for j in range(n)])],
    "compact: path kept leaf first": [
        (oracle.compact, "kept_nodes", lambda row, n: [] if n < 0 else [0] + [int(row[j]) for j in range(n)][::-1])],
    "stochastic: no residual after a rejection": [
        (oracle.stochastic, "residual", lambda r, S, q: r.astype(np.float32))],
    "stochastic: residual not clamped at zero": [
        (oracle.stochastic, "residual", lambda r, S, q: r.astype(np.float32) - np.float32(S) * q.astype(np.float32))],
    "stochastic: acceptance ratio inverted": [
        (oracle.stochastic, "child_passes", lambda u, S, qx, rx: (float(u) * float(rx) < S * float(qx), 1.0))],
    "stochastic: siblings tried last first": [
        (oracle.stochastic, "children_of", lambda row, n, u: [c for c in range(n - 1, 0, -1) if int(row[c]) == u])],
    "budget: counts every passing candidate": [
        (oracle.expand, "budget_cut", lambda sc, bl: sum(1 for j, x in enumerate(sc, 1) if np.float32(x) > bl[j]))],
    "budget: a tie passes": [
        (oracle.expand, "budget_cut", lambda sc, bl: next((j - 1 for j, x in enumerate(sc, 1) if not np.float32(x) >= bl[j]), len(sc)))],
    "stop: the m - 1 bound taken as strict": [
        (oracle.expand, "best_child_kept", lambda place, m, run: place < m - 1 and run == place)],
    "stop: the verify budget ignored": [
        (oracle.expand, "best_child_kept", lambda place, m, run: place <= m - 1)],
    "candidates: ties to the higher id": [
        (oracle.candidates, "top_candidates",
         lambda s, C: (len(s) - 1 - np.argsort(-np.asarray(s, np.float32)[::-1], kind="stable"))[:C])],
    "candidates: dot products summed in float32": [
        (oracle.candidates, "dot_rows",
         lambda M, x: (np.asarray(M, np.float32) @ np.asarray(x, np.float32)).astype(np.float64))],
    "candidates: lowest scores selected": [
        (oracle.candidates, "top_candidates",
         lambda s, C: np.argsort(np.asarray(s, np.float32), kind="stable")[:C])],
    "expand: midpoint window too wide": [
        (oracle.expand, "_near_fp32_midpoint", lambda x: _midpoint_dist(x) <= 1e-10 * abs(x))],
    "expand: midpoint window too narrow": [
        (oracle.expand, "_near_fp32_midpoint", lambda x: _midpoint_dist(x) <= 1e-14 * abs(x))],
    "expand: distance taken to the float32 value": [
        (oracle.expand, "_near_fp32_midpoint", lambda x: abs(x - float(np.float32(x))) <= 1e-12 * abs(x))],
    "candidates: midpoint window too wide": [
        (oracle.candidates, "_fp32_near_midpoint",
         lambda x: np.vectorize(lambda v: 0 < _midpoint_dist(v) <= 1e-10 * abs(v))(np.asarray(x, np.float64)))],
    "candidates: midpoint window too narrow": [
        (oracle.candidates, "_fp32_near_midpoint",
         lambda x: np.vectorize(lambda v: 0 < _midpoint_dist(v) <= 1e-14 * abs(v))(np.asarray(x, np.float64)))],
    "candidates: a sum on the midpoint flagged": [
        (oracle.candidates, "_fp32_near_midpoint",
         lambda x: np.vectorize(lambda v: _midpoint_dist(v) <= 1e-12 * abs(v))(np.asarray(x, np.float64)))],
    "stochastic: decision window too wide": [(oracle.stochastic, "_EPS", 1e-6)],
    "stochastic: decision window too narrow": [(oracle.stochastic, "_EPS", 1e-12)],
    "compact: one node short": [
        (oracle.compact, "kept_nodes", lambda row, n: [] if n < 0 else [0] + [int(row[j]) for j in range(n - 1)])],
}


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_mutation_is_caught(name, monkeypatch):
    for module, attr, repl in MUTATIONS[name]:
        monkeypatch.setattr(module, attr, repl)
    assert oracle_pins.failing_pins(), f"no pin noticed: {name}"


def test_unmutated_oracle_passes_every_pin():
    assert oracle_pins.failing_pins() == []
