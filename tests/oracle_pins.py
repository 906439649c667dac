"""Checks that pin the oracle to facts outside itself.

Each ``pin_*`` returns True when the oracle agrees with something it does not
compute itself: a closed form, a library routine (torch's scaled-dot-product
attention and logsumexp on the CPU, scipy's logsumexp and softmax), a brute force
that uses a different algorithm, or the structural facts the pages print.  The
pin tests assert them; the mutation tests plant mistakes in the oracle and assert
that at least one pin notices.
"""

import json
import os

import numpy as np
import scipy.special
import torch

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ------------------------------------------------------------------ tree structure

def _children(parent_row, n):
    kids = [[] for _ in range(n)]
    for i in range(1, n):
        kids[int(parent_row[i])].append(i)
    return kids


def brute_ancestry(parent_row, n):
    """(depth, ancestor matrix) by breadth-first search from the root and by
    collecting each node's subtree -- no upward walks."""
    kids = _children(parent_row, n)
    depth = [-1] * n
    depth[0] = 0
    queue = [0]
    while queue:
        j = queue.pop(0)
        for c in kids[j]:
            depth[c] = depth[j] + 1
            queue.append(c)
    is_anc = np.zeros((n, n), dtype=bool)          # is_anc[i, j]: j is i or an ancestor of i
    for j in range(n):
        stack = [j]
        while stack:
            x = stack.pop()
            is_anc[x, j] = True
            stack.extend(kids[x])
    return np.asarray(depth), is_anc


def pin_tree_example():
    """The pages' depth-3, 10-token example tree (reading of its lost figure)."""
    fx = json.load(open(os.path.join(GOLDEN, "eagle1_example_tree.json")))
    facts = fx["facts_printed_by_the_page"]
    par = np.asarray(fx["reading_parent"], dtype=np.int32)
    n = len(par)
    anc, depth, pos, st = oracle.tree_build(par[None, :], [n], [0])
    ok = st[0] == 0 and n == facts["example_tree_tokens"]
    ok &= int(depth[0].max()) == facts["example_tree_depth"]
    ok &= n > int(depth[0].max())
    # left-heavy: at every level, children counts never increase from left to right
    kids = _children(par, n)
    for d in range(int(depth[0].max()) + 1):
        level = [i for i in range(n) if depth[0, i] == d]
        counts = [len(kids[i]) for i in level]
        ok &= counts == sorted(counts, reverse=True)
    # the bitsets written out by hand from the parent array: node -> {itself, ancestors}
    by_hand = [0x1, 0x3, 0x5, 0x9, 0x1 | 0x2 | 0x10, 0x1 | 0x2 | 0x20, 0x1 | 0x4 | 0x40,
               0x1 | 0x2 | 0x10 | 0x80, 0x1 | 0x2 | 0x10 | 0x100, 0x1 | 0x2 | 0x20 | 0x200]
    ok &= [int(a) for a in anc[0, :n]] == by_hand
    ok &= list(depth[0, :n]) == [0, 1, 1, 1, 2, 2, 2, 3, 3, 3]
    return bool(ok)


def pin_tree_closed_forms(n=64):
    chain = synth.random_parents(None, n, "chain")
    star = synth.random_parents(None, n, "star")
    par = np.stack([chain, star])
    anc, depth, pos, st = oracle.tree_build(par, [n, n], [7, 0])
    ok = list(st) == [0, 0]
    ok &= all(int(anc[0, i]) == (1 << (i + 1)) - 1 for i in range(n))
    ok &= all(int(depth[0, i]) == i and int(pos[0, i]) == 7 + i for i in range(n))
    ok &= all(int(anc[1, i]) == (1 | (1 << i)) for i in range(n))
    ok &= all(int(depth[1, i]) == (0 if i == 0 else 1) for i in range(n))
    return bool(ok)


def pin_tree_bruteforce(seed, trials=20):
    rng = np.random.default_rng(seed)
    for t in range(trials):
        n = int(rng.integers(1, 65))
        shape = ["random", "chain", "star", "broom"][t % 4]
        par = synth.random_parents(rng, n, shape)
        row = np.full(64, -1, dtype=np.int32)
        row[:n] = par
        L = int(rng.integers(0, 5000))
        anc, depth, pos, st = oracle.tree_build(row[None, :], [n], [L])
        bd, bm = brute_ancestry(par, n)
        if st[0] != 0 or not np.array_equal(depth[0, :n], bd) or not np.array_equal(pos[0, :n], bd + L):
            return False
        for i in range(n):
            bits = int(anc[0, i])
            if [bool((bits >> j) & 1) for j in range(n)] != list(bm[i]) or bits >> n:
                return False
        if np.any(anc[0, n:] != 0) or np.any(depth[0, n:] != -1):
            return False
    return True


def pin_tree_status():
    S = oracle
    cases = [  # (parent prefix, n, expected status)
        ([-1, 0, 1], 3, S.STATUS_OK),
        ([0, 0, 1], 3, S.STATUS_BAD_PARENT),          # root with a parent
        ([-1, 0, 2], 3, S.STATUS_BAD_PARENT),         # parent == self
        ([-1, 2, 0], 3, S.STATUS_BAD_PARENT),         # parent after the child
        ([-1, -5, 0], 3, S.STATUS_BAD_PARENT),        # parent below -1
        ([-1, 0, -1], 3, S.STATUS_SECOND_ROOT),
        ([-1, -1, 7], 3, S.STATUS_SECOND_ROOT),       # the first offending node decides
        ([-1, 0, 1], 0, S.STATUS_BAD_N),
        ([-1, 0, 1], 65, S.STATUS_BAD_N),
    ]
    for par, n, want in cases:
        row = np.full(64, -1, dtype=np.int32)
        row[:len(par)] = par
        anc, depth, pos, st = oracle.tree_build(row[None, :], [n], None)
        if st[0] != want:
            return False
        if want != 0 and (np.any(anc != 0) or np.any(depth != -1) or np.any(pos != -1)):
            return False
    return True


# ------------------------------------------------------------------ attention

def _t(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))


def _case(seed, B=3, Hq=4, Hkv=2, D=16, lens=(9, 0, 3), n=(12, 6, 1), shapes=None):
    inp, parent, nn = synth.random_attention_case(seed, B, Hq, Hkv, D, lens, n, dtype="f32",
                                                  std=1.0, n_max=64, shapes=shapes)
    return inp, parent, nn


def _oracle_attn(inp, parent, nn):
    return oracle.tree_verify_attn(inp.q, inp.k_tree, inp.v_tree, inp.k_prefix, inp.v_prefix,
                                   inp.prefix_offsets, parent, nn)


def pin_attn_path_invariant(seed=1, tol=1e-10):
    """Each node's output = plain attention of that one query over prefix ++ its
    root path (library SDPA, no mask), and lse = torch.logsumexp of the scores."""
    inp, parent, nn = _case(seed)
    out, lse = _oracle_attn(inp, parent, nn)
    B, _, Hq, D = inp.q.shape
    G = Hq // inp.k_tree.shape[2]
    for b in range(B):
        o0, o1 = inp.prefix_offsets[b], inp.prefix_offsets[b + 1]
        _, is_anc = brute_ancestry(parent[b], int(nn[b]))
        for i in range(int(nn[b])):
            path = [j for j in range(int(nn[b])) if is_anc[i, j]]
            for h in range(Hq):
                g = h // G
                keys = np.concatenate([inp.k_prefix[o0:o1, g], inp.k_tree[b, path, g]])
                vals = np.concatenate([inp.v_prefix[o0:o1, g], inp.v_tree[b, path, g]])
                qq = _t(inp.q[b, i, h])[None, None, :]
                ref = torch.nn.functional.scaled_dot_product_attention(
                    qq, _t(keys)[None], _t(vals)[None], scale=1.0 / np.sqrt(D))[0, 0].numpy()
                l_ref = torch.logsumexp(_t(keys) @ _t(inp.q[b, i, h]) / np.sqrt(D), 0).item()
                if np.max(np.abs(ref - out[b, i, h])) > tol or abs(l_ref - lse[b, i, h]) > tol:
                    return False
    return True


def pin_attn_chain_is_causal(seed=2, L=11, n=13, tol=1e-10):
    """A chain tree equals causal attention over prefix ++ chain (library SDPA, is_causal)."""
    inp, parent, nn = _case(seed, B=1, Hq=2, Hkv=1, D=16, lens=(L,), n=(n,), shapes=["chain"])
    out, _ = _oracle_attn(inp, parent, nn)
    D = inp.q.shape[3]
    for h in range(2):
        keys = np.concatenate([inp.k_prefix[:, 0], inp.k_tree[0, :n, 0]])
        vals = np.concatenate([inp.v_prefix[:, 0], inp.v_tree[0, :n, 0]])
        qs = np.concatenate([np.zeros((L, D), np.float32), inp.q[0, :n, h]])   # prefix rows unused
        ref = torch.nn.functional.scaled_dot_product_attention(
            _t(qs)[None], _t(keys)[None], _t(vals)[None], is_causal=True,
            scale=1.0 / np.sqrt(D))[0, L:].numpy()
        if np.max(np.abs(ref - out[0, :n, h])) > tol:
            return False
    return True


def pin_attn_star(seed=3, L=5, n=9, tol=1e-10):
    """In a star every node sees the prefix, the root and itself -- nothing else."""
    inp, parent, nn = _case(seed, B=1, Hq=1, Hkv=1, D=16, lens=(L,), n=(n,), shapes=["star"])
    out, _ = _oracle_attn(inp, parent, nn)
    D = inp.q.shape[3]
    for i in range(n):
        sel = [0] if i == 0 else [0, i]
        keys = np.concatenate([inp.k_prefix[:, 0], inp.k_tree[0, sel, 0]])
        vals = np.concatenate([inp.v_prefix[:, 0], inp.v_tree[0, sel, 0]])
        ref = torch.nn.functional.scaled_dot_product_attention(
            _t(inp.q[0, i, 0])[None, None], _t(keys)[None], _t(vals)[None],
            scale=1.0 / np.sqrt(D))[0, 0].numpy()
        if np.max(np.abs(ref - out[0, i, 0])) > tol:
            return False
    return True


def pin_attn_empty_prefix(seed=4, n=10, tol=1e-10):
    """L = 0: pure tree attention, the root sees only itself (its output is its own V)."""
    inp, parent, nn = _case(seed, B=1, Hq=2, Hkv=2, D=16, lens=(0,), n=(n,))
    out, lse = _oracle_attn(inp, parent, nn)
    D = inp.q.shape[3]
    ok = np.max(np.abs(out[0, 0, :] - inp.v_tree[0, 0, :].astype(np.float64))) <= tol
    for h in range(2):
        l_root = float(inp.q[0, 0, h].astype(np.float64) @ inp.k_tree[0, 0, h].astype(np.float64)) / np.sqrt(D)
        ok &= abs(lse[0, 0, h] - l_root) <= tol
    return bool(ok)


def pin_attn_one_hot_mask(seed=5, n=40, L=7, D=128):
    """Exact mask probe: tree V rows are unit vectors e_j and prefix V is zero in the
    first 64 coordinates, so out[i][j] is exactly 0 off i's path and > 0 on it."""
    inp, parent, nn = _case(seed, B=1, Hq=2, Hkv=1, D=D, lens=(L,), n=(n,))
    inp.v_tree[:] = 0
    for j in range(n):
        inp.v_tree[0, j, 0, j] = 1.0
    inp.v_prefix[:, :, :64] = 0
    out, _ = _oracle_attn(inp, parent, nn)
    _, is_anc = brute_ancestry(parent[0], n)
    for i in range(n):
        for h in range(2):
            on = out[0, i, h, :n] > 0
            off = out[0, i, h, :n] == 0.0
            if not (np.array_equal(on, is_anc[i]) and np.array_equal(off, ~is_anc[i])):
                return False
    return True


def pin_attn_sibling_relabel(seed=6, tol=1e-12):
    """Relabelling siblings (keeping parent < child) permutes the outputs the same way."""
    inp, parent, nn = _case(seed, B=1, Hq=2, Hkv=1, D=16, lens=(4,), n=(6,))
    par = np.array([-1, 0, 0, 0, 1, 2] + [-1] * 58, dtype=np.int32)[None]
    out, _ = _oracle_attn(inp, par, nn)
    perm = [0, 2, 1, 3, 5, 4]           # new index of each old node: swap 1<->2 and 4<->5
    par2 = np.full_like(par, -1)
    for old in range(6):
        par2[0, perm[old]] = -1 if old == 0 else perm[par[0, old]]
    inp2 = synth.AttnInputs(**{**inp.__dict__})
    for name in ("q", "k_tree", "v_tree"):
        a = getattr(inp, name).copy()
        a[0, perm] = getattr(inp, name)[0, :6]
        setattr(inp2, name, a)
    out2, _ = _oracle_attn(inp2, par2, nn)
    return bool(np.max(np.abs(out2[0, perm] - out[0, :6])) <= tol)


def pin_attn_one_matches_full(seed=7):
    inp, parent, nn = _case(seed)
    out, lse = _oracle_attn(inp, parent, nn)
    for b in range(3):
        for i in range(int(nn[b])):
            for h in range(4):
                o, l = oracle.attention.tree_verify_attn_one(
                    inp.q, inp.k_tree, inp.v_tree, inp.k_prefix, inp.v_prefix, inp.prefix_offsets,
                    parent, b, h, i)
                if np.max(np.abs(o - out[b, i, h])) > 1e-12 or abs(l - lse[b, i, h]) > 1e-12:
                    return False
    return True


# ------------------------------------------------------------------ expansion / rerank

def quantised_logits(rng, shape):
    """Logits on a 0.5 grid so that equal logits and equal scores are common."""
    return (rng.integers(-8, 9, size=shape) * 0.5).astype(np.float32)


def brute_expand_one(levels, k, m, root):
    """One sequence, nodes named by their token path; every ranking is a plain sorted()."""
    V = levels[0].shape[-1]
    everything = []                    # (path, score, creation)
    frontier = [((), np.float32(0.0))]
    made = 0
    for rows in levels:
        cand = []
        for f, (path, sc) in enumerate(frontier):
            row = rows[f]
            lse32 = np.float32(scipy.special.logsumexp(row.astype(np.float64)))
            for t in sorted(range(V), key=lambda t: (-float(row[t]), t))[:k]:
                cand.append((path + (t,), np.float32(sc + np.float32(row[t] - lse32)), made))
                made += 1
        everything += cand
        frontier = [(p, s) for p, s, _ in sorted(cand, key=lambda x: (-float(x[1]), x[2]))[:k]]
    kept = sorted(everything, key=lambda x: (-float(x[1]), x[2]))[:m - 1]
    kept.sort(key=lambda x: (len(x[0]), x[2]))
    paths = [()] + [p for p, _, _ in kept]
    parent = [-1] + [paths.index(p[:-1]) for p, _, _ in kept]
    token = [root] + [p[-1] for p, _, _ in kept]
    score = [np.float32(0.0)] + [s for _, s, _ in kept]
    return parent, token, score


def _levels(rng, B, S, k, V, quant=True):
    out = []
    for s in range(S):
        shape = (B, 1 if s == 0 else k, V)
        out.append(quantised_logits(rng, shape) if quant else
                   (rng.standard_normal(shape) * 2).astype(np.float32))
    return out


def pin_expand_bruteforce(seed=11, trials=12):
    rng = np.random.default_rng(seed)
    for t in range(trials):
        k = [1, 2, 3][t % 3]
        S = 1 + t % 3
        V = 16
        B = 2
        levels = _levels(rng, B, S, k, V, quant=(t % 2 == 0))
        m = int(rng.integers(1, 12))
        roots = rng.integers(0, V, size=B)
        res = oracle.expand_rerank(levels, k, m, roots, n_max=64)
        for b in range(B):
            par, tok, sc = brute_expand_one([lv[b] for lv in levels], k, m, int(roots[b]))
            n = len(par)
            if res.status[b] != 0 or res.n_nodes[b] != n:
                return False
            if list(res.parent[b, :n]) != par or list(res.token[b, :n]) != tok:
                return False
            if res.score[b, :n].tobytes() != np.asarray(sc, np.float32).tobytes():
                return False
    return True


def pin_expand_closed_forms(seed=12):
    rng = np.random.default_rng(seed)
    ok = True
    # k = 1: a chain of the row argmaxes (lowest id among equal maxima)
    levels = _levels(rng, 1, 5, 1, 16)
    res = oracle.expand_rerank(levels, 1, 64, [3])
    ok &= res.n_nodes[0] == 6 and list(res.parent[0, :6]) == [-1, 0, 1, 2, 3, 4]
    ok &= list(res.token[0, 1:6]) == [int(np.flatnonzero(lv[0, 0] == lv[0, 0].max())[0]) for lv in levels]
    # one level: a star of the m-1 best root-row tokens in logit order
    levels = _levels(rng, 1, 1, 6, 16)
    res = oracle.expand_rerank(levels, 6, 5, [0])
    row = levels[0][0, 0]
    best = sorted(range(16), key=lambda t: (-float(row[t]), t))[:4]
    ok &= res.n_nodes[0] == 5 and list(res.parent[0, :5]) == [-1, 0, 0, 0, 0]
    ok &= list(res.token[0, 1:5]) == best
    # m - 1 >= pool keeps every generated node: k + (S-1) k^2
    levels = _levels(rng, 1, 3, 2, 16)
    res = oracle.expand_rerank(levels, 2, 64, [0])
    ok &= res.n_nodes[0] == 1 + 2 + 2 * 4
    return bool(ok)


def pin_expand_value_is_path_product(seed=13, tol=2e-5):
    """exp(score) equals the product of the softmax confidences along the node's path
    (the global-acceptance value), computed with scipy's softmax in float64.  Two
    levels, so every level-1 token is distinct and names its logit row uniquely."""
    rng = np.random.default_rng(seed)
    k, V = 4, 50
    levels = _levels(rng, 1, 2, k, V, quant=False)
    res = oracle.expand_rerank(levels, k, 64, [0])
    n = int(res.n_nodes[0])
    if n != 1 + k + k * k:
        return False
    par, tok = res.parent[0], res.token[0]
    rank_of = {int(t): r for r, t in enumerate(res.frontier_tokens[0][0])}
    for i in range(1, n):
        if par[i] == 0:
            prob = scipy.special.softmax(levels[0][0, 0].astype(np.float64))[tok[i]]
        else:
            p = par[i]
            prob = (scipy.special.softmax(levels[0][0, 0].astype(np.float64))[tok[p]] *
                    scipy.special.softmax(levels[1][0, rank_of[int(tok[p])]].astype(np.float64))[tok[i]])
        if abs(np.exp(np.float64(res.score[0, i])) - prob) > tol * prob:
            return False
    return True


def pin_expand_invariants(seed=14):
    """Ancestor closure, scores never increase along a path, kept = the best m-1 by
    (score, creation) -- on 2*N(0,1) logits as in the dynamic-tree workloads."""
    rng = np.random.default_rng(seed)
    levels = _levels(rng, 3, 5, 4, 200, quant=False)
    res = oracle.expand_rerank(levels, 4, [20, 64, 2], [1, 2, 3])
    ok = list(res.status) == [0, 0, 0]
    ok &= list(res.n_nodes) == [20, 64, 2]          # pool = 4 + 4 * 16 = 68 >= 63
    for b in range(3):
        n = int(res.n_nodes[b])
        for i in range(1, n):
            p = res.parent[b, i]
            ok &= 0 <= p < i and res.score[b, i] <= res.score[b, p]
    return bool(ok)


def pin_expand_nonfinite():
    """A NaN row fails its sequence at that level: the level before keeps its frontier,
    the failing level and the rest report none; an out-of-range m fails at the last level."""
    rng = np.random.default_rng(15)
    levels = _levels(rng, 3, 3, 2, 16, quant=False)
    levels[1][1, 1, 5] = np.nan
    res = oracle.expand_rerank(levels, 2, [5, 5, 65], [0, 0, 0])
    ok = list(res.status) == [0, oracle.STATUS_NONFINITE, oracle.STATUS_BAD_N]
    ok &= res.n_nodes[1] == 0 and np.all(res.parent[1] == -1) and res.n_nodes[2] == 0
    ok &= np.all(res.frontier_tokens[0][1] >= 0) and np.all(res.frontier_tokens[1][1] == -1)
    ok &= np.all(res.frontier_tokens[1][2] >= 0) and np.all(res.frontier_tokens[2][2] == -1)
    return bool(ok)


# ------------------------------------------------------------------ acceptance

def brute_accept_one(par, tok, tgt, n):
    """Top-down: from the root, step into every child whose token equals the target's
    token after the current node; keep the deepest node reached (lowest index on ties)."""
    kids = _children(par, n)
    best, best_d = 0, 0
    stack = [(0, 0)]
    while stack:
        x, d = stack.pop()
        if d > best_d or (d == best_d and x < best):
            best, best_d = x, d
        for c in kids[x]:
            if int(tok[c]) == int(tgt[x]):
                stack.append((c, d + 1))
    path = []
    j = best
    while j != 0:
        path.append(j)
        j = int(par[j])
    return best_d, best, int(tgt[best]), path[::-1]


def pin_accept_bruteforce(seed=21, trials=200):
    rng = np.random.default_rng(seed)
    for t in range(trials):
        n = int(rng.integers(1, 65))
        par = np.full(64, -1, dtype=np.int32)
        par[:n] = synth.random_parents(rng, n, ["random", "chain", "star", "broom"][t % 4])
        V = [2, 3, 5, 32000][t % 4]              # small vocabularies make duplicates common
        tok = rng.integers(0, V, size=64).astype(np.int32)
        tgt = rng.integers(0, V, size=64).astype(np.int32)
        al, best, bonus, path = oracle.tree_accept(par[None], tok[None], tgt[None], [n])
        d, bb, bo, pp = brute_accept_one(par, tok, tgt, n)
        if (al[0], best[0], bonus[0]) != (d, bb, bo) or list(path[0, :d]) != pp or np.any(path[0, d:] != -1):
            return False
    return True


def pin_accept_closed_forms():
    n = 9
    chain = np.full(64, -1, np.int32)
    chain[:n] = synth.random_parents(None, n, "chain")
    tok = np.arange(100, 164, dtype=np.int32)
    tgt_all = np.roll(tok, -1).astype(np.int32)      # target after node i is node i+1's token
    al, best, bonus, path = oracle.tree_accept(chain[None], tok[None], tgt_all[None], [n])
    ok = al[0] == n - 1 and best[0] == n - 1 and bonus[0] == tgt_all[n - 1]
    ok &= list(path[0, :n - 1]) == list(range(1, n))
    tgt_none = np.full(64, 7, np.int32)
    al, best, bonus, path = oracle.tree_accept(chain[None], tok[None], tgt_none[None], [n])
    ok &= al[0] == 0 and best[0] == 0 and bonus[0] == 7 and np.all(path[0] == -1)
    # duplicate siblings: nodes 1 and 2 both carry the target's token; 2 leads deeper
    par = np.full(64, -1, np.int32)
    par[:5] = [-1, 0, 0, 2, 1]
    tok = np.zeros(64, np.int32)
    tok[:5] = [0, 5, 5, 6, 9]
    tgt = np.zeros(64, np.int32)
    tgt[:5] = [5, 8, 6, 4, 3]
    al, best, bonus, path = oracle.tree_accept(par[None], tok[None], tgt[None], [5])
    ok &= al[0] == 2 and best[0] == 3 and bonus[0] == 4 and list(path[0, :2]) == [2, 3]
    # equal depth: lowest index wins
    tgt[:5] = [5, 9, 6, 4, 3]
    al, best, bonus, path = oracle.tree_accept(par[None], tok[None], tgt[None], [5])
    ok &= al[0] == 2 and best[0] == 3
    tok[4] = 9
    tgt[2] = 1
    al, best, bonus, path = oracle.tree_accept(par[None], tok[None], tgt[None], [5])
    ok &= al[0] == 2 and best[0] == 4 and list(path[0, :2]) == [1, 4]
    # root only
    al, best, bonus, path = oracle.tree_accept(par[None], tok[None], tgt[None], [1])
    ok &= al[0] == 0 and best[0] == 0 and bonus[0] == tgt[0]
    # invalid trees give -1
    al, best, bonus, path = oracle.tree_accept(par[None], tok[None], tgt[None], [0])
    ok &= al[0] == -1 and best[0] == -1 and bonus[0] == -1
    return bool(ok)


# ----------------------------------------------------------------------------- compaction

def _compact_case(seed, B=5, n_max=64, Hkv=2, D=8, rows=600):
    rng = np.random.default_rng(seed)
    parent = np.full((B, n_max), -1, np.int32)
    nn = rng.integers(1, n_max + 1, size=B).astype(np.int32)
    for b in range(B):
        for i in range(1, int(nn[b])):
            parent[b, i] = rng.integers(0, i)
    tok = rng.integers(0, 5, size=(B, n_max)).astype(np.int32)       # small vocabulary: many hits
    tgt = rng.integers(0, 5, size=(B, n_max)).astype(np.int32)
    kt = rng.standard_normal((B, n_max, Hkv, D)).astype(np.float32)
    vt = rng.standard_normal((B, n_max, Hkv, D)).astype(np.float32)
    kd = rng.standard_normal((rows, Hkv, D)).astype(np.float32)
    vd = rng.standard_normal((rows, Hkv, D)).astype(np.float32)
    dst = (np.arange(B) * (rows // B)).astype(np.int64)
    return parent, nn, tok, tgt, kt, vt, kd, vd, dst


def pin_compact_chain():
    """A chain whose every draft token is the target's: the whole tree, in order, and
    nothing past it."""
    parent, nn, tok, tgt, kt, vt, kd, vd, dst = _compact_case(5, B=1)
    n = 20
    nn[0] = n
    parent[0, :] = -1
    parent[0, 1:n] = np.arange(n - 1)
    tgt[0, :n - 1] = tok[0, 1:n]
    alen, best, _, path = oracle.tree_accept(parent, tok, tgt, nn)
    if alen[0] != n - 1 or best[0] != n - 1:
        return False
    k2, v2 = oracle.kv_compact(kt, vt, path, alen, kd, vd, dst)
    return (np.array_equal(k2[:n], kt[0, :n]) and np.array_equal(v2[:n], vt[0, :n]) and
            np.array_equal(k2[n:], kd[n:]) and np.array_equal(v2[n:], vd[n:]))


def pin_compact_root_only():
    """No draft token matches: only the root's row is written."""
    parent, nn, tok, tgt, kt, vt, kd, vd, dst = _compact_case(6, B=1)
    nn[0] = 10
    parent[0, :10] = [-1, 0, 0, 1, 1, 2, 3, 3, 4, 8]
    tgt[0] = -7
    alen, _, _, path = oracle.tree_accept(parent, tok, tgt, nn)
    if alen[0] != 0:
        return False
    k2, v2 = oracle.kv_compact(kt, vt, path, alen, kd, vd, dst)
    return (np.array_equal(k2[0], kt[0, 0]) and np.array_equal(v2[0], vt[0, 0]) and
            np.array_equal(k2[1:], kd[1:]) and np.array_equal(v2[1:], vd[1:]))


def pin_compact_root_path(seed=7):
    """Row 0 is the root; each further row's node is the child of the previous row's
    node on the way to the chosen node (an independent walk up from the chosen node);
    nothing else of the destination changes."""
    parent, nn, tok, tgt, kt, vt, kd, vd, dst = _compact_case(seed)
    alen, best, _, path = oracle.tree_accept(parent, tok, tgt, nn)
    k2, v2 = oracle.kv_compact(kt, vt, path, alen, kd, vd, dst)
    written = np.zeros(kd.shape[0], bool)
    for b in range(parent.shape[0]):
        chain = [int(best[b])]
        while chain[-1] != 0:
            chain.append(int(parent[b, chain[-1]]))
        chain = chain[::-1]
        if len(chain) != int(alen[b]) + 1:
            return False
        for j, node in enumerate(chain):
            r = int(dst[b]) + j
            if not (np.array_equal(k2[r], kt[b, node]) and np.array_equal(v2[r], vt[b, node])):
                return False
            written[r] = True
    return np.array_equal(k2[~written], kd[~written]) and np.array_equal(v2[~written], vd[~written])


def pin_compact_edges():
    """A rejected tree (accept_len -1) copies nothing; rows past the buffer are skipped."""
    parent, nn, tok, tgt, kt, vt, kd, vd, dst = _compact_case(10, B=2, rows=40)
    path = np.full((2, 64), -1, np.int32)
    path[1, :5] = [1, 2, 3, 4, 5]
    alen = np.array([-1, 5], np.int32)
    dst = np.array([0, 37], np.int64)                                    # rows 37..42: 3 fit
    k2, _ = oracle.kv_compact(kt, vt, path, alen, kd, vd, dst)
    return (np.array_equal(k2[:37], kd[:37]) and np.array_equal(k2[37], kt[1, 0]) and
            np.array_equal(k2[38], kt[1, 1]) and np.array_equal(k2[39], kt[1, 2]))


# ----------------------------------------------------------------------------- stochastic acceptance

def _softmax_rows(rng, shape, scale=1.0):
    x = rng.standard_normal(shape) * scale
    e = np.exp(x - x.max(axis=-1, keepdims=True))
    return (e / e.sum(axis=-1, keepdims=True)).astype(np.float32)


def pin_stochastic_greedy_limit(seed=51, trials=40):
    """One-hot target distributions (at target_next[u]) and distinct sibling tokens:
    for any uniforms the walk is greedy acceptance (checked against tree_accept)."""
    rng = np.random.default_rng(seed)
    V, n_max = 12, 16
    for _ in range(trials):
        n = int(rng.integers(1, n_max + 1))
        parent = np.full((1, n_max), -1, np.int32)
        tok = np.zeros((1, n_max), np.int32)
        for i in range(1, n):
            parent[0, i] = rng.integers(0, i)
        for u in range(n):
            kids = [c for c in range(1, n) if parent[0, c] == u]
            tok[0, kids] = rng.choice(V, size=len(kids), replace=False)
        tgt = rng.integers(0, V, size=(1, n_max)).astype(np.int32)
        p = np.zeros((1, n_max, V), np.float32)
        p[0, np.arange(n_max), tgt[0]] = 1.0
        q = _softmax_rows(rng, (1, n_max, V))
        ua = rng.random((1, n_max)).astype(np.float32)
        ub = rng.random(1).astype(np.float32)
        nn = np.array([n], np.int32)
        a, bst, bon, path, ind = oracle.tree_accept_stochastic(parent, tok, nn, p, q, ua, ub)
        ga, gb, gbon, gpath = oracle.tree_accept(parent, tok, tgt, nn)
        if ind[0] or a[0] != ga[0] or bst[0] != gb[0] or bon[0] != gbon[0] or not np.array_equal(path, gpath):
            return False
    return True


def pin_stochastic_hand_example():
    """V = 4, root children with tokens 2 and 0, p = (0.1, 0.2, 0.3, 0.4), q = (0.25,
    0.25, 0.5, 0).  Token 2 passes iff u < 0.3 / 0.5 = 0.6; after its rejection the
    residual is (0, 0, 0, 0.4), token 0 then fails whatever u, and the bonus is token 3
    whatever u; a passing token 2 moves to its leaf, whose bonus comes from its own
    row: (0, 1, 0, 0) gives token 1."""
    parent = np.array([[-1, 0, 0, -1]], np.int32)
    tok = np.array([[9, 2, 0, 0]], np.int32)
    nn = np.array([3], np.int32)
    p = np.zeros((1, 4, 4), np.float32)
    p[0, 0] = [0.1, 0.2, 0.3, 0.4]
    p[0, 1] = [0.0, 1.0, 0.0, 0.0]
    p[0, 2] = [1.0, 0.0, 0.0, 0.0]
    q = np.zeros((1, 4, 4), np.float32)
    q[0, 0] = [0.25, 0.25, 0.5, 0.0]
    for u1, ub, want in [(0.7, 0.01, (0, 0, 3)), (0.7, 0.99, (0, 0, 3)), (0.59, 0.5, (1, 1, 1)),
                         (0.0, 0.99, (1, 1, 1))]:
        ua = np.array([[0.0, u1, 0.3, 0.0]], np.float32)
        a, bst, bon, _, ind = oracle.tree_accept_stochastic(parent, tok, nn, p, q, ua,
                                                            np.array([ub], np.float32))
        if ind[0] or (int(a[0]), int(bst[0]), int(bon[0])) != want:
            return False
    return True


def pin_stochastic_preserves_target(seed=52, trials=20000):
    """Candidates drawn independently from the draft distribution: the first token the
    walk emits (the passing child's token, else the bonus) follows the target's
    distribution (rejection sampling leaves the output distribution unchanged)."""
    rng = np.random.default_rng(seed)
    V, k = 5, 3
    p0 = np.array([0.05, 0.4, 0.15, 0.3, 0.1], np.float32)
    q0 = np.array([0.3, 0.1, 0.3, 0.1, 0.2], np.float32)
    parent = np.array([[-1] + [0] * k], np.int32)
    nn = np.array([k + 1], np.int32)
    p = np.zeros((1, k + 1, V), np.float32)
    p[0, 0] = p0
    p[0, 1:] = 1.0 / V
    q = np.zeros((1, k + 1, V), np.float32)
    q[0, 0] = q0
    counts = np.zeros(V)
    for _ in range(trials):
        tok = np.zeros((1, k + 1), np.int32)
        tok[0, 1:] = rng.choice(V, size=k, p=q0 / q0.sum())
        ua = rng.random((1, k + 1)).astype(np.float32)
        ub = rng.random(1).astype(np.float32)
        a, bst, bon, _, _ = oracle.tree_accept_stochastic(parent, tok, nn, p, q, ua, ub)
        counts[int(tok[0, bst[0]]) if a[0] == 1 else int(bon[0])] += 1
    expect = trials * p0.astype(np.float64)
    chi2 = float(np.sum((counts - expect) ** 2 / expect))
    return chi2 < 20.0                       # 4 degrees of freedom: p-value ~ 5e-4


# ----------------------------------------------------------------------------- verify budget

def _budget_case(seed=61):
    rng = np.random.default_rng(seed)
    B, k, S, V = 3, 4, 4, 50
    steps = [(rng.standard_normal((B, 1 if s == 0 else k, V)) * 2).astype(np.float32) for s in range(S)]
    return steps, k, rng.integers(0, V, size=B)


def pin_budget_limits():
    """A bar of -inf keeps what the plain rerank keeps; +inf keeps the root only; a
    bar just under the j-th best score keeps exactly j candidates."""
    steps, k, roots = _budget_case()
    plain = oracle.expand_rerank(steps, k, 20, roots)
    lo = oracle.expand_rerank(steps, k, 20, roots, budget_log=np.full(64, -np.inf, np.float32))
    hi = oracle.expand_rerank(steps, k, 20, roots, budget_log=np.full(64, np.inf, np.float32))
    if not (np.array_equal(plain.parent, lo.parent) and np.array_equal(plain.n_nodes, lo.n_nodes)):
        return False
    if not np.all(hi.n_nodes == 1):
        return False
    for b in range(3):
        sc = np.sort(plain.score[b, 1:plain.n_nodes[b]])[::-1]       # best first
        for j in (1, 5, 11):
            bar = np.full(64, -np.inf, np.float32)
            bar[j + 1:] = sc[j]                                       # candidate j+1 ties the bar
            cut = oracle.expand_rerank(steps, k, 20, roots, budget_log=bar)
            if cut.n_nodes[b] != j + 1:
                return False
            # the kept nodes are exactly the plain tree's j best, ancestors included
            kept = np.sort(cut.score[b, 1:j + 1])[::-1]
            if not np.array_equal(kept, sc[:j]):
                return False
            par = cut.parent[b, 1:j + 1]
            if not np.all((par >= 0) & (par < np.arange(1, j + 1))):
                return False
    return True


def pin_budget_first_failure_stops():
    """A bar that only the 3rd candidate fails keeps two, though later ones pass."""
    steps, k, roots = _budget_case(62)
    plain = oracle.expand_rerank(steps, k, 12, roots)
    bar = np.full(64, -np.inf, np.float32)
    bar[3] = np.inf
    cut = oracle.expand_rerank(steps, k, 12, roots, budget_log=bar)
    return bool(np.all(cut.n_nodes == 3)) and bool(np.all(plain.n_nodes == 12))



# ------------------------------------------------------------------ per-level stop

def _stop_cases(seed):
    """Small dynamic trees (quantised logits: ties common) with verify budgets from a
    convex synthetic cost table, plus the two extreme budgets and none."""
    rng = np.random.default_rng(seed)
    for t in range(8):
        B, k, S, V = 4, [2, 3, 4, 8][t % 4], [5, 5, 5, 4][t % 4], [20, 40, 60, 100][t % 4]
        steps = _levels(rng, B, S, k, V, quant=t % 2 == 0)
        m = rng.integers(2, 65, size=B)
        j = np.arange(64, dtype=np.float64)
        marginal = 0.05 + 0.02 * j                         # d/dN of a convex cost table
        for bar in (np.log(10.0 ** rng.uniform(-4, -1) * marginal).astype(np.float32),
                    np.full(64, -np.inf, np.float32), np.full(64, np.inf, np.float32), None):
            if bar is not None:
                bar[0] = -np.inf
            yield steps, k, m, bar, rng.integers(0, V, size=B)


def _depth(parent_row, i):
    d = 0
    while i > 0:
        i = int(parent_row[i])
        d += 1
    return d


def pin_stop_means_deepest_level_kept(seed=71):
    """more[s][b] = 1 exactly when the tree reranked right after level s + 1 keeps a
    node of that level (the deepest level drafted so far)."""
    for steps, k, m, bar, roots in _stop_cases(seed):
        more = oracle.expand.draft_continue(steps, k, m, bar)
        for s in range(len(steps)):
            res = oracle.expand_rerank(steps[:s + 1], k, m, roots, budget_log=bar)
            for b in range(len(m)):
                deepest = max(_depth(res.parent[b], i) for i in range(int(res.n_nodes[b])))
                if int(more[s, b]) != int(deepest == s + 1):
                    return False
    return True


def pin_stop_is_lossless(seed=72):
    """Stopping at the first level whose flag is 0 and reranking there gives the same
    tree as drafting every level."""
    seen = 0
    for steps, k, m, bar, roots in _stop_cases(seed):
        more = oracle.expand.draft_continue(steps, k, m, bar)
        full = oracle.expand_rerank(steps, k, m, roots, budget_log=bar)
        for b in range(len(m)):
            zeros = np.flatnonzero(more[:, b] == 0)
            if len(zeros) == 0 or zeros[0] == len(steps) - 1:
                continue
            s0 = int(zeros[0])
            cut = oracle.expand_rerank(steps[:s0 + 1], k, m, roots, budget_log=bar)
            seen += 1
            if not (cut.n_nodes[b] == full.n_nodes[b] and np.array_equal(cut.parent[b], full.parent[b])
                    and np.array_equal(cut.token[b], full.token[b])
                    and cut.score[b].tobytes() == full.score[b].tobytes()):
                return False
    return seen >= 20                          # the stop is exercised, not vacuous


def pin_stop_limits():
    """A budget of +inf stops at once; a failing row gives 0 from its level on; m = 1
    never drafts."""
    steps, k, roots = _budget_case(63)
    hi = oracle.expand.draft_continue(steps, k, 20, np.full(64, np.inf, np.float32))
    one = oracle.expand.draft_continue(steps, k, 1, None)
    bad = [x.copy() for x in steps]
    bad[2][1, 0, 3] = np.inf
    nf = oracle.expand.draft_continue(bad, k, 63, None)
    ok = not hi.any() and not one.any()
    ok &= bool(np.all(nf[:2, 1] == 1)) and bool(np.all(nf[2:, 1] == 0)) and bool(np.all(nf[:, 0] == 1))
    return bool(ok)



# ------------------------------------------------------------------ low-rank candidate head

def _f32_of_fraction(q):
    """The float32 nearest to the rational q (ties to even), found without double rounding."""
    from fractions import Fraction
    f = np.float32(float(q))
    best = None
    for c in (np.nextafter(f, np.float32(-np.inf)), f, np.nextafter(f, np.float32(np.inf))):
        d = abs(Fraction(float(c)) - q)
        key = (d, int(np.float32(c).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, c)
    return np.float32(best[1])


def _exact_dot_f32(u, v):
    from fractions import Fraction
    return _f32_of_fraction(sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(u, v)))


def _bf16_values(rng, shape, scale=1.0):
    return synth.bf16_to_f32(synth.bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32)))


def pin_candidates_exact_dots(seed=91):
    """Every logit is the exactly rounded dot product: candidates W[v].h, the others
    Bm[v].z with z the exactly rounded A h (rational arithmetic on the bf16 values)."""
    rng = np.random.default_rng(seed)
    d, r, V, C = 24, 6, 40, 7
    h = _bf16_values(rng, (2, d))
    A, Bm, W = _bf16_values(rng, (r, d), 0.3), _bf16_values(rng, (V, r)), _bf16_values(rng, (V, d), 0.3)
    logits, cand, _, _ = oracle.candidate_logits(h, A, Bm, W, C)
    for i in range(2):
        z = np.array([_exact_dot_f32(A[j], h[i]) for j in range(r)], dtype=np.float32)
        s = np.array([_exact_dot_f32(Bm[v], z) for v in range(V)], dtype=np.float32)
        best = sorted(range(V), key=lambda v: (-float(s[v]), v))[:C]
        if list(cand[i]) != best:
            return False
        for v in range(V):
            want = _exact_dot_f32(W[v], h[i]) if v in best else s[v]
            if logits[i, v].tobytes() != np.float32(want).tobytes():
                return False
    return True


def pin_candidates_low_rank_exact():
    """When the LM head is exactly Bm A (small integers), the low-rank score equals the
    full logit, so the row is the full logits row whatever C is, and the candidates
    are its C largest (ties to the lower id)."""
    rng = np.random.default_rng(92)
    d, r, V = 16, 4, 30
    A = rng.integers(-3, 4, size=(r, d)).astype(np.float32)
    Bm = rng.integers(-3, 4, size=(V, r)).astype(np.float32)
    W = (Bm @ A).astype(np.float32)
    h = rng.integers(-2, 3, size=(3, d)).astype(np.float32)
    full = (h.astype(np.float64) @ W.T.astype(np.float64)).astype(np.float32)
    for C in (1, 5, 30):
        logits, cand, _, _ = oracle.candidate_logits(h, A, Bm, W, C)
        if not np.array_equal(logits, full):
            return False
        for i in range(3):
            if list(cand[i]) != sorted(range(V), key=lambda v: (-float(full[i, v]), v))[:C]:
                return False
    return True


def pin_candidates_all_exact():
    """C = V: every entry is the full logit W h."""
    rng = np.random.default_rng(93)
    d, r, V = 32, 8, 50
    h = _bf16_values(rng, (2, d))
    A, Bm, W = _bf16_values(rng, (r, d)), _bf16_values(rng, (V, r)), _bf16_values(rng, (V, d))
    logits, _, _, _ = oracle.candidate_logits(h, A, Bm, W, V)
    return all(logits[i, v].tobytes() == _exact_dot_f32(W[v], h[i]).tobytes()
               for i in range(2) for v in range(V))


# ---------------------------------------------------------------- indeterminate flags

def _f32_midpoints(values):
    """float64 midpoints between float32 values and their next float32 up (exact:
    25 significant bits fit a float64)."""
    f = np.asarray(values, dtype=np.float32)
    hi = np.nextafter(f, np.float32(np.inf))
    return (f.astype(np.float64) + hi.astype(np.float64)) / 2.0


_FLAG_PROBES = np.array([1.2345678, -3.75e-3, 1234.5, 0.69314718, -41.0], dtype=np.float32)


def pin_expand_midpoint_flag():
    """The expansion's float64 log-normaliser is flagged exactly when it lies within
    1e-12 (relative) of a float32 rounding midpoint -- on it included: values on a
    midpoint, 1e-13 off either side are flagged; 1e-11 off, or on a float32 value
    (half an ulp, about 6e-8, away) are not.  Then through expand_rerank: a row of V equal
    logits l has the log-normaliser l + log V exactly as the oracle sums it; the search
    below picks (l, V) next to a midpoint (flagged) and far from every one (not)."""
    helper = oracle.expand._near_fp32_midpoint
    for m in _f32_midpoints(_FLAG_PROBES):
        for x, want in ((m, True), (m * (1 + 1e-13), True), (m * (1 - 1e-13), True),
                        (m * (1 + 1e-11), False), (m * (1 - 1e-11), False),
                        (float(np.float32(m)), False)):
            if bool(helper(np.float64(x))) != want:
                return False
    Vs = np.arange(8, 1 << 17, dtype=np.int64)
    logs = np.log(Vs.astype(np.float64))
    near = far = None
    for l in np.float32(0.5) + np.arange(64, dtype=np.float32) * np.float32(1.0 / 64):
        lse = np.float64(l) + logs
        f = lse.astype(np.float32)
        d = np.minimum(np.abs(lse - _f32_midpoints(f)),
                       np.abs(lse - _f32_midpoints(np.nextafter(f, np.float32(-np.inf)))))
        hit = np.nonzero(d <= 2e-13 * np.abs(lse))[0]
        if near is None and len(hit):
            near = (l, int(Vs[hit[0]]))
        if far is None:
            miss = np.nonzero(d >= 1e-9 * np.abs(lse))[0]
            far = (l, int(Vs[miss[0]])) if len(miss) else None
        if near is not None and far is not None:
            break
    if near is None or far is None:
        return False
    for (l, V), want in ((near, True), (far, False)):
        level = np.full((1, 1, V), l, dtype=np.float32)
        res = oracle.expand_rerank([level], 2, 3, np.array([0], np.int32))
        if bool(res.indeterminate[0]) != want:
            return False
    return True


def pin_candidates_midpoint_flag():
    """The candidate head flags a float64 dot product within 1e-12 (relative) of a
    float32 rounding midpoint and not exactly on it (a sum on a midpoint was carried
    exactly and rounds to even on both sides): 1e-13 off either side flagged; on it,
    1e-11 off, or on a float32 value not."""
    helper = oracle.candidates._fp32_near_midpoint
    xs, want = [], []
    for m in _f32_midpoints(_FLAG_PROBES):
        for x, w in ((m, False), (m * (1 + 1e-13), True), (m * (1 - 1e-13), True),
                     (m * (1 + 1e-11), False), (m * (1 - 1e-11), False),
                     (float(np.float32(m)), False)):
            xs.append(x)
            want.append(w)
    return bool(np.array_equal(helper(np.array(xs, dtype=np.float64)), np.array(want)))


def _stoch_two_node(r_root, q_root, x, ua, ub):
    """A root with one child of token x: target weights r (root row) and draft q;
    the child's own target row is one-hot."""
    V = len(r_root)
    parent = np.array([[-1, 0]], np.int32)
    tok = np.array([[0, x]], np.int32)
    p = np.zeros((1, 2, V), np.float32)
    p[0, 0] = r_root
    p[0, 1, 0] = 1.0
    q = np.zeros((1, 2, V), np.float32)
    q[0, 0] = q_root
    q[0, 1, 0] = 1.0
    return oracle.tree_accept_stochastic(parent, tok, np.array([2], np.int32), p, q,
                                         np.array([[0.0, ua]], np.float32),
                                         np.array([ub], np.float32))


def pin_stochastic_margins():
    """Stochastic acceptance reports a sequence as indeterminate exactly when a decision
    lies within 1e-9 (relative) of its threshold.  Target weights r = (1/2, 1/4, 1/4, t)
    have the float64 sum S = 1 + t exactly.  The child of token 1 with draft q(1) = 1/2
    and u = 1/2 is tested by u S q(1) = (1 + t) / 4 < r(1) = 1/4: it fails, with
    relative margin t.  t = 2^-33 (1.2e-10) is flagged, t = 2^-28 (3.7e-9) is not, and
    u one float32 step below 1/2 passes by 6e-8, unflagged.  The bonus draw of a root
    without children is the first index whose running sum (1/2, 3/4, 1, 1 + t) passes
    u S: u = 3/4 gives index 2 at 3/4 t (6.5e-11 for t = 2^-33) from the boundary
    3/4, flagged; u = 0.6 gives index 1 far from both boundaries."""
    q = np.array([0.25, 0.5, 0.25, 0.0], np.float32)
    half_down = float(np.nextafter(np.float32(0.5), np.float32(0.0)))
    for t, ua, want_pass, want_flag in ((2.0 ** -33, 0.5, False, True), (2.0 ** -28, 0.5, False, False),
                                        (2.0 ** -33, half_down, True, False)):
        r = np.array([0.5, 0.25, 0.25, t], np.float32)
        alen, best, bonus, path, indet = _stoch_two_node(r, q, 1, ua, 0.6)
        if bool(alen[0] == 1) != want_pass or bool(indet[0]) != want_flag:
            return False
    for t, ub, want_idx, want_flag in ((2.0 ** -33, 0.75, 2, True), (2.0 ** -33, 0.6, 1, False),
                                       (2.0 ** -20, 0.75, 2, False)):
        r = np.array([0.5, 0.25, 0.25, t], np.float32)
        p = r[None, None, :].copy()
        res = oracle.tree_accept_stochastic(np.array([[-1]], np.int32), np.zeros((1, 1), np.int32),
                                            np.array([1], np.int32), p, p.copy(),
                                            np.zeros((1, 1), np.float32), np.array([ub], np.float32))
        if int(res[2][0]) != want_idx or bool(res[4][0]) != want_flag:
            return False
    return True


ALL_PINS = {
    "tree_example": pin_tree_example,
    "tree_closed_forms": pin_tree_closed_forms,
    "tree_bruteforce": lambda: pin_tree_bruteforce(0),
    "tree_status": pin_tree_status,
    "attn_path_invariant": pin_attn_path_invariant,
    "attn_chain_is_causal": pin_attn_chain_is_causal,
    "attn_star": pin_attn_star,
    "attn_empty_prefix": pin_attn_empty_prefix,
    "attn_one_hot_mask": pin_attn_one_hot_mask,
    "attn_sibling_relabel": pin_attn_sibling_relabel,
    "attn_one_matches_full": pin_attn_one_matches_full,
    "expand_bruteforce": pin_expand_bruteforce,
    "expand_closed_forms": pin_expand_closed_forms,
    "expand_value_is_path_product": pin_expand_value_is_path_product,
    "expand_invariants": pin_expand_invariants,
    "expand_nonfinite": pin_expand_nonfinite,
    "accept_bruteforce": pin_accept_bruteforce,
    "accept_closed_forms": pin_accept_closed_forms,
    "compact_chain": pin_compact_chain,
    "compact_root_only": pin_compact_root_only,
    "compact_root_path": pin_compact_root_path,
    "compact_edges": pin_compact_edges,
    "stochastic_greedy_limit": pin_stochastic_greedy_limit,
    "stochastic_hand_example": pin_stochastic_hand_example,
    "stochastic_preserves_target": pin_stochastic_preserves_target,
    "budget_limits": pin_budget_limits,
    "budget_first_failure_stops": pin_budget_first_failure_stops,
    "stop_means_deepest_level_kept": pin_stop_means_deepest_level_kept,
    "stop_is_lossless": pin_stop_is_lossless,
    "stop_limits": pin_stop_limits,
    "candidates_exact_dots": pin_candidates_exact_dots,
    "candidates_low_rank_exact": pin_candidates_low_rank_exact,
    "candidates_all_exact": pin_candidates_all_exact,
    "expand_midpoint_flag": pin_expand_midpoint_flag,
    "candidates_midpoint_flag": pin_candidates_midpoint_flag,
    "stochastic_margins": pin_stochastic_margins,
}


def failing_pins(names=None):
    """Names of pins that fail (or raise) -- used by the mutation tests."""
    bad = []
    for name, fn in ALL_PINS.items():
        if names is not None and name not in names:
            continue
        try:
            if not fn():
                bad.append(name)
        except Exception:
            bad.append(name)
    return bad
