"""HIP path against the oracle, through the C ABI, on the GPU.

Integer outputs (bitsets, depths, positions, statuses, selected nodes, tokens,
accepted lengths, paths) and the float32 expansion scores must match bit for bit;
attention outputs must satisfy max|err| <= 2e-2 and max|err| <= 1e-2 * max|oracle|.
"""

import numpy as np
import pytest
import torch

import oracle
import oracle.attention
import synth
import tree_attention_verify_ancestor_amd as tv
from gpu_helpers import (DEV, anc_u64, attn_close, attn_device_inputs, dev_i32, dev_i64,
                         dev_input, host, run_attn, run_expand)

pytestmark = pytest.mark.gpu


# ----------------------------------------------------------------------------- tree_build

def _check_build(parent, n_nodes, prefix_len=None):
    anc_r, dep_r, pos_r, st_r = oracle.tree_build(parent, n_nodes, prefix_len)
    anc, dep, pos, st = tv.tree_build(dev_i32(parent), dev_i32(n_nodes),
                                      None if prefix_len is None else dev_i32(prefix_len))
    torch.cuda.synchronize()
    assert np.array_equal(st.cpu().numpy(), st_r)
    assert np.array_equal(anc_u64(anc), anc_r)
    assert np.array_equal(dep.cpu().numpy(), dep_r)
    if prefix_len is not None:
        assert np.array_equal(pos.cpu().numpy(), pos_r)


def test_tree_build_static_workloads():
    for wid in (1, 2):
        w = synth.WORKLOADS[wid]
        parent, nn = synth.static_tree(w)
        _check_build(parent, nn, synth.prefix_lengths(w).astype(np.int32))


@pytest.mark.parametrize("n_max", [64, 37, 1])
def test_tree_build_random(n_max):
    rng = np.random.default_rng(100 + n_max)
    B = 257
    parent = np.full((B, n_max), -1, dtype=np.int32)
    nn = rng.integers(1, n_max + 1, size=B).astype(np.int32)
    for b in range(B):
        parent[b, :nn[b]] = synth.random_parents(rng, int(nn[b]), ["random", "chain", "star", "broom"][b % 4])
        parent[b, nn[b]:] = rng.integers(-3, 70, size=n_max - nn[b])        # padding is ignored
    _check_build(parent, nn, rng.integers(0, 100000, size=B).astype(np.int32))


def test_tree_build_malformed():
    cases = [([-1, 0, 1], 3), ([0, 0, 1], 3), ([-1, 0, 2], 3), ([-1, 2, 0], 3), ([-1, -5, 0], 3),
             ([-1, 0, -1], 3), ([-1, -1, 7], 3), ([-1, 0, 1], 0), ([-1, 0, 1], 65), ([-1, 0, 1], -4),
             ([-1] + [0] * 63, 64), ([-1, 0, 1, 2, 64], 5)]
    parent = np.full((len(cases), 64), -1, dtype=np.int32)
    nn = np.zeros(len(cases), dtype=np.int32)
    for b, (p, n) in enumerate(cases):
        parent[b, :len(p)] = p
        nn[b] = n
    _check_build(parent, nn, np.arange(len(cases), dtype=np.int32))


# ----------------------------------------------------------------------------- tree_accept

def _check_accept(parent, token, target, nn):
    r = oracle.tree_accept(parent, token, target, nn)
    par = dev_i32(parent)
    d_nn = dev_i32(nn)
    anc, depth, pos, st = tv.tree_build(par, d_nn)
    got = tv.tree_accept(par, depth, anc, d_nn, dev_i32(token), dev_i32(target))
    torch.cuda.synchronize()
    for g, e, name in zip(got, r, ("accept_len", "best", "bonus", "path")):
        assert np.array_equal(g.cpu().numpy(), e), name


@pytest.mark.parametrize("vocab", [2, 3, 7, 32000])
def test_accept_random(vocab):
    rng = np.random.default_rng(200 + vocab)
    B = 300
    parent = np.full((B, 64), -1, dtype=np.int32)
    nn = rng.integers(1, 65, size=B).astype(np.int32)
    for b in range(B):
        parent[b, :nn[b]] = synth.random_parents(rng, int(nn[b]), ["random", "chain", "star", "broom"][b % 4])
    token = rng.integers(0, vocab, size=(B, 64)).astype(np.int32)
    target = rng.integers(0, vocab, size=(B, 64)).astype(np.int32)
    nn[::37] = 0                           # invalid trees give -1 everywhere
    _check_accept(parent, token, target, nn)


def test_accept_workload_targets():
    for wid in (1, 2):
        w = synth.WORKLOADS[wid]
        parent, nn = synth.static_tree(w)
        tok = synth.static_draft_tokens(w)
        _check_accept(parent, tok, synth.target_ids(w, parent, tok, nn), nn)


def test_accept_full_chain_and_no_match():
    n = 64
    parent = np.stack([synth.random_parents(None, n, "chain")] * 2)
    token = np.stack([np.arange(100, 164, dtype=np.int32)] * 2)
    target = np.stack([np.roll(token[0], -1), np.full(64, 7, np.int32)])
    _check_accept(parent, token, target, np.array([n, n], np.int32))


# ----------------------------------------------------------------------------- expansion

def _check_expand(levels, k, m, roots, m_per_seq=None, budget_log=None):
    ref = oracle.expand_rerank(levels, k, m if m_per_seq is None else m_per_seq, roots,
                               budget_log=budget_log)
    out, fronts = run_expand(levels, k, m, roots, m_per_seq=m_per_seq, budget_log=budget_log)
    st = out.seq_status.cpu().numpy()
    assert np.array_equal(st, ref.status)
    n = out.n_nodes.cpu().numpy()
    assert np.array_equal(n, ref.n_nodes)
    # sequences whose log-normaliser lies next to a float32 midpoint are compared on
    # status and size only; none does on these seeds
    assert not ref.indeterminate.any(), f"{int(ref.indeterminate.sum())} sequences excluded"
    ok = ~ref.indeterminate
    assert np.array_equal(out.parent.cpu().numpy()[ok], ref.parent[ok])
    assert np.array_equal(out.token.cpu().numpy()[ok], ref.token[ok])
    assert out.score.cpu().numpy()[ok].tobytes() == ref.score[ok].tobytes()
    for s in range(len(levels)):
        assert np.array_equal(fronts[s][ok], ref.frontier_tokens[s][ok]), f"frontier {s}"
    return ref


SMALL_EXPAND = [  # (B, k, S, V, m, quantised)
    (3, 1, 4, 16, 64, True), (3, 2, 3, 16, 9, True), (4, 3, 3, 16, 64, True),
    (2, 5, 4, 100, 30, False), (5, 8, 3, 1000, 64, False), (2, 10, 4, 777, 40, True),
    (2, 16, 2, 4096, 64, False), (3, 4, 5, 33, 2, True), (2, 6, 6, 50, 1, False),
    # rows split over many chunks: ties across lanes, waves and chunks; odd vocab sizes
    (2, 10, 3, 50000, 40, True), (3, 4, 3, 20001, 16, True), (1, 16, 2, 9001, 64, False),
    (1, 2, 2, 600000, 4, True), (1, 3, 2, 600001, 5, False),
    # fewer lanes hold logits than k: every logit of the chunk is a candidate
    (2, 8, 3, 16, 20, False), (2, 16, 2, 40, 30, False),
]


@pytest.mark.parametrize("case", SMALL_EXPAND)
def test_expand_small(case):
    B, k, S, V, m, quant = case
    rng = np.random.default_rng(hash(case) % (2 ** 32))
    levels = []
    for s in range(S):
        shape = (B, 1 if s == 0 else k, V)
        if quant:
            levels.append((rng.integers(-6, 7, size=shape) * 0.5).astype(np.float32))
        else:
            levels.append((rng.standard_normal(shape) * 2).astype(np.float32))
    _check_expand(levels, k, m, rng.integers(0, V, size=B))


@pytest.mark.parametrize("V", [64, 40000])
def test_expand_nonfinite_and_m_per_seq(V):
    rng = np.random.default_rng(7)
    B, k, S = 4, 3, 3
    levels = [(rng.standard_normal((B, 1 if s == 0 else k, V)) * 2).astype(np.float32) for s in range(S)]
    levels[1][1, 2, 11 * V // 64] = np.nan
    levels[2][2, 0, V - 1] = np.inf
    m_seq = np.array([5, 20, 64, 70], dtype=np.int32)          # the last is out of range
    _check_expand(levels, k, 64, rng.integers(0, V, size=B), m_per_seq=m_seq)


@pytest.mark.parametrize("wid", [3, 4, 5])
def test_expand_workload(wid):
    w = synth.WORKLOADS[wid]
    kc = synth.kept_counts(w) if isinstance(w.m, tuple) else None
    ref = _check_expand(synth.draft_logits(w), w.k, w.m if kc is None else 64,
                        synth.root_tokens(w), m_per_seq=kc)
    assert not ref.indeterminate.any()


# ----------------------------------------------------------------------------- attention

def _check_attn(inp, parent, nn, what, lse_too=True):
    ref, ref_lse = oracle.tree_verify_attn(inp.f32("q"), inp.f32("k_tree"), inp.f32("v_tree"),
                                           inp.f32("k_prefix"), inp.f32("v_prefix"),
                                           inp.prefix_offsets, parent, nn)
    lens = np.diff(inp.prefix_offsets)
    out, lse, st, _ = run_attn(attn_device_inputs(inp), parent, nn, int(lens.max()))
    assert np.all(st.cpu().numpy() == 0)
    ok, msg = attn_close(host(out), ref, what)
    assert ok, msg
    if lse_too:
        err = np.max(np.abs(lse.cpu().numpy().astype(np.float64) - ref_lse))
        assert err <= 2e-2, f"{what} lse err {err}"
    return out, lse


SMALL_ATTN = [  # (B, Hq, Hkv, D, prefix lengths, node counts)
    (1, 1, 1, 128, (0,), (1,)),
    (1, 2, 2, 128, (1,), (10,)),
    (2, 8, 2, 128, (63, 65), (33, 64)),
    (3, 32, 8, 128, (300, 1, 777), (60, 7, 64)),
    (2, 8, 1, 128, (1000, 2049), (64, 17)),
    (4, 4, 4, 64, (129, 0, 64, 511), (26, 64, 1, 40)),
    (2, 16, 2, 64, (5000, 300), (64, 50)),
    (1, 32, 32, 128, (2048,), (26,)),
    (5, 64, 8, 128, (700, 10, 1500, 64, 0), (64, 3, 64, 32, 64)),
    # 65..128 rows per KV head (eight waves as four row groups x two key halves)
    (2, 4, 2, 64, (300, 1000), (64, 40)),
    (1, 6, 3, 128, (777,), (50,)),
    # one sequence with 240 rows per KV head: 64-row units, one workgroup per CU
    (1, 32, 8, 128, (3000,), (60,)),
    # eight or more sequences: ragged ones take their (sequence, chunk) pairs by work
    (9, 8, 2, 128, (3000, 17, 0, 900, 2500, 64, 1200, 5, 640), (64, 3, 20, 64, 1, 33, 50, 64, 10)),
    (12, 16, 4, 64, (100, 2000, 50, 700, 1, 0, 3000, 256, 128, 900, 1500, 30),
     (5, 64, 30, 12, 64, 2, 40, 64, 7, 19, 64, 26)),
    (8, 4, 4, 64, (500,) * 8, (20,) * 8),
    # 1024 rows per KV head, four 256-row blocks: trees filling all four take two key
    # chunks per workgroup, the others one
    (4, 32, 2, 128, (3000, 2100, 777, 0), (64, 40, 1, 61)),
    (4, 32, 2, 64, (1500, 3000, 0, 2500), (61, 64, 50, 64)),
]


@pytest.mark.parametrize("case", SMALL_ATTN)
def test_attn_small_bf16(case):
    B, Hq, Hkv, D, lens, ns = case
    inp, parent, nn = synth.random_attention_case(abs(hash(case)) % 10000, B, Hq, Hkv, D, lens, ns,
                                                  dtype="bf16", std=0.5)
    _check_attn(inp, parent, nn, f"case {case}")


@pytest.mark.parametrize("D", [64, 128])
def test_attn_few_rows(D):
    """At most 32 rows per KV head (n_max 16, one query head per KV head): four waves
    split each stage's keys and merge through LDS."""
    inp, parent, nn = synth.random_attention_case(4242 + D, 3, 2, 2, D, (100, 0, 2500), (16, 9, 16),
                                                  dtype="bf16", std=0.5, n_max=16)
    _check_attn(inp, parent, nn, f"few rows D={D}")


@pytest.mark.parametrize("std", [0.5, 2.0])
def test_attn_fp32(std):
    inp, parent, nn = synth.random_attention_case(17, 3, 4, 2, 64, (32, 0, 333), (10, 64, 5),
                                                  dtype="f32", std=std)
    _check_attn(inp, parent, nn, "fp32")


def test_attn_tiny_workload():
    w = synth.WORKLOADS[1]
    parent, nn = synth.static_tree(w)
    _check_attn(synth.attention_inputs(w), parent, nn, "workload 1")


# Every launch shape of tree_verify_attn (name: batch, n_max, query heads per KV head, KV
# heads, and the plan's waves / row groups / key splits / 32-row tiles per wave).
ATTN_SHAPES = {
    "32 rows: four waves split the keys": (2, 32, 1, 2, (4, 1, 4, 1)),
    "64 rows: four waves, two tiles each": (2, 64, 1, 2, (4, 1, 4, 2)),
    "256 rows in few units: 64-row units": (2, 64, 4, 2, (4, 1, 4, 2)),
    "128 rows: four row groups x two key halves": (2, 64, 2, 2, (8, 4, 2, 1)),
    "512 rows: eight waves of one tile": (4, 64, 8, 8, (8, 8, 1, 1)),
    "1024 rows: four row blocks of eight waves": (4, 64, 16, 2, (8, 8, 1, 1)),
}
# the same shapes with nine ragged sequences (ranked by work where eight waves own one
# tile each: the ranking applies from eight sequences on)
RAGGED_SHAPES = {
    "32 rows": (32, 1, 2, (4, 1, 4, 1)),
    "64 rows": (64, 1, 2, (4, 1, 4, 2)),
    "256 rows in few units": (64, 4, 1, (4, 1, 4, 2)),
    "128 rows": (64, 2, 2, (8, 4, 2, 1)),
    "512 rows": (64, 8, 8, (8, 8, 1, 1)),
}
RAGGED_LENS = (3000, 17, 0, 900, 2500, 64, 1200, 5, 640)


def _plan_of(B, n_max, G, Hkv, D, lens):
    p = tv.attn_plan(B, n_max, G * Hkv, Hkv, D, int(max(lens)))
    return p, (p["waves"], p["row_groups"], p["key_splits"], p["tiles_per_wave"])


def _one_hot_inputs(seed, B, n_max, G, Hkv, D, lens, ns):
    """Tree V rows are unit vectors: node j's V is e_j; prefix V is 0 in coordinates
    0..63.  Then out[i][h][j] (j < 64) is i's softmax weight of node j: exactly 0 off
    i's root path and > 0 on it, whatever the tolerance."""
    inp, parent, nn = synth.random_attention_case(seed, B, G * Hkv, Hkv, D, lens, ns, dtype="bf16",
                                                  std=0.5, n_max=n_max)
    one = synth.bf16_bits(np.float32([1.0]))[0]
    inp.v_tree[:, :, :, :64] = 0
    for j in range(n_max):
        inp.v_tree[:, j, :, j] = one
    inp.v_prefix[:, :, :64] = 0
    return inp, parent, nn


def _assert_one_hot(o, parent, nn, n_max):
    anc, _, _, _ = oracle.tree_build(parent, nn, None)
    for b in range(len(nn)):
        for i in range(int(nn[b])):
            on = np.array([(int(anc[b, i]) >> j) & 1 for j in range(n_max)], dtype=bool)
            blk = o[b, i, :, :n_max]
            assert np.all(blk[:, ~on] == 0.0), ("leak", b, i, np.nonzero(blk[:, ~on])[1][:5])
            assert np.all(blk[:, on] > 0.0), ("lost", b, i)
            assert np.all(o[b, i, :, n_max:64] == 0.0), (b, i)
        assert np.all(o[b, int(nn[b]):] == 0.0), ("padding", b)


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("shape", list(ATTN_SHAPES))
def test_attn_one_hot_mask_exact(shape, D):
    """The exact mask probe on every launch shape, with prefixes of several key chunks."""
    B, n_max, G, Hkv, want = ATTN_SHAPES[shape]
    lens = (3000, 1777) if B == 2 else (3000, 2100, 777, 0)
    ns = (n_max, n_max - 5) if B == 2 else (n_max, 40, 1, n_max - 3)
    plan, got = _plan_of(B, n_max, G, Hkv, D, lens)
    assert got == want and plan["n_chunks"] > 1, plan
    inp, parent, nn = _one_hot_inputs(31 + G + D + n_max, B, n_max, G, Hkv, D, lens, ns)
    out, _, st, _ = run_attn(attn_device_inputs(inp), parent, nn, max(lens))
    assert np.all(st.cpu().numpy() == 0)
    _assert_one_hot(host(out), parent, nn, n_max)


@pytest.mark.parametrize("shape", list(RAGGED_SHAPES))
def test_attn_ragged_marker_exact(shape):
    """Nine ragged sequences (prefix 0..3000): sequence b's prefix V carries 1 in
    coordinate 64 + b and every other prefix and tree V is 0 in coordinates 64..127, so
    out[b'][i][h][64 + b] must be exactly 0 for every b' != b (no sequence sees another's
    prefix) and > 0 for b' == b with a prefix.  The tree one-hot probe runs beside it in
    coordinates 0..63."""
    n_max, G, Hkv, want = RAGGED_SHAPES[shape]
    B, D = 9, 128
    base = (64, 3, 20, 64, 1, 33, 50, 64, 10)
    ns = tuple(min(n, n_max) for n in base)
    plan, got = _plan_of(B, n_max, G, Hkv, D, RAGGED_LENS)
    assert got == want, plan
    inp, parent, nn = _one_hot_inputs(500 + n_max + G, B, n_max, G, Hkv, D, RAGGED_LENS, ns)
    one = synth.bf16_bits(np.float32([1.0]))[0]
    inp.v_tree[:, :, :, 64:] = 0
    inp.v_prefix[:, :, 64:] = 0
    offs = inp.prefix_offsets
    for b in range(B):
        inp.v_prefix[offs[b]:offs[b + 1], :, 64 + b] = one
    out, _, st, _ = run_attn(attn_device_inputs(inp), parent, nn, max(RAGGED_LENS))
    assert np.all(st.cpu().numpy() == 0)
    o = host(out)
    _assert_one_hot(o, parent, nn, n_max)
    for bp in range(B):
        rows = o[bp, :int(nn[bp])]
        for b in range(B):
            col = rows[:, :, 64 + b]
            if b != bp:
                assert np.all(col == 0.0), ("marker of", b, "seen by", bp)
            elif RAGGED_LENS[b] > 0:
                assert np.all(col > 0.0), ("own marker lost", b)
            else:
                assert np.all(col == 0.0), b
        assert np.all(rows[:, :, 64 + B:] == 0.0), bp


@pytest.mark.parametrize("ragged", [False, True])
def test_attn_negative_prefix_offset(ragged):
    """A sequence whose prefix offset is negative fails with TV_SEQ_BAD_PREFIX and its
    rows are zero; nothing before the prefix buffer is read, and the other sequences are
    exact (a ragged batch of nine takes the ranked order, whose work weights read the
    offsets too)."""
    B = 9 if ragged else 3
    lens = RAGGED_LENS if ragged else (900, 1500, 64)
    ns = (64, 3, 20, 64, 1, 33, 50, 64, 10) if ragged else (64, 30, 64)
    inp, parent, nn = synth.random_attention_case(71 + B, B, 64, 8, 128, lens, ns, std=0.5)
    bad = 1
    offs = inp.prefix_offsets.copy()
    offs[bad] = -64                          # a valid length past the front of the buffer
    good = [b for b in range(B) if b != bad and offs[b + 1] - offs[b] == lens[b]]
    d = attn_device_inputs(inp)
    d["offsets"] = dev_i64(offs)
    out, lse, st, _ = run_attn(d, parent, nn, int(max(offs[b + 1] - offs[b] for b in range(B))))
    st = st.cpu().numpy()
    assert st[bad] == 5                                           # TV_SEQ_BAD_PREFIX
    o = host(out)
    assert np.all(o[bad] == 0.0) and np.all(lse.cpu().numpy()[bad] == 0.0)
    ref, _ = oracle.tree_verify_attn(inp.f32("q"), inp.f32("k_tree"), inp.f32("v_tree"),
                                     inp.f32("k_prefix"), inp.f32("v_prefix"), offs, parent, nn,
                                     batches=good)
    for b in good:
        assert st[b] == 0
        ok, msg = attn_close(o[b], ref[b], f"sequence {b}")
        assert ok, msg


def test_attn_negative_prefix_offset_fp32():
    inp, parent, nn = synth.random_attention_case(73, 3, 4, 2, 64, (40, 100, 7), (10, 64, 5),
                                                  dtype="f32", std=0.5)
    offs = inp.prefix_offsets.copy()
    offs[0] = -8
    d = attn_device_inputs(inp)
    d["offsets"] = dev_i64(offs)
    out, lse, st, _ = run_attn(d, parent, nn, 100)
    st = st.cpu().numpy()
    assert st[0] == 5 and st[1] == 0 and st[2] == 0
    o = host(out)
    assert np.all(o[0] == 0.0)
    ref, _ = oracle.tree_verify_attn(inp.q, inp.k_tree, inp.v_tree, inp.k_prefix, inp.v_prefix,
                                     offs, parent, nn, batches=[1, 2])
    for b in (1, 2):
        ok, msg = attn_close(o[b], ref[b], f"fp32 sequence {b}")
        assert ok, msg


@pytest.mark.parametrize("G,n_max", [(8, 64), (4, 30), (1, 64), (1, 20)])
def test_attn_score_outliers(G, n_max):
    """Keys whose scores lie far above every earlier key of their chunk: beyond the
    range a fixed per-chunk softmax reference can carry, so the rows involved must be
    recomputed exactly (here the weights are nearly one-hot on the outliers)."""
    Hkv = 2
    inp, parent, nn = synth.random_attention_case(77 + G, 2, G * Hkv, Hkv, 128, (5000, 700),
                                                  (n_max, n_max - 3), std=0.5, n_max=n_max)
    u = synth.bf16_bits(np.full(128, 0.7, np.float32))
    big = synth.bf16_bits(np.full(128, 5.6, np.float32))       # score 8x that of u.u
    inp.q[:] = u
    inp.k_prefix[4321, 1] = big                                # a late prefix key, head 1
    inp.k_prefix[5000 + 650, 0] = big                          # sequence 1, head 0
    inp.k_tree[0, n_max - 1, 0] = big                          # the deepest tree slot
    _check_attn(inp, parent, nn, f"outliers G={G} n_max={n_max}")


def test_attn_deterministic():
    inp, parent, nn = synth.random_attention_case(5, 3, 32, 8, 128, (3000, 100, 4097), (64, 20, 50))
    d = attn_device_inputs(inp)
    a1, l1, _, _ = run_attn(d, parent, nn, 4097)
    a2, l2, _, _ = run_attn(d, parent, nn, 4097)
    assert torch.equal(a1.view(torch.int16), a2.view(torch.int16)) and torch.equal(l1, l2)


def test_attn_workspace_reused():
    """Consecutive calls on one workspace (whose chunk counters each call must leave
    cleared) give the same, correct results -- also with different trees in between."""
    inp, parent, nn = synth.random_attention_case(11, 2, 16, 16, 128, (2048, 1500), (26, 40))
    d = attn_device_inputs(inp)
    ws = tv.attn_workspace(torch.bfloat16, 2, 64, 16, 16, 128, 2048)
    ref, _ = oracle.tree_verify_attn(inp.f32("q"), inp.f32("k_tree"), inp.f32("v_tree"),
                                     inp.f32("k_prefix"), inp.f32("v_prefix"),
                                     inp.prefix_offsets, parent, nn)
    par, nnd = dev_i32(parent), dev_i32(nn)
    anc, _, _, _ = tv.tree_build(par, nnd)
    outs = []
    for _ in range(3):
        out, _, _ = tv.tree_verify_attn(d["q"], d["k_tree"], d["v_tree"], d["k_prefix"],
                                        d["v_prefix"], d["offsets"], nnd, anc, 2048, ws=ws)
        torch.cuda.synchronize()
        outs.append(host(out))
    for o in outs:
        ok, msg = attn_close(o, ref, "workspace reuse")
        assert ok, msg
    assert np.array_equal(outs[0], outs[2])


def test_attn_workload2_full():
    w = synth.WORKLOADS[2]
    parent, nn = synth.static_tree(w)
    _check_attn(synth.attention_inputs(w), parent, nn, "workload 2")


def test_attn_workload3_full():
    w = synth.WORKLOADS[3]
    ref = oracle.expand_rerank(synth.draft_logits(w), w.k, w.m, synth.root_tokens(w))
    _check_attn(synth.attention_inputs(w), ref.parent, ref.n_nodes, "workload 3")


@pytest.mark.slow
@pytest.mark.parametrize("wid", [4, 5])
def test_attn_workload_full(wid):
    """Full-size workloads 4 and 5 in the bench's launch configuration (trees from the
    workload's expansion, max prefix = the longest sequence), every output element and
    lse against the float64 oracle."""
    w = synth.WORKLOADS[wid]
    kc = synth.kept_counts(w) if isinstance(w.m, tuple) else None
    tree = oracle.expand_rerank(synth.draft_logits(w), w.k, w.m if kc is None else kc,
                                synth.root_tokens(w))
    inp = synth.attention_inputs(w)
    _check_attn(inp, tree.parent, tree.n_nodes, f"workload {wid}")


# ----------------------------------------------------------------------------- whole path

def test_pipeline_workload3():
    """expand x S -> tree_build -> tree_verify_attn -> tree_accept, all on the GPU."""
    w = synth.WORKLOADS[3]
    levels = synth.draft_logits(w)
    roots = synth.root_tokens(w)
    ref_tree = oracle.expand_rerank(levels, w.k, w.m, roots)
    out, _ = run_expand(levels, w.k, w.m, roots)
    anc, depth, pos, st = tv.tree_build(out.parent, out.n_nodes)
    inp = synth.attention_inputs(w)
    d = attn_device_inputs(inp)
    att, lse, ast = tv.tree_verify_attn(d["q"], d["k_tree"], d["v_tree"], d["k_prefix"],
                                        d["v_prefix"], d["offsets"], out.n_nodes, anc, w.prefix)
    tgt = synth.target_ids(w, ref_tree.parent, ref_tree.token, ref_tree.n_nodes)
    acc = tv.tree_accept(out.parent, depth, anc, out.n_nodes, out.token, dev_i32(tgt))
    torch.cuda.synchronize()
    ref_attn, _ = oracle.tree_verify_attn(inp.f32("q"), inp.f32("k_tree"), inp.f32("v_tree"),
                                          inp.f32("k_prefix"), inp.f32("v_prefix"),
                                          inp.prefix_offsets, ref_tree.parent, ref_tree.n_nodes)
    ok, msg = attn_close(host(att), ref_attn, "pipeline")
    assert ok, msg
    ref_acc = oracle.tree_accept(ref_tree.parent, ref_tree.token, tgt, ref_tree.n_nodes)
    for g, e in zip(acc, ref_acc):
        assert np.array_equal(g.cpu().numpy(), e)


# ----------------------------------------------------------------------------- KV compaction

@pytest.mark.parametrize("dtype,D,Hkv", [("bf16", 128, 8), ("f32", 64, 2), ("bf16", 64, 1)])
def test_kv_compact_after_accept(dtype, D, Hkv):
    """tree_build -> tree_accept -> tree_kv_compact on the device against the oracle's
    accept and compaction, bit for bit on the destination (written and untouched rows),
    with one sequence's rows running past the end of the destination."""
    rng = np.random.default_rng(900 + D + Hkv)
    B, n_max = 7, 64
    parent = np.full((B, n_max), -1, np.int32)
    nn = rng.integers(1, n_max + 1, size=B).astype(np.int32)
    nn[0], nn[1] = 1, 64
    for b in range(B):
        for i in range(1, int(nn[b])):
            parent[b, i] = rng.integers(max(0, i - 3), i)                # deep, narrow trees
    tok = rng.integers(0, 3, size=(B, n_max)).astype(np.int32)
    tgt = rng.integers(0, 3, size=(B, n_max)).astype(np.int32)
    parent[1, 1:] = np.arange(63)                                        # sequence 1: a chain whose
    tgt[1, :63] = tok[1, 1:]                                             # every token passes
    draw = (lambda s: synth.bf16_bits(rng.standard_normal(s).astype(np.float32))) if dtype == "bf16" \
        else (lambda s: rng.standard_normal(s).astype(np.float32))
    kt, vt = draw((B, n_max, Hkv, D)), draw((B, n_max, Hkv, D))
    rows = 70 * B
    kd, vd = draw((rows, Hkv, D)), draw((rows, Hkv, D))
    dst = (np.arange(B) * 70).astype(np.int64)
    dst[B - 1] = rows - 5                                                # only five rows fit

    alen_r, best_r, _, path_r = oracle.tree_accept(parent, tok, tgt, nn)
    kd_r, vd_r = oracle.kv_compact(kt, vt, path_r, alen_r, kd, vd, dst)

    par_d, nn_d = dev_i32(parent), dev_i32(nn)
    anc, depth, _, _ = tv.tree_build(par_d, nn_d)
    alen, best, _, path = tv.tree_accept(par_d, depth, anc, nn_d, dev_i32(tok), dev_i32(tgt))
    k_dst, v_dst = dev_input(kd, dtype), dev_input(vd, dtype)
    tv.tree_kv_compact(dev_input(kt, dtype), dev_input(vt, dtype), path, alen, k_dst, v_dst,
                       torch.from_numpy(dst).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(alen.cpu().numpy(), alen_r)
    bits = (lambda t: t.view(torch.int16).cpu().numpy().view(np.uint16)) if dtype == "bf16" \
        else (lambda t: t.cpu().numpy())
    assert np.array_equal(bits(k_dst), kd_r)
    assert np.array_equal(bits(v_dst), vd_r)
    assert alen_r[1] == 63 and alen_r[0] == 0                            # whole chain; root only


def test_kv_compact_rejected_tree_copies_nothing():
    B, n_max, Hkv, D = 2, 64, 2, 64
    kt = torch.randn((B, n_max, Hkv, D), device=DEV).to(torch.bfloat16)
    vt = torch.randn((B, n_max, Hkv, D), device=DEV).to(torch.bfloat16)
    kd = torch.zeros((100, Hkv, D), device=DEV, dtype=torch.bfloat16)
    vd = torch.zeros((100, Hkv, D), device=DEV, dtype=torch.bfloat16)
    path = torch.full((B, n_max), -1, dtype=torch.int32, device=DEV)
    alen = torch.tensor([-1, 0], dtype=torch.int32, device=DEV)
    dst = torch.tensor([0, 50], dtype=torch.int64, device=DEV)
    tv.tree_kv_compact(kt, vt, path, alen, kd, vd, dst)
    torch.cuda.synchronize()
    written = torch.zeros(100, dtype=torch.bool)
    written[50] = True
    assert torch.equal(kd[50], kt[1, 0]) and torch.equal(vd[50], vt[1, 0])
    assert torch.count_nonzero(kd[~written.to(DEV)]) == 0 and torch.count_nonzero(vd[~written.to(DEV)]) == 0


# ----------------------------------------------------------------------------- stochastic acceptance

def _stochastic_case(seed, B, V, n_max=64, scale=2.0, one_hot=False):
    """Random trees whose children's tokens are drawn (without repeats) from the draft
    distribution of their parent; target rows close to the draft rows, so that about
    half of the candidates pass."""
    rng = np.random.default_rng(seed)
    parent = np.full((B, n_max), -1, np.int32)
    nn = rng.integers(1, n_max + 1, size=B).astype(np.int32)
    for b in range(B):
        for i in range(1, int(nn[b])):
            parent[b, i] = rng.integers(max(0, i - 6), i)
    lq = rng.standard_normal((B, n_max, V)) * scale
    lp = lq + rng.standard_normal((B, n_max, V)) * 0.7
    sm = lambda x: (np.exp(x - x.max(-1, keepdims=True)) / np.exp(x - x.max(-1, keepdims=True)).sum(-1, keepdims=True))
    q = sm(lq).astype(np.float32)
    p = sm(lp).astype(np.float32)
    tgt = rng.integers(0, V, size=(B, n_max)).astype(np.int32)
    if one_hot:
        p = np.zeros_like(p)
        p[np.arange(B)[:, None], np.arange(n_max)[None, :], tgt] = 1.0
    tok = np.zeros((B, n_max), np.int32)
    for b in range(B):
        for u in range(int(nn[b])):
            kids = [c for c in range(1, int(nn[b])) if parent[b, c] == u]
            if kids:
                w = q[b, u].astype(np.float64)
                tok[b, kids] = rng.choice(V, size=len(kids), replace=False, p=w / w.sum())
        if one_hot:                        # make some children match the target
            for c in range(1, int(nn[b])):
                if rng.random() < 0.6:
                    sib = [s for s in range(1, int(nn[b])) if parent[b, s] == parent[b, c] and s != c]
                    if tgt[b, parent[b, c]] not in tok[b, sib]:
                        tok[b, c] = tgt[b, parent[b, c]]
    ua = rng.random((B, n_max)).astype(np.float32)
    ub = rng.random(B).astype(np.float32)
    return parent, nn, tok, tgt, p, q, ua, ub


def _run_stochastic(parent, nn, tok, p, q, ua, ub, split=True):
    par_d, nn_d = dev_i32(parent), dev_i32(nn)
    anc, _, _, _ = tv.tree_build(par_d, nn_d)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)
    out = tv.tree_accept_stochastic(par_d, anc, nn_d, dev_i32(tok), f(p), f(q), f(ua), f(ub),
                                    split=split)
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in out]


# split: the vocabulary over several workgroups per sequence where the workspace query
# asks for one (every case here but the two smallest vocabularies); False: one
# workgroup per sequence
SPLIT = [pytest.param(True, id="split"), pytest.param(False, id="onewg")]


@pytest.mark.parametrize("split", SPLIT)
@pytest.mark.parametrize("seed,B,V", [(1, 6, 1000), (2, 4, 5000), (3, 2, 32000), (4, 8, 37),
                                      (5, 32, 32000), (6, 1, 32000)])
def test_accept_stochastic_matches_oracle(seed, B, V, split):
    parent, nn, tok, tgt, p, q, ua, ub = _stochastic_case(seed, B, V)
    alen_r, best_r, bonus_r, path_r, indet = oracle.tree_accept_stochastic(parent, tok, nn, p, q, ua, ub)
    alen, best, bonus, path = _run_stochastic(parent, nn, tok, p, q, ua, ub, split)
    assert not indet.any(), f"{int(indet.sum())} sequences excluded"     # none on these seeds
    ok = ~indet
    assert np.array_equal(alen[ok], alen_r[ok])
    assert np.array_equal(best[ok], best_r[ok])
    assert np.array_equal(bonus[ok], bonus_r[ok])
    assert np.array_equal(path[ok], path_r[ok])
    assert alen_r.max() >= 1                                         # some candidates passed


@pytest.mark.parametrize("split", SPLIT)
def test_accept_stochastic_workload4_vocab(split):
    """The 70B-shaped workload's own dynamic trees (four sequences of 64 nodes) over its
    128256-token vocabulary, past the LDS cap, against the oracle bit for bit."""
    w = synth.WORKLOADS[4]
    tree = oracle.expand_rerank(synth.draft_logits(w), w.k, w.m, synth.root_tokens(w))
    B, n_max, V = w.B, w.n_max, w.V
    rng = np.random.default_rng(404)
    lq = rng.standard_normal((B, n_max, V), dtype=np.float32) * np.float32(2.0)
    lp = lq + rng.standard_normal((B, n_max, V), dtype=np.float32) * np.float32(0.7)
    sm = lambda x: (np.exp(x - x.max(-1, keepdims=True)) / np.exp(x - x.max(-1, keepdims=True)).sum(-1, keepdims=True))
    q = sm(lq.astype(np.float64)).astype(np.float32)
    p = sm(lp.astype(np.float64)).astype(np.float32)
    tok = np.zeros((B, n_max), np.int32)
    parent, nn = tree.parent, tree.n_nodes
    for b in range(B):
        for u in range(int(nn[b])):
            kids = [c for c in range(1, int(nn[b])) if parent[b, c] == u]
            if kids:
                wts = q[b, u].astype(np.float64)
                tok[b, kids] = rng.choice(V, size=len(kids), replace=False, p=wts / wts.sum())
    ua = rng.random((B, n_max)).astype(np.float32)
    ub = rng.random(B).astype(np.float32)
    alen_r, best_r, bonus_r, path_r, indet = oracle.tree_accept_stochastic(parent, tok, nn, p, q, ua, ub)
    alen, best, bonus, path = _run_stochastic(parent, nn, tok, p, q, ua, ub, split)
    assert not indet.any(), f"{int(indet.sum())} sequences excluded"
    assert np.array_equal(alen, alen_r) and np.array_equal(best, best_r)
    assert np.array_equal(bonus, bonus_r) and np.array_equal(path, path_r)
    assert alen_r.max() >= 1


@pytest.mark.parametrize("split", SPLIT)
@pytest.mark.parametrize("seed,B,V", [(12, 5, 40000), (13, 3, 200003)])
def test_accept_stochastic_large_vocab(seed, B, V, split):
    """Vocabularies past the LDS cap (weights recomputed from p and q every pass, or
    kept per slice), against the oracle bit for bit."""
    parent, nn, tok, tgt, p, q, ua, ub = _stochastic_case(seed, B, V)
    alen_r, best_r, bonus_r, path_r, indet = oracle.tree_accept_stochastic(parent, tok, nn, p, q, ua, ub)
    alen, best, bonus, path = _run_stochastic(parent, nn, tok, p, q, ua, ub, split)
    assert not indet.any(), f"{int(indet.sum())} sequences excluded"
    assert np.array_equal(alen, alen_r) and np.array_equal(best, best_r)
    assert np.array_equal(bonus, bonus_r) and np.array_equal(path, path_r)


@pytest.mark.parametrize("seed,B,V,n_max", [(21, 128, 16385, 16), (22, 200, 40000, 8)])
def test_accept_stochastic_split_plan_edges(seed, B, V, n_max):
    """The sliced path at its plan's edges: 128 sequences of 16385 tokens take the
    fewest slices it uses (two of 8193 tokens: 256 compute units over 128 sequences,
    16384 tokens of LDS per slice); 200 sequences of 40000 tokens are past the compute
    units and stream with one workgroup each.  Against the oracle bit for bit."""
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    need = tv.lib().tree_accept_stochastic_workspace_size(B, n_max, V)
    if cus >= 256:
        assert (need > 0) == (B == 128), need
    parent, nn, tok, tgt, p, q, ua, ub = _stochastic_case(seed, B, V, n_max=n_max)
    alen_r, best_r, bonus_r, path_r, indet = oracle.tree_accept_stochastic(parent, tok, nn, p, q, ua, ub)
    alen, best, bonus, path = _run_stochastic(parent, nn, tok, p, q, ua, ub, True)
    assert not indet.any(), f"{int(indet.sum())} sequences excluded"
    assert np.array_equal(alen, alen_r) and np.array_equal(best, best_r)
    assert np.array_equal(bonus, bonus_r) and np.array_equal(path, path_r)


@pytest.mark.parametrize("split", SPLIT)
@pytest.mark.parametrize("V", [300, 50000])
def test_accept_stochastic_greedy_limit_equals_tree_accept(V, split):
    """One-hot target rows: the device's stochastic walk equals its greedy acceptance
    (r in LDS, recomputed past the LDS cap, or in slices)."""
    parent, nn, tok, tgt, p, q, ua, ub = _stochastic_case(9, 6, V, one_hot=True)
    alen, best, bonus, path = _run_stochastic(parent, nn, tok, p, q, ua, ub, split)
    par_d, nn_d = dev_i32(parent), dev_i32(nn)
    anc, depth, _, _ = tv.tree_build(par_d, nn_d)
    g = [t.cpu().numpy() for t in tv.tree_accept(par_d, depth, anc, nn_d, dev_i32(tok), dev_i32(tgt))]
    assert np.array_equal(alen, g[0]) and np.array_equal(best, g[1])
    assert np.array_equal(bonus, g[2]) and np.array_equal(path, g[3])
    assert g[0].max() >= 2


@pytest.mark.parametrize("split", SPLIT)
@pytest.mark.parametrize("V", [64, 20000])
def test_accept_stochastic_invalid_tree(V, split):
    parent, nn, tok, tgt, p, q, ua, ub = _stochastic_case(10, 3, V)
    parent[1, 5] = 7                                                 # a forward link: rejected
    nn[2] = 0
    alen, best, bonus, path = _run_stochastic(parent, nn, tok, p, q, ua, ub, split)
    for b in (1, 2):
        assert alen[b] == -1 and best[b] == -1 and bonus[b] == -1 and np.all(path[b] == -1)
    assert alen[0] >= 0


def test_accept_stochastic_split_plan_and_workspace():
    """The workspace query asks for slices where the vocabulary and the batch leave
    room (one 64-bit word triple per sequence, node and slice), none for tiny
    vocabularies or batches past the compute units; a workspace smaller than the query
    is refused."""
    L = tv.lib()
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    assert L.tree_accept_stochastic_workspace_size(1, 64, 300) == 0
    assert L.tree_accept_stochastic_workspace_size(cus + 1, 64, 32000) == 0
    assert L.tree_accept_stochastic_workspace_size(64, 64, 128256) == 0      # 8 slices each
    need = L.tree_accept_stochastic_workspace_size(4, 64, 128256)
    P = min(64, cus // 4)
    assert need == (4 * 64 * P * 24 + 255) // 256 * 256
    parent, nn, tok, tgt, p, q, ua, ub = _stochastic_case(11, 4, 3000)
    par_d, nn_d = dev_i32(parent), dev_i32(nn)
    anc, _, _, _ = tv.tree_build(par_d, nn_d)
    f = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)
    need = L.tree_accept_stochastic_workspace_size(4, 64, 3000)
    assert need > 0
    ws = torch.empty((need,), dtype=torch.uint8, device=DEV)
    outs = [torch.empty(4, dtype=torch.int32, device=DEV) for _ in range(3)]
    args = [4, 64, 3000] + [x.data_ptr() for x in (par_d, anc, nn_d, dev_i32(tok), f(p), f(q), f(ua), f(ub))]
    args += [o.data_ptr() for o in outs] + [None]
    st = L.tree_accept_stochastic(*args, ws.data_ptr(), need - 8, None)
    assert st == 5                                                   # TV_ERR_WORKSPACE
    st = L.tree_accept_stochastic(*args, ws.data_ptr() + 8, need, None)
    assert st == 5                                                   # misaligned
    torch.cuda.synchronize()



# ----------------------------------------------------------------------------- verify budget

@pytest.mark.parametrize("wid", [3, 5])
def test_expand_verify_budget(wid):
    """The final rerank under a verify budget derived from a cost table that grows past
    16 nodes: bit-exact against the oracle, and narrower trees than without it."""
    w = synth.WORKLOADS[wid]
    cost = np.concatenate([np.full(16, 20.0), 20.0 + 0.5 * np.arange(1, 49)]).astype(np.float32)
    bar = tv.budget_thresholds(cost, 1e-4)
    kc = synth.kept_counts(w) if isinstance(w.m, tuple) else None
    ref = _check_expand(synth.draft_logits(w), w.k, w.m if kc is None else 64, synth.root_tokens(w),
                        m_per_seq=kc, budget_log=bar)
    plain = oracle.expand_rerank(synth.draft_logits(w), w.k, w.m if kc is None else kc,
                                 synth.root_tokens(w))
    assert np.all(ref.n_nodes <= plain.n_nodes) and np.any(ref.n_nodes < plain.n_nodes)
    assert np.all(ref.n_nodes >= np.minimum(plain.n_nodes, 16))


def test_expand_budget_limits_on_device():
    rng = np.random.default_rng(71)
    levels = [(rng.standard_normal((2, 1 if s == 0 else 6, 500)) * 2).astype(np.float32) for s in range(4)]
    roots = rng.integers(0, 500, size=2)
    for bar in (np.full(64, -np.inf, np.float32), np.full(64, np.inf, np.float32)):
        ref = _check_expand(levels, 6, 40, roots, budget_log=bar)
        assert np.all(ref.n_nodes == (40 if bar[1] < 0 else 1))


# ----------------------------------------------------------------------------- per-level stop

def _stop_on_device(levels, k, m, m_per_seq, bar):
    """Every level of tree_expand_rerank, each followed by tree_draft_continue; returns
    the flags [S][B]."""
    B, S = levels[0].shape[0], len(levels)
    ws = tv.expand_workspace(B, k, S)
    out = tv.ExpandOutputs(B, 64, k, DEV)
    roots = dev_i32(np.zeros(B, np.int32))
    mps = None if m_per_seq is None else dev_i32(m_per_seq)
    bud = None if bar is None else torch.from_numpy(np.ascontiguousarray(bar, np.float32)).to(DEV)
    flags = []
    for s in range(S):
        final = (m if m_per_seq is None else 64) if s == S - 1 else 0
        tv.tree_expand_rerank(ws, s + 1, torch.from_numpy(levels[s]).to(DEV), k, S, final_m=int(final),
                              m_per_seq=mps, root_token=roots, out=out, budget_log=bud)
        more = tv.tree_draft_continue(ws, B, k, S, m=0 if m_per_seq is not None else m,
                                      m_per_seq=mps, budget_log=bud)
        flags.append(more.cpu().numpy().copy())
    return np.stack(flags)


def _bars(rng):
    cost = (20.0 + 0.05 * np.arange(1, 65) + 0.01 * np.arange(1, 65) ** 2).astype(np.float32)
    return [tv.budget_thresholds(cost, float(10.0 ** rng.uniform(-4, -1.5))),
            np.full(64, -np.inf, np.float32), np.full(64, np.inf, np.float32), None]


@pytest.mark.parametrize("seed,B,k,S,V,tied", [(1, 4, 2, 6, 40, True), (2, 6, 4, 5, 300, False),
                                              (3, 3, 8, 4, 2000, True), (4, 8, 10, 4, 32000, False)])
def test_draft_continue_matches_oracle(seed, B, k, S, V, tied):
    rng = np.random.default_rng(seed)
    levels = []
    for s in range(S):
        shape = (B, 1 if s == 0 else k, V)
        levels.append((rng.integers(-6, 6, size=shape) * 0.5).astype(np.float32) if tied
                      else (rng.standard_normal(shape) * 2).astype(np.float32))
    m_seq = rng.integers(2, 64, size=B).astype(np.int32)
    for bar in _bars(rng):
        for m, mps in ((int(m_seq[0]), None), (0, m_seq)):
            ref = oracle.expand.draft_continue(levels, k, m if mps is None else mps, bar)
            got = _stop_on_device(levels, k, m, mps, bar)
            assert np.array_equal(got, ref), (bar is None, m, got.T, ref.T)


@pytest.mark.parametrize("wid", [3, 5])
def test_draft_continue_workload(wid):
    """Workloads 3 and 5 with a verify budget from a cost table: the device's flags equal
    the oracle's after every level, and some sequence stops before the last level."""
    w = synth.WORKLOADS[wid]
    cost = np.concatenate([np.full(16, 20.0), 20.0 + 0.5 * np.arange(1, 49)]).astype(np.float32)
    bar = tv.budget_thresholds(cost, 1e-3)
    kc = synth.kept_counts(w) if isinstance(w.m, tuple) else None
    levels = synth.draft_logits(w)
    ref = oracle.expand.draft_continue(levels, w.k, w.m if kc is None else kc, bar)
    got = _stop_on_device(levels, w.k, w.m if kc is None else 0, kc, bar)
    assert np.array_equal(got, ref)
    assert np.any(ref[:-1] == 0)


def test_expand_rerank_at_every_level():
    """final_m at every level: after each level the outputs hold the oracle's tree of
    the levels done so far, and the next level continues on the same workspace."""
    rng = np.random.default_rng(81)
    B, k, S, V = 5, 4, 5, 700
    levels = [(rng.standard_normal((B, 1 if s == 0 else k, V)) * 2).astype(np.float32) for s in range(S)]
    roots = rng.integers(0, V, size=B).astype(np.int32)
    m_seq = np.array([2, 9, 30, 64, 17], np.int32)
    ws = tv.expand_workspace(B, k, S)
    out = tv.ExpandOutputs(B, 64, k, DEV)
    for s in range(S):
        tv.tree_expand_rerank(ws, s + 1, torch.from_numpy(levels[s]).to(DEV), k, S, final_m=64,
                              m_per_seq=dev_i32(m_seq), root_token=dev_i32(roots), out=out)
        ref = oracle.expand_rerank(levels[:s + 1], k, m_seq, roots)
        assert np.array_equal(out.n_nodes.cpu().numpy(), ref.n_nodes)
        assert np.array_equal(out.parent.cpu().numpy(), ref.parent)
        assert np.array_equal(out.token.cpu().numpy(), ref.token)
        assert out.score.cpu().numpy().tobytes() == ref.score.tobytes()


@pytest.mark.parametrize("wid", [3, 5])
def test_draft_tree_stops_without_changing_the_tree(wid):
    """The harness's drafting loop stops before the last level on the EAGLE-2 and
    serving workloads under a cost-table budget, and its tree equals the oracle's tree
    over every level."""
    from tree_attention_verify_ancestor_amd import harness
    w = synth.WORKLOADS[wid]
    cost = np.concatenate([np.full(16, 20.0), 20.0 + 0.5 * np.arange(1, 49)]).astype(np.float32)
    bar = tv.budget_thresholds(cost, 1e-3)
    kc = synth.kept_counts(w) if isinstance(w.m, tuple) else None
    levels = synth.draft_logits(w)
    roots = synth.root_tokens(w)
    out, drafted = harness.draft_tree(
        lambda step, front: torch.from_numpy(levels[step - 1]).to(DEV), w.B, w.k, w.S,
        m=w.m if kc is None else 0, m_per_seq=None if kc is None else dev_i32(kc),
        budget_log=torch.from_numpy(bar).to(DEV), root_token=dev_i32(roots))
    ref = oracle.expand_rerank(levels, w.k, w.m if kc is None else kc, roots, budget_log=bar)
    assert drafted < w.S
    assert np.array_equal(out.n_nodes.cpu().numpy(), ref.n_nodes)
    assert np.array_equal(out.parent.cpu().numpy(), ref.parent)
    assert np.array_equal(out.token.cpu().numpy(), ref.token)
    assert out.score.cpu().numpy().tobytes() == ref.score.tobytes()


# ----------------------------------------------------------------------------- cost table

def test_cost_table_measure_and_lookup():
    """The calibration measures this library's own tree_verify_attn over a batch x context
    x node-count grid: latency grows with the node count where verification is MFMA-bound
    (4 x 16384 keys, 512 query rows per KV head at 64 nodes), a second measurement agrees
    within 15%, the lookup returns the measured (running-maximum) row at grid points, and
    calibrate() at one point gives the same bars as the table there."""
    from tree_attention_verify_ancestor_amd import harness
    kw = dict(batch=(1, 4), context=(2048, 16384), nodes=(1, 16, 32, 64), reps=5)
    t1 = harness.CostTable.measure(64, 8, **kw)
    t2 = harness.CostTable.measure(64, 8, **kw)
    c1, c2 = t1.cost_us, t2.cost_us
    assert np.all(c1 > 0) and np.all(np.abs(c1 - c2) <= 0.15 * np.maximum(c1, c2)), (c1, c2)
    assert c1[1, 1, 3] > 1.5 * c1[1, 1, 0], c1[1, 1]              # MFMA-bound: nodes cost
    for i, B in enumerate(kw["batch"]):
        for j, L in enumerate(kw["context"]):
            got = t1.cost(B, L)
            assert np.all(np.diff(got) >= 0)
            want = np.maximum.accumulate(c1[i, j])
            assert np.array_equal(got[[0, 15, 31, 63]], want.astype(np.float32)), (B, L)
    bars = t1.budget_log(4, 16384, 1e-4)
    assert np.array_equal(bars, tv.budget_thresholds(t1.cost(4, 16384), 1e-4))
    one = harness.calibrate(4, 16384, 64, 8, n_points=kw["nodes"], reps=5)
    assert np.all(np.diff(one) >= 0) and one.shape == (64,)
    assert np.all(np.abs(one[[0, 63]] - t1.cost(4, 16384)[[0, 63]]) <= 0.15 * one[[0, 63]])
    j = harness.CostTable.from_json(t1.to_json())
    assert np.allclose(j.cost(2, 5000), t1.cost(2, 5000), rtol=1e-3)


# ----------------------------------------------------------------------------- low-rank candidate head

def _cand_inputs(seed, rows, d, r, V):
    """bf16 bits of h ~ N(0,1), A ~ N(0,1/d) (z ~ N(0,1)), Bm and W scaled for logits
    of standard deviation about 2, as the dynamic-tree workloads' draft logits."""
    rng = np.random.default_rng(seed)
    bits = lambda sh, sc: synth.bf16_bits((rng.standard_normal(sh) * sc).astype(np.float32))
    return (bits((rows, d), 1.0), bits((r, d), d ** -0.5), bits((V, r), 2 * r ** -0.5),
            bits((V, d), 2 * d ** -0.5))


def _bf16_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(DEV).view(torch.bfloat16)


@pytest.mark.parametrize("seed,rows,d,r,V,C", [(1, 3, 72, 32, 1000, 13), (2, 10, 4096, 256, 32000, 64),
                                              (3, 40, 512, 128, 5000, 256), (4, 2, 64, 32, 37, 37),
                                              (5, 9, 136, 96, 3001, 40),
                                              # scores past the LDS cache (a 128256-token vocabulary)
                                              (6, 4, 256, 64, 128256, 64)])
def test_candidate_logits_matches_oracle(seed, rows, d, r, V, C):
    """Bit-exact logits and candidate lists against the oracle, except entries (and
    lists) the oracle flags as depending on the order of a float64 sum."""
    hb, Ab, Bb, Wb = _cand_inputs(seed, rows, d, r, V)
    f = synth.bf16_to_f32
    ref, rc, rind, rcind = oracle.candidate_logits(f(hb), f(Ab), f(Bb), f(Wb), C)
    lg, cd = tv.tree_candidate_logits(_bf16_dev(hb), _bf16_dev(Ab), _bf16_dev(Bb), _bf16_dev(Wb), C)
    torch.cuda.synchronize()
    lg, cd = lg.cpu().numpy(), cd.cpu().numpy()
    # entries next to a float32 midpoint (the oracle's float64 sum could round either
    # way in another order) are excluded: 0-9 of them per case on these seeds, never a
    # candidate list
    assert int(rind.sum()) <= 16, f"{int(rind.sum())} entries excluded"
    assert not rcind.any(), f"{int(rcind.sum())} candidate lists excluded"
    ok = ~rind
    assert np.array_equal(lg.view(np.uint32)[ok], ref.view(np.uint32)[ok])
    for i in range(rows):
        assert np.array_equal(cd[i], rc[i]), i


@pytest.mark.parametrize("V", [3000, 40000])
def test_candidate_logits_tied_scores(V):
    """Token rows of Bm repeat every 50 tokens, so scores tie across many ids and the
    C-th place falls inside a tie: candidates must follow the lower id (in LDS and,
    past its cache, over the whole row)."""
    hb, Ab, Bb, Wb = _cand_inputs(11, 4, 256, 64, V)
    Bb = np.ascontiguousarray(np.tile(Bb[:50], (V // 50, 1)))
    f = synth.bf16_to_f32
    for C in (7, 64, 130):
        ref, rc, rind, rcind = oracle.candidate_logits(f(hb), f(Ab), f(Bb), f(Wb), C)
        lg, cd = tv.tree_candidate_logits(_bf16_dev(hb), _bf16_dev(Ab), _bf16_dev(Bb), _bf16_dev(Wb), C)
        torch.cuda.synchronize()
        lg, cd = lg.cpu().numpy(), cd.cpu().numpy()
        assert not rind.any() and not rcind.any()          # nothing excluded on this seed
        assert np.array_equal(lg.view(np.uint32), ref.view(np.uint32))
        for i in range(4):
            assert np.array_equal(cd[i], rc[i]), (C, i)


def test_candidate_head_feeds_expansion():
    """Two draft levels whose logits come from the candidate head: the device tree equals
    the oracle's expansion of the oracle's candidate logits."""
    k, V, d, r, C = 6, 3000, 256, 64, 32
    hb1, Ab, Bb, Wb = _cand_inputs(8, 1, d, r, V)      # seeds whose entries are all determinate
    hb2 = _cand_inputs(8, k, d, r, V)[0]
    f = synth.bf16_to_f32
    levels_ref, levels_dev = [], []
    for hb in (hb1, hb2):
        ref, _, rind, _ = oracle.candidate_logits(f(hb), f(Ab), f(Bb), f(Wb), C)
        assert not rind.any()
        levels_ref.append(ref[None])
        lg, _ = tv.tree_candidate_logits(_bf16_dev(hb), _bf16_dev(Ab), _bf16_dev(Bb), _bf16_dev(Wb), C)
        levels_dev.append(lg[None])
    roots = np.array([5], np.int32)
    ref = oracle.expand_rerank(levels_ref, k, 20, roots)
    ws = tv.expand_workspace(1, k, 2)
    out = tv.ExpandOutputs(1, 64, k, DEV)
    for s in range(2):
        tv.tree_expand_rerank(ws, s + 1, levels_dev[s], k, 2, final_m=20 if s == 1 else 0,
                              root_token=dev_i32(roots), out=out)
    torch.cuda.synchronize()
    assert np.array_equal(out.parent.cpu().numpy(), ref.parent)
    assert np.array_equal(out.token.cpu().numpy(), ref.token)
    assert out.score.cpu().numpy().tobytes() == ref.score.tobytes()
