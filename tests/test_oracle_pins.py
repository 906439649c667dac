"""The oracle against what the pages and the mathematics fix (CPU only)."""

import numpy as np
import pytest
import torch

import oracle
import oracle_pins
import synth


@pytest.mark.parametrize("name", list(oracle_pins.ALL_PINS))
def test_pin(name):
    assert oracle_pins.ALL_PINS[name](), name


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_tree_bruteforce_more_seeds(seed):
    assert oracle_pins.pin_tree_bruteforce(seed, trials=30)


@pytest.mark.parametrize("seed", [31, 32])
def test_accept_bruteforce_more_seeds(seed):
    assert oracle_pins.pin_accept_bruteforce(seed, trials=150)


@pytest.mark.parametrize("seed", [41, 42, 43])
def test_expand_bruteforce_more_seeds(seed):
    assert oracle_pins.pin_expand_bruteforce(seed, trials=9)


def test_bf16_rounding_matches_torch():
    """The generator's bf16 rounding equals torch's float32 -> bfloat16 conversion."""
    x = np.random.default_rng(0).standard_normal(100000).astype(np.float32) * 3
    x[:4] = [1.00390625, 1.005859375, -1.00390625, 65504.0]      # exact halfway cases
    ours = synth.bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(synth.bf16_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_workload_shapes():
    """Static trees of the first two workloads have the stated sizes and depths."""
    for wid, n, d in [(1, 10, 3), (2, 26, 5)]:
        w = synth.WORKLOADS[wid]
        parent, nn = synth.static_tree(w)
        anc, depth, pos, st = oracle.tree_build(parent, nn, synth.prefix_lengths(w))
        assert st[0] == 0 and nn[0] == n and depth[0].max() == d
        assert pos[0, 0] == w.prefix
    lens = synth.prefix_lengths(synth.WORKLOADS[5])
    m = synth.kept_counts(synth.WORKLOADS[5])
    assert lens.min() >= 512 and lens.max() <= 8192 and len(lens) == 32
    assert m.min() >= 16 and m.max() <= 64


def test_tiny_workload_end_to_end():
    """Workload 1 through every oracle step: tree, attention, acceptance."""
    w = synth.WORKLOADS[1]
    inp = synth.attention_inputs(w)
    parent, nn = synth.static_tree(w)
    anc, depth, pos, st = oracle.tree_build(parent, nn, synth.prefix_lengths(w))
    out, lse = oracle.tree_verify_attn(inp.q, inp.k_tree, inp.v_tree, inp.k_prefix, inp.v_prefix,
                                       inp.prefix_offsets, parent, nn)
    assert np.all(np.isfinite(out)) and np.all(out[0, 10:] == 0)
    tok = synth.static_draft_tokens(w)
    tgt = synth.target_ids(w, parent, tok, nn)
    al, best, bonus, path = oracle.tree_accept(parent, tok, tgt, nn)
    assert 0 <= al[0] <= 3 and bonus[0] == tgt[0, best[0]]


def test_dynamic_workload_tree_small():
    """Workload 3's draft logits through expansion: 60 nodes, depth <= 6, ancestors kept."""
    w = synth.WORKLOADS[3]
    res = oracle.expand_rerank(synth.draft_logits(w), w.k, w.m, synth.root_tokens(w))
    assert res.status[0] == 0 and res.n_nodes[0] == 60 and not res.indeterminate[0]
    anc, depth, pos, st = oracle.tree_build(res.parent, res.n_nodes, None)
    assert st[0] == 0 and depth[0].max() <= 6


@pytest.mark.parametrize("seed", [8, 9, 10])
def test_compact_root_path_more_seeds(seed):
    assert oracle_pins.pin_compact_root_path(seed)
