"""The plan-variant build of the library (another work partition and order, the same
arithmetic) against the product build, on the GPU: every output must be bit-identical.
An LDS race, a missing barrier or a reduction whose order depends on scheduling would
show up as a difference here (the surveys' race check: results identical across
work-partition variants)."""

import contextlib
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import tree_attention_verify_ancestor_amd as tv
from tree_attention_verify_ancestor_amd import _lib
from gpu_helpers import attn_device_inputs, dev_i32, run_attn, run_expand

pytestmark = pytest.mark.gpu

VARIANT = os.path.join(os.path.dirname(_lib.LIB_PATH), "libtreeverify_variant.so")


@contextlib.contextmanager
def variant_library():
    """Route every binding call to the plan-variant build for the duration."""
    saved = _lib.lib()
    _lib._lib = _lib.load(VARIANT)
    try:
        yield
    finally:
        _lib._lib = saved


def _attn_both(inp, parent, nn, max_prefix):
    d = attn_device_inputs(inp)
    a = run_attn(d, parent, nn, max_prefix)
    with variant_library():
        b = run_attn(d, parent, nn, max_prefix)
    return a, b


ATTN_CASES = [  # (B, Hq, Hkv, D, prefix lengths, node counts): every launch shape
    (2, 2, 2, 128, (3000, 1777), (32, 27)),
    (2, 2, 2, 64, (3000, 1777), (64, 59)),
    (2, 8, 2, 128, (3000, 1777), (64, 59)),
    (2, 4, 2, 128, (3000, 1777), (64, 59)),
    (4, 64, 8, 128, (3000, 2100, 777, 0), (64, 40, 1, 61)),
    (9, 64, 8, 128, (3000, 17, 0, 900, 2500, 64, 1200, 5, 640), (64, 3, 20, 64, 1, 33, 50, 64, 10)),
    (3, 32, 8, 128, (4096, 4096, 4096), (60, 60, 60)),
]


def test_variant_build_plans_differently():
    a = tv.attn_plan(4, 64, 64, 8, 128, 3000)
    with variant_library():
        b = tv.attn_plan(4, 64, 64, 8, 128, 3000)
    assert b["grid"] == a["grid"] + 64 and {k: v for k, v in a.items() if k != "grid"} == \
        {k: v for k, v in b.items() if k != "grid"}


@pytest.mark.parametrize("case", ATTN_CASES)
def test_attention_identical_across_plans(case):
    B, Hq, Hkv, D, lens, ns = case
    n_max = max(ns) if max(ns) <= 32 else 64
    inp, parent, nn = synth.random_attention_case(900 + B + Hq + D, B, Hq, Hkv, D, lens, ns,
                                                  std=0.5, n_max=n_max)
    (o1, l1, s1, _), (o2, l2, s2, _) = _attn_both(inp, parent, nn, max(lens))
    assert torch.equal(s1, s2)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), case
    assert torch.equal(l1, l2), case


def test_attention_workload5_identical_across_plans():
    w = synth.WORKLOADS[5]
    kc = synth.kept_counts(w)
    tree = oracle.expand_rerank(synth.draft_logits(w), w.k, kc, synth.root_tokens(w))
    inp = synth.attention_inputs(w)
    (o1, l1, _, _), (o2, l2, _, _) = _attn_both(inp, tree.parent, tree.n_nodes,
                                                int(np.diff(inp.prefix_offsets).max()))
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


EXPAND_CASES = [  # (B, k, S, V, m): rows split into chunks of different sizes
    (2, 10, 3, 50000, 40), (3, 4, 3, 20001, 16), (1, 16, 2, 9001, 64), (2, 8, 4, 128256, 64),
    (4, 3, 3, 600001, 9),
]


@pytest.mark.parametrize("case", EXPAND_CASES)
def test_expansion_identical_across_plans(case):
    B, k, S, V, m = case
    rng = np.random.default_rng(sum(case))
    levels = [(rng.standard_normal((B, 1 if s == 0 else k, V)) * 2).astype(np.float32) for s in range(S)]
    roots = rng.integers(0, V, size=B)
    ref = oracle.expand_rerank(levels, k, m, roots)
    assert not ref.indeterminate.any()          # no row's float32 normaliser is order-dependent
    a, fa = run_expand(levels, k, m, roots)
    with variant_library():
        b, fb = run_expand(levels, k, m, roots)
    for name in ("parent", "token", "n_nodes", "seq_status"):
        assert torch.equal(getattr(a, name), getattr(b, name)), name
    assert torch.equal(a.score.view(torch.int32), b.score.view(torch.int32))
    for x, y in zip(fa, fb):
        assert np.array_equal(x, y)
