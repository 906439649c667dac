"""The allocation-free attention entry point (tree_verify_attn_noalloc) against the
workspace entry point (tree_verify_attn), through the C ABI on the GPU: two calls in a
row on one GPU, the second with a smaller input, each bit for bit equal to the
workspace call (same kernels and plan) and within the attention tolerance of the
oracle."""

import numpy as np
import pytest
import torch

import oracle
import synth
import tree_attention_verify_ancestor_amd as tv
from gpu_helpers import attn_close, attn_device_inputs, dev_i32, host

pytestmark = pytest.mark.gpu


def _both(inp, parent, nn, max_prefix):
    d = attn_device_inputs(inp)
    par, nnd = dev_i32(parent), dev_i32(nn)
    anc, _, _, _ = tv.tree_build(par, nnd)
    ref_out, ref_lse, ref_st = tv.tree_verify_attn(d["q"], d["k_tree"], d["v_tree"], d["k_prefix"],
                                                   d["v_prefix"], d["offsets"], nnd, anc, max_prefix)
    B, n_max, Hq, D = d["q"].shape
    out = torch.empty((B, n_max, Hq, D), dtype=d["q"].dtype, device=d["q"].device)
    lse = torch.empty((B, n_max, Hq), dtype=torch.float32, device=d["q"].device)
    st = torch.empty((B,), dtype=torch.int32, device=d["q"].device)
    tv.tree_verify_attn_noalloc(d["q"], d["k_tree"], d["v_tree"], d["k_prefix"], d["v_prefix"],
                                d["offsets"], nnd, anc, max_prefix, out, st, lse=lse)
    torch.cuda.synchronize()
    return (ref_out, ref_lse, ref_st), (out, lse, st)


def test_noalloc_matches_workspace_call_twice():
    cases = [  # (seed, B, Hq, Hkv, D, prefix lengths, node counts): several key chunks each
        (1, 4, 64, 8, 128, (6000, 4100, 2500, 3000), (64, 50, 64, 13)),
        (2, 2, 16, 4, 128, (1800, 900), (40, 64)),
    ]
    for seed, B, Hq, Hkv, D, lens, ns in cases:
        plan = tv.attn_plan(B, 64, Hq, Hkv, D, max(lens))
        assert plan["n_chunks"] > 1, plan                      # the scratch is used
        inp, parent, nn = synth.random_attention_case(seed, B, Hq, Hkv, D, lens, ns, std=0.5)
        (ro, rl, rs), (o, l, s) = _both(inp, parent, nn, max(lens))
        assert torch.equal(s, rs) and int(s.abs().sum()) == 0
        assert torch.equal(o.view(torch.int16), ro.view(torch.int16)), f"case {seed}: out differs"
        assert torch.equal(l, rl), f"case {seed}: lse differs"
        ref, _ = oracle.tree_verify_attn(inp.f32("q"), inp.f32("k_tree"), inp.f32("v_tree"),
                                         inp.f32("k_prefix"), inp.f32("v_prefix"),
                                         inp.prefix_offsets, parent, nn)
        ok, msg = attn_close(host(o), ref, f"noalloc case {seed}")
        assert ok, msg


def test_noalloc_rejects_partials_past_the_scratch():
    """Sizes whose chunk partials exceed the 128 MiB scratch fail before any launch: 511
    sequences of 256 rows (one KV head) and an 8192-key prefix take two chunks each."""
    B, n_max, Hq, Hkv, D, L = 511, 64, 4, 1, 128, 8192
    need = tv.lib().tree_verify_attn_workspace_size(1, B, n_max, Hq, Hkv, D, L)
    assert need > 128 << 20, need
    dev = "cuda"
    q = torch.zeros((B, n_max, Hq, D), dtype=torch.bfloat16, device=dev)
    kt = torch.zeros((B, n_max, Hkv, D), dtype=torch.bfloat16, device=dev)
    kp = torch.zeros((1, Hkv, D), dtype=torch.bfloat16, device=dev)
    offs = torch.zeros((B + 1,), dtype=torch.int64, device=dev)
    nn = torch.ones((B,), dtype=torch.int32, device=dev)
    anc = torch.ones((B, n_max), dtype=torch.int64, device=dev)
    out = torch.empty_like(q)
    st = torch.empty((B,), dtype=torch.int32, device=dev)
    with pytest.raises(tv.TreeVerifyError) as e:
        tv.tree_verify_attn_noalloc(q, kt, kt, kp, kp, offs, nn, anc, L, out, st)
    assert e.value.code == 5                                   # TV_ERR_WORKSPACE
