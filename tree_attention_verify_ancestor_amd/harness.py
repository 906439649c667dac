"""Cost table for the verify budget: tree_verify_attn latency against the node count.

"Technical analysis of EAGLE-4", section "EAGLE-4 verification trees and the
harness": before serving, a one-time calibration on the target GPU builds a table of
verification latency against batch size, context length and candidate count; the
harness then adds candidates while the gain in cumulative probability per unit of
marginal cost stays above a threshold, and stops drafting once it falls below.
calibrate() measures this library's own tree_verify_attn (HIP events around graph
replays) at one (batch, context) for a few node counts and interpolates the rest; budget_thresholds() (the library's host
helper) turns the table into the per-place bars tree_expand_rerank takes;
draft_tree() drafts level by level and stops with tree_draft_continue.

Usage: python -m tree_attention_verify_ancestor_amd.harness   (prints JSON tables)
"""

import json

import numpy as np
import torch

from . import ops

DEFAULT_N = (1, 4, 8, 16, 24, 32, 40, 48, 56, 64)


def calibrate(B, L, Hq, Hkv, D=128, n_points=DEFAULT_N, reps=20, device="cuda", seed=0):
    """Returns float32 cost_us[64]: cost_us[N-1] = microseconds of one bf16
    tree_verify_attn call with N nodes per tree (chains), prefix L per sequence."""
    g = torch.Generator(device=device).manual_seed(seed)
    n_max = 64
    bf = dict(dtype=torch.bfloat16, device=device)
    q = (torch.randn((B, n_max, Hq, D), generator=g, device=device) * 0.5).to(torch.bfloat16)
    kt = (torch.randn((B, n_max, Hkv, D), generator=g, device=device) * 0.5).to(torch.bfloat16)
    vt = (torch.randn((B, n_max, Hkv, D), generator=g, device=device) * 0.5).to(torch.bfloat16)
    kp = (torch.randn((B * L, Hkv, D), generator=g, device=device) * 0.5).to(torch.bfloat16)
    vp = (torch.randn((B * L, Hkv, D), generator=g, device=device) * 0.5).to(torch.bfloat16)
    offs = torch.arange(B + 1, dtype=torch.int64, device=device) * L
    parent = torch.full((B, n_max), -1, dtype=torch.int32, device=device)
    parent[:, 1:] = torch.arange(n_max - 1, dtype=torch.int32, device=device)
    ws = ops.attn_workspace(torch.bfloat16, B, n_max, Hq, Hkv, D, L, device)
    out = torch.empty((B, n_max, Hq, D), **bf)
    meas = []
    for n in n_points:
        nn = torch.full((B,), n, dtype=torch.int32, device=device)
        anc, _, _, _ = ops.tree_build(parent, nn)
        call = lambda: ops.tree_verify_attn(q, kt, vt, kp, vp, offs, nn, anc, L, out=out, ws=ws,
                                            want_lse=False)
        call()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(reps):
                call()
        graph.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(3):
            graph.replay()
        e1.record()
        torch.cuda.synchronize()
        meas.append(e0.elapsed_time(e1) * 1e3 / (3 * reps))
    cost = np.interp(np.arange(1, n_max + 1), np.asarray(n_points, float), np.asarray(meas))
    return np.maximum.accumulate(cost).astype(np.float32)      # latency never falls with N


def budget_thresholds(cost_us, threshold):
    return ops.budget_thresholds(cost_us, threshold)


def draft_tree(level_logits, B, k, max_steps, m=0, m_per_seq=None, budget_log=None,
               root_token=None, n_max=64, ws=None, out=None):
    """The harness's drafting loop: expand level by level, rerank after every level
    (final_m at each call, so `out` always holds the tree of the levels done), and stop
    once tree_draft_continue reports for every sequence that another level cannot change
    its tree -- the harness's "decide when to stop drafting".

    level_logits(step, frontier_token) -> fp32 [B][1 if step == 1 else k][vocab]: the
    drafter's logits for the frontier of the previous level (frontier_token [B][k], the
    tokens by rank).  Reading the flags costs one host synchronisation per level.
    Returns (out, levels drafted)."""
    dev = root_token.device if root_token is not None else "cuda"
    if ws is None:
        ws = ops.expand_workspace(B, k, max_steps, dev)
    if out is None:
        out = ops.ExpandOutputs(B, n_max, k, dev)
    final = m if m_per_seq is None else n_max
    for step in range(1, max_steps + 1):
        ops.tree_expand_rerank(ws, step, level_logits(step, out.frontier_token), k, max_steps,
                               final_m=final, m_per_seq=m_per_seq, root_token=root_token,
                               n_max=n_max, out=out, budget_log=budget_log)
        if step == max_steps:
            break
        more = ops.tree_draft_continue(ws, B, k, max_steps, m=0 if m_per_seq is not None else m,
                                       m_per_seq=m_per_seq, budget_log=budget_log)
        if not bool(more.any()):
            break
    return out, step


def _main():
    shapes = {"B1_L2048_mha32": (1, 2048, 32, 32), "B1_L4096_gqa32x8": (1, 4096, 32, 8),
              "B4_L32768_gqa64x8": (4, 32768, 64, 8), "B32_L4352_gqa32x8": (32, 4352, 32, 8)}
    res = {}
    for name, (B, L, Hq, Hkv) in shapes.items():
        c = calibrate(B, L, Hq, Hkv)
        res[name] = {"cost_us": [round(float(x), 2) for x in c]}
        print(json.dumps({name: res[name]}), flush=True)


if __name__ == "__main__":
    _main()
