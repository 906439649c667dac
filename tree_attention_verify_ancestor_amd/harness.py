"""Cost table for the verify budget: tree_verify_attn latency against batch, context
length and node count.

"Technical analysis of EAGLE-4", section "EAGLE-4 verification trees and the
harness": before serving, a one-time calibration on the target GPU builds a table of
verification latency against batch size, context length and candidate count; the
harness then adds candidates while the gain in cumulative probability per unit of
marginal cost stays above a threshold, and stops drafting once it falls below.

CostTable.measure() times this library's own tree_verify_attn (bf16, chain trees, HIP
events around graph replays) over a grid of batch sizes, context lengths and node
counts.  CostTable.cost(B, L) reads the latency of N = 1..64 nodes at the caller's
batch and context through the library's host helper tree_cost_lookup (interpolation
in log batch and log context, linear in N); budget_log() turns that into the
per-place bars tree_expand_rerank takes (tree_budget_thresholds); draft_tree() drafts
level by level and stops with tree_draft_continue.

Usage: python -m tree_attention_verify_ancestor_amd.harness [out.json]
"""

import json
import sys

import numpy as np
import torch

from . import ops

GRID_BATCH = (1, 4, 16, 32)
GRID_CONTEXT = (1024, 4096, 16384, 32768)
GRID_NODES = (1, 8, 16, 24, 32, 48, 64)


def _time_calls(Hq, Hkv, D, B, L, nodes, bufs, reps, device):
    """Microseconds of one call at each node count (graph replays of reps calls)."""
    q, kt, vt, kp, vp = bufs
    n_max = 64
    qb, ktb, vtb = q[:B], kt[:B], vt[:B]
    kpb, vpb = kp[:B * L], vp[:B * L]
    offs = torch.arange(B + 1, dtype=torch.int64, device=device) * L
    parent = torch.full((B, n_max), -1, dtype=torch.int32, device=device)
    parent[:, 1:] = torch.arange(n_max - 1, dtype=torch.int32, device=device)
    ws = ops.attn_workspace(torch.bfloat16, B, n_max, Hq, Hkv, D, L, device)
    out = torch.empty((B, n_max, Hq, D), dtype=torch.bfloat16, device=device)
    res = []
    for n in nodes:
        nn = torch.full((B,), n, dtype=torch.int32, device=device)
        anc, _, _, _ = ops.tree_build(parent, nn)
        call = lambda: ops.tree_verify_attn(qb, ktb, vtb, kpb, vpb, offs, nn, anc, L, out=out,
                                            ws=ws, want_lse=False)
        call()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for _ in range(reps):
                call()
        graph.replay()
        torch.cuda.synchronize()
        # each replay timed on its own and the median kept: a host stall between two
        # replays (the GPU idles while it lasts) then moves one sample, not the figure
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(5)]
        for e0, e1 in ev:
            e0.record()
            graph.replay()
            e1.record()
        torch.cuda.synchronize()
        res.append(float(np.median([e0.elapsed_time(e1) for e0, e1 in ev])) * 1e3 / reps)
    return res


def _buffers(Hq, Hkv, D, B, L, device, seed):
    g = torch.Generator(device=device).manual_seed(seed)
    r = lambda shape: (torch.randn(shape, generator=g, device=device) * 0.5).to(torch.bfloat16)
    return (r((B, 64, Hq, D)), r((B, 64, Hkv, D)), r((B, 64, Hkv, D)), r((B * L, Hkv, D)),
            r((B * L, Hkv, D)))


class CostTable:
    """Latency of tree_verify_attn over a grid: cost_us[i][j][k] microseconds at batch
    batch[i], context context[j] and nodes[k] nodes per tree, for one head shape."""

    def __init__(self, batch, context, nodes, cost_us, Hq, Hkv, D=128):
        self.batch, self.context, self.nodes = tuple(batch), tuple(context), tuple(nodes)
        self.cost_us = np.asarray(cost_us, dtype=np.float32)
        self.Hq, self.Hkv, self.D = Hq, Hkv, D

    @classmethod
    def measure(cls, Hq, Hkv, D=128, batch=GRID_BATCH, context=GRID_CONTEXT, nodes=GRID_NODES,
                reps=10, device="cuda", seed=0):
        """Time every grid point on the device (one set of buffers of the largest size)."""
        bufs = _buffers(Hq, Hkv, D, max(batch), max(context), device, seed)
        cost = np.zeros((len(batch), len(context), len(nodes)), np.float32)
        for i, B in enumerate(batch):
            for j, L in enumerate(context):
                cost[i, j] = _time_calls(Hq, Hkv, D, B, L, nodes, bufs, reps, device)
        del bufs
        return cls(batch, context, nodes, cost, Hq, Hkv, D)

    def cost(self, B, L, n_max=64):
        """float32 [n_max]: latency with N = 1..n_max nodes at batch B and context L."""
        return ops.cost_lookup(self.batch, self.context, self.nodes, self.cost_us, B, L, n_max)

    def budget_log(self, B, L, threshold, n_max=64):
        """The verify budget's bars at batch B and context L (tree_budget_thresholds)."""
        return ops.budget_thresholds(self.cost(B, L, n_max), threshold)

    def to_json(self):
        return {"Hq": self.Hq, "Hkv": self.Hkv, "D": self.D, "batch": list(self.batch),
                "context": list(self.context), "nodes": list(self.nodes),
                "cost_us": [[[round(float(x), 3) for x in r] for r in p] for p in self.cost_us]}

    @classmethod
    def from_json(cls, d):
        return cls(d["batch"], d["context"], d["nodes"], d["cost_us"], d["Hq"], d["Hkv"], d["D"])


def calibrate(B, L, Hq, Hkv, D=128, n_points=GRID_NODES, reps=20, device="cuda", seed=0):
    """float32 cost_us[64] at one (batch, context): the node points measured on the
    device, the rest read through tree_cost_lookup (a one-point batch / context grid)."""
    bufs = _buffers(Hq, Hkv, D, B, L, device, seed)
    meas = _time_calls(Hq, Hkv, D, B, L, n_points, bufs, reps, device)
    del bufs
    return ops.cost_lookup([B], [max(L, 1)], n_points, np.asarray(meas, np.float32)[None, None, :],
                           B, L)


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
    """Measure the grid for the head shapes of the studied workloads and print it as JSON
    (to the file named on the command line as well)."""
    tables = {}
    for name, (Hq, Hkv) in {"mha32": (32, 32), "gqa32x8": (32, 8), "gqa64x8": (64, 8)}.items():
        tables[name] = CostTable.measure(Hq, Hkv).to_json()
        print(json.dumps({name: tables[name]}), flush=True)
    if len(sys.argv) > 1:
        json.dump(tables, open(sys.argv[1], "w"), indent=1)


if __name__ == "__main__":
    _main()
