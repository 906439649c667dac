#!/usr/bin/env python3
"""Throughput of the draft-tree verification hot path on one MI355X.

One step is one pass of the whole path over one batch of synthetic input:
  dynamic-tree workloads: tree_expand_rerank for every level (rerank on the last),
  then tree_build, tree_verify_attn and tree_accept;
  static-tree workloads:  tree_build, tree_verify_attn and tree_accept.
The metric is node.head queries per second (sum over sequences of n_nodes * Hq per
step, divided by the step time).  Inputs are resident in HBM before timing starts;
each step reads its own copy of every input, rotating over enough copies (>= 1 GiB)
that the 256 MiB last-level cache cannot serve repeated reads.

Each step is captured once per input copy into a HIP graph (so host launch cost is
not what is timed) and the graphs are replayed.  The dominant kernel's roofline uses
the tree_verify_attn call: its algorithmic bytes (prefix K/V + tree K/V + Q + O)
divided by its average duration, measured with HIP events on its stream around
graph replays of back-to-back attention calls over the rotated copies.  The CPU
baseline is the plain oracle timed on a bounded sample on the host cores.  The KV
compaction that follows acceptance (tree_kv_compact), the rejection-sampling
acceptance (tree_accept_stochastic, on seeded target/draft distributions) and the
draft model's low-rank candidate head (tree_candidate_logits, synthetic weights) are
timed the same way, outside the step, and reported beside it.

The roofline of the attention call is the binding one for its arithmetic intensity
(algorithmic flops per algorithmic byte against the 312.5 flop/B ridge of 2.5 PFLOP/s
dense bf16 over 8 TB/s): MFMA for the long-prefix 70B-shaped batch (512 query rows per
KV head), HBM for the others; the other fraction is reported beside it.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 4]
"""

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "tree-verify attn: node·head queries/s; KV HBM GB/s as % of peak"
UNIT = "node·head queries/s"
HBM_PEAK_GBS = 8000.0                    # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0           # MI355X dense bf16
DEFAULT_WORKLOAD = 4                     # the 70B-shaped long-prefix batch (4 x 32768 keys)
RIDGE_FLOP_PER_BYTE = MFMA_BF16_PEAK_TFLOPS * 1e12 / (HBM_PEAK_GBS * 1e9)   # 312.5
ROTATE_BYTES = 1 << 30


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", type=int, default=DEFAULT_WORKLOAD, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="bounded CPU work for the oracle baseline (0 disables it)")
    ap.add_argument("--attn-reps", type=int, default=20,
                    help="replays of the back-to-back attention graph for the kernel timing")
    ap.add_argument("--copy-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB three times "
                         "(the known-size reference for HBM byte counters), then exit")
    return ap.parse_args()


def kernel_source_hash():
    """Hash of the attention kernel source; recorded counter traffic is valid only for it."""
    p = os.path.join(ROOT, "tree_attention_verify_ancestor_amd", "csrc", "attn.hip")
    return hashlib.sha256(open(p, "rb").read()).hexdigest()[:16]


def recorded_traffic(workload_name):
    """Counter-measured HBM bytes per attention launch from profiles/, if still valid."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(p):
        return None
    try:
        rec = json.load(open(p)).get(workload_name)
    except (ValueError, OSError):
        return None
    if not rec or rec.get("attn_source_sha256_16") != kernel_source_hash():
        return None
    return rec.get("bytes_per_launch")


class Inputs:
    """Host-side synthetic inputs of one workload (numpy), shared by GPU and CPU legs."""

    def __init__(self, w):
        import synth
        self.w = w
        self.attn = synth.attention_inputs(w)
        self.lens = np.diff(self.attn.prefix_offsets)
        self.dynamic = not isinstance(w.tree, list)
        if self.dynamic:
            self.levels = synth.draft_logits(w)
            self.roots = synth.root_tokens(w)
            self.m_seq = synth.kept_counts(w) if isinstance(w.m, tuple) else None
        else:
            self.parent, self.n_nodes = synth.static_tree(w)
            self.tokens = synth.static_draft_tokens(w)
            self.target = synth.target_ids(w, self.parent, self.tokens, self.n_nodes)

    def algorithmic_bytes(self, n_nodes):
        """Prefix K/V + tree K/V + Q + O bytes of one attention launch."""
        w = self.w
        el = 2 if w.dtype == "bf16" else 4
        prefix = int(self.lens.sum()) * w.Hkv * w.D * 2 * el
        nodes = int(np.sum(n_nodes))
        tree = nodes * w.Hkv * w.D * 2 * el
        qo = nodes * w.Hq * w.D * 2 * el
        return prefix + tree + qo

    def algorithmic_flops(self, parent, n_nodes):
        """2*D multiply-adds for QK and for PV per visible (query row, key) pair."""
        w = self.w
        tot = 0
        for b in range(w.B):
            n = int(n_nodes[b])
            depth_sum = 0
            for i in range(n):
                d, j = 0, i
                while j > 0:
                    j = int(parent[b, j])
                    d += 1
                depth_sum += d + 1
            tot += (n * int(self.lens[b]) + depth_sum) * w.Hq
        return 4.0 * w.D * tot


def gpu_leg(args, inp):
    import torch
    import synth
    import tree_attention_verify_ancestor_amd as tv

    w = inp.w
    dev = "cuda"
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32

    def to_dev(a):
        if w.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    i32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(dev)
    per_copy = inp.algorithmic_bytes(np.full(w.B, w.n_max)) + sum(
        lv.nbytes for lv in getattr(inp, "levels", []))
    R = max(2, math.ceil(ROTATE_BYTES / per_copy))
    base = dict(q=to_dev(inp.attn.q), k_tree=to_dev(inp.attn.k_tree), v_tree=to_dev(inp.attn.v_tree),
                k_prefix=to_dev(inp.attn.k_prefix), v_prefix=to_dev(inp.attn.v_prefix))
    offsets = torch.from_numpy(inp.attn.prefix_offsets).to(dev)
    prefix_len = i32(inp.lens)
    copies = []
    for r in range(R):
        c = {k: v.clone() for k, v in base.items()}
        if inp.dynamic:
            c["levels"] = [torch.from_numpy(lv).to(dev) for lv in inp.levels]
            c["ws"] = tv.expand_workspace(w.B, w.k, w.S, dev)
            c["exp"] = tv.ExpandOutputs(w.B, w.n_max, w.k, dev)
        copies.append(c)
    del base
    max_prefix = int(inp.lens.max())
    attn_ws = tv.attn_workspace(dt, w.B, w.n_max, w.Hq, w.Hkv, w.D, max_prefix, dev)
    roots = i32(inp.roots) if inp.dynamic else None
    m_seq = i32(inp.m_seq) if inp.dynamic and inp.m_seq is not None else None
    if not inp.dynamic:
        parent_d, nn_d = i32(inp.parent), i32(inp.n_nodes)
        tok_d, tgt_d = i32(inp.tokens), i32(inp.target)

    def tree_of(c):
        if not inp.dynamic:
            return parent_d, nn_d, tok_d
        e = c["exp"]
        for s in range(w.S):
            final = (64 if m_seq is not None else w.m) if s == w.S - 1 else 0
            tv.tree_expand_rerank(c["ws"], s + 1, c["levels"][s], w.k, w.S, final_m=final,
                                  m_per_seq=m_seq, root_token=roots, n_max=w.n_max, out=e)
        return e.parent, e.n_nodes, e.token

    def attention(c, nn, anc):
        return tv.tree_verify_attn(c["q"], c["k_tree"], c["v_tree"], c["k_prefix"], c["v_prefix"],
                                   offsets, nn, anc, max_prefix, ws=attn_ws)

    if inp.dynamic:
        # target ids follow the built tree (input preparation, outside any timing)
        par, nn, tok = tree_of(copies[0])
        torch.cuda.synchronize()
        tgt_d = i32(synth.target_ids(w, par.cpu().numpy(), tok.cpu().numpy(), nn.cpu().numpy()))
        tree_host = (par.cpu().numpy(), nn.cpu().numpy())
    else:
        tree_host = (inp.parent, inp.n_nodes)

    def step(c):
        par, nn, tok = tree_of(c)
        anc, depth, pos, st = tv.tree_build(par, nn, prefix_len)
        out, lse, ast = attention(c, nn, anc)
        acc = tv.tree_accept(par, depth, anc, nn, tok, tgt_d)
        return out, lse, acc

    # eager warm-up (allocator, code objects), then one graph per input copy
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for c in copies[:2]:
            step(c)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graphs, keep = [], []
    for c in copies:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            keep.append(step(c))
        graphs.append(g)
    torch.cuda.synchronize()

    for i in range(args.warmup):
        graphs[i % R].replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(args.steps):
        graphs[i % R].replay()
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    step_ms_events = e0.elapsed_time(e1) / args.steps
    step_ms_wall = (t1 - t0) * 1e3 / args.steps

    # attention launches back to back over the rotated copies
    anc_nn = []
    for c in copies:
        par, nn, _ = tree_of(c)
        anc, _, _, _ = tv.tree_build(par, nn, prefix_len)
        anc_nn.append((nn, anc))
    torch.cuda.synchronize()
    ag = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        for c, (nn, anc) in zip(copies, anc_nn):
            attention(c, nn, anc)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(ag):
        att_keep = [attention(c, nn, anc) for c, (nn, anc) in zip(copies, anc_nn)]
    ag.replay()
    torch.cuda.synchronize()
    a0 = torch.cuda.Event(enable_timing=True)
    a1 = torch.cuda.Event(enable_timing=True)
    a0.record(stream)
    for _ in range(args.attn_reps):
        ag.replay()
    a1.record(stream)
    torch.cuda.synchronize()
    attn_ms = a0.elapsed_time(a1) / (args.attn_reps * R)
    # the spread over replays: each replay timed on its own (R back-to-back calls)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(args.attn_reps + 1)]
    ev[0].record(stream)
    for i in range(args.attn_reps):
        ag.replay()
        ev[i + 1].record(stream)
    torch.cuda.synchronize()
    per_call = np.array([ev[i].elapsed_time(ev[i + 1]) / R for i in range(args.attn_reps)])
    attn_pct = {q: float(np.percentile(per_call, p)) for q, p in (("p10", 10), ("p50", 50), ("p90", 90))}

    # KV compaction after acceptance (outside the step): each copy's accepted
    # continuation into a destination cache, launches back to back
    comp_in, rows_written = [], 0
    for c in copies:
        par, nn, tok = tree_of(c)
        anc, depth, _, _ = tv.tree_build(par, nn, prefix_len)
        alen, _, _, path = tv.tree_accept(par, depth, anc, nn, tok, tgt_d)
        comp_in.append((c, path, alen))
        rows_written += int((alen.clamp(min=-1) + 1).sum().item())
    k_dst = torch.empty((w.B * w.n_max, w.Hkv, w.D), dtype=dt, device=dev)
    v_dst = torch.empty_like(k_dst)
    dst_row = torch.arange(w.B, dtype=torch.int64, device=dev) * w.n_max
    compact = lambda c, path, alen: tv.tree_kv_compact(c["k_tree"], c["v_tree"], path, alen,
                                                       k_dst, v_dst, dst_row)
    with torch.cuda.stream(side):
        for ci in comp_in:
            compact(*ci)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    cg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cg):
        for ci in comp_in:
            compact(*ci)
    cg.replay()
    torch.cuda.synchronize()
    a0.record(stream)
    for _ in range(args.attn_reps):
        cg.replay()
    a1.record(stream)
    torch.cuda.synchronize()
    compact_ms = a0.elapsed_time(a1) / (args.attn_reps * R)
    el = 2 if w.dtype == "bf16" else 4
    compact_bytes = rows_written / R * w.Hkv * w.D * el * 2 * 2      # K and V, read and write

    # stochastic (rejection-sampling) acceptance on the first copy's tree, with seeded
    # target / draft distributions over the workload's vocabulary (up to 512 MiB of them)
    stoch = None
    V = int(w.V)
    if w.B * w.n_max * V * 8 <= (512 << 20):
        rng = np.random.default_rng(77)
        lq = rng.standard_normal((w.B, w.n_max, V), dtype=np.float32) * 2
        lp = lq + rng.standard_normal((w.B, w.n_max, V), dtype=np.float32) * np.float32(0.7)
        soft = lambda x: torch.softmax(torch.from_numpy(x).to(dev), dim=-1).contiguous()
        p_t, q_d = soft(lp), soft(lq)
        ua = torch.from_numpy(rng.random((w.B, w.n_max), dtype=np.float32)).to(dev)
        ub = torch.from_numpy(rng.random(w.B, dtype=np.float32)).to(dev)
        par, nn, tok = tree_of(copies[0])
        anc, _, _, _ = tv.tree_build(par, nn, prefix_len)
        run_s = lambda: tv.tree_accept_stochastic(par, anc, nn, tok, p_t, q_d, ua, ub)
        with torch.cuda.stream(side):
            run_s()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        sg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(sg):
            s_keep = [run_s() for _ in range(4)]
        sg.replay()
        torch.cuda.synchronize()
        a0.record(stream)
        for _ in range(args.attn_reps):
            sg.replay()
        a1.record(stream)
        torch.cuda.synchronize()
        stoch = {"us_per_call": a0.elapsed_time(a1) / (args.attn_reps * 4) * 1e3, "vocab": V,
                 "accepted_per_seq": float(s_keep[0][0].float().mean().item())}
    # the low-rank candidate head (outside the step) at a draft shape: one row per
    # frontier node (k, or 10 for a static tree), hidden size 4096, rank 256, the
    # workload's vocabulary (32000 for a static tree), 64 candidates; synthetic bf16
    # weights, the low-rank factors rotated over >= 512 MiB of copies
    rows_c = int(w.k) if inp.dynamic else 10
    Vc = int(w.V) if inp.dynamic else 32000
    dc, rc, Cc = 4096, 256, 64
    gen = torch.Generator(device=dev).manual_seed(5)
    rnd = lambda shape, sc: (torch.randn(shape, generator=gen, device=dev) * sc).to(torch.bfloat16)
    W_c = rnd((Vc, dc), 2 * dc ** -0.5)
    per_c = (rc * dc + Vc * rc) * 2
    n_c = max(2, math.ceil((512 << 20) / per_c))
    facs = [(rnd((rc, dc), dc ** -0.5), rnd((Vc, rc), 2 * rc ** -0.5)) for _ in range(n_c)]
    h_c = rnd((rows_c, dc), 1.0)
    lg_c = torch.empty((rows_c, Vc), dtype=torch.float32, device=dev)
    cd_c = torch.empty((rows_c, Cc), dtype=torch.int32, device=dev)
    ws_c = torch.empty((tv.lib().tree_candidate_workspace_size(rows_c, rc, Vc),), dtype=torch.uint8, device=dev)
    run_c = lambda fa: tv.tree_candidate_logits(h_c, fa[0], fa[1], W_c, Cc, logits=lg_c, cand=cd_c, ws=ws_c)
    with torch.cuda.stream(side):
        run_c(facs[0])
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    cg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(cg):
        for fa in facs:
            run_c(fa)
    cg.replay()
    torch.cuda.synchronize()
    a0.record(stream)
    for _ in range(max(1, args.attn_reps // 4)):
        cg.replay()
    a1.record(stream)
    torch.cuda.synchronize()
    cand_ms = a0.elapsed_time(a1) / (max(1, args.attn_reps // 4) * n_c)
    cand_bytes = (rc * dc + Vc * rc + rows_c * dc + rows_c * Cc * dc) * 2 + rows_c * Vc * 4
    cand = {"us_per_call": cand_ms * 1e3, "rows": rows_c, "hidden": dc, "rank": rc, "vocab": Vc,
            "candidates": Cc, "bytes_per_call": cand_bytes,
            "GB/s": cand_bytes / (cand_ms * 1e-3) / 1e9,
            "full_head_bytes": Vc * dc * 2 + rows_c * dc * 2 + rows_c * Vc * 4}
    del facs, W_c
    return dict(step_ms=step_ms_events, step_ms_wall=step_ms_wall, attn_ms=attn_ms, attn_pct=attn_pct,
                copies=R,
                tree=tree_host, compact_ms=compact_ms, compact_bytes=compact_bytes,
                compact_rows=rows_written / R, stochastic=stoch, candidates=cand)


def copy_reference(mib):
    """Three plain copy kernels of `mib` MiB: each reads and writes exactly mib MiB of HBM
    (an elementwise kernel, not the runtime's memcpy, so that counters see it)."""
    import torch
    src = torch.ones((mib << 20) // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_per_launch": mib << 20, "launches": 3}), flush=True)


def cpu_leg(args, inp, tree):
    """The oracle as it stands, on the host cores, over a bounded number of steps."""
    import oracle
    import synth
    from threadpoolctl import threadpool_limits, threadpool_info
    cores = len(os.sched_getaffinity(0))
    with threadpool_limits(limits=cores):
        blas = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
        return _cpu_steps(args, inp, oracle, synth, blas)


def _cpu_steps(args, inp, oracle, synth, blas):
    w = inp.w
    a = inp.attn
    q, kt, vt = a.f32("q"), a.f32("k_tree"), a.f32("v_tree")
    kp, vp = a.f32("k_prefix"), a.f32("v_prefix")
    # target ids for the accept step (input preparation, not timed)
    tgts = {}
    for b in range(min(w.B, 64)):
        if inp.dynamic:
            res = oracle.expand_rerank([lv[b:b + 1] for lv in inp.levels], w.k,
                                       w.m if inp.m_seq is None else inp.m_seq[b:b + 1],
                                       inp.roots[b:b + 1])
            tgts[b] = synth.target_ids(w, res.parent, res.token, res.n_nodes)
        else:
            tgts[b] = inp.target[b:b + 1]
    steps = 0
    queries = 0
    t0 = time.perf_counter()
    # whole steps on the first sequences until the time budget is spent
    order = list(range(w.B))
    while time.perf_counter() - t0 < args.cpu_seconds:
        b = order[steps % min(w.B, 64)]
        if inp.dynamic:
            res = oracle.expand_rerank([lv[b:b + 1] for lv in inp.levels], w.k,
                                       w.m if inp.m_seq is None else inp.m_seq[b:b + 1],
                                       inp.roots[b:b + 1])
            par, nn, tok = res.parent, res.n_nodes, res.token
        else:
            par, nn, tok = inp.parent[b:b + 1], inp.n_nodes[b:b + 1], inp.tokens[b:b + 1]
        oracle.tree_build(par, nn, inp.lens[b:b + 1])
        o0, o1 = int(a.prefix_offsets[b]), int(a.prefix_offsets[b + 1])
        oracle.tree_verify_attn(q[b:b + 1], kt[b:b + 1], vt[b:b + 1], kp[o0:o1], vp[o0:o1],
                                np.array([0, o1 - o0]), par, nn)
        oracle.tree_accept(par, tok, tgts[b], nn)
        queries += int(nn[0]) * w.Hq
        steps += 1
    dt = time.perf_counter() - t0
    return dict(value=queries / dt, unit=UNIT, cores=int(blas), kind="oracle",
                sample=f"{steps} single-sequence passes of the full path (expand/rerank when the "
                       f"tree is dynamic, tree build, float64 masked attention, accept) over "
                       f"sequences 0..{min(steps, w.B) - 1}, {dt:.1f} s of CPU time")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the library "
              f"runs on one GPU and does not shard across GPUs)", file=sys.stderr)
        sys.exit(2)
    if args.copy_mib > 0:
        copy_reference(args.copy_mib)
        return
    import synth
    w = synth.WORKLOADS[args.workload]
    inp = Inputs(w)
    g = gpu_leg(args, inp)
    parent, n_nodes = g["tree"]
    queries = int(np.sum(n_nodes)) * w.Hq
    value = queries / (g["step_ms"] * 1e-3)
    abytes = inp.algorithmic_bytes(n_nodes)
    aflops = inp.algorithmic_flops(parent, n_nodes)
    achieved_gbs = abytes / (g["attn_ms"] * 1e-3) / 1e9
    mfma_tflops = aflops / (g["attn_ms"] * 1e-3) / 1e12
    mfma_bound = w.dtype == "bf16" and aflops / abytes > RIDGE_FLOP_PER_BYTE
    line = {
        "metric": METRIC, "value": value, "unit": UNIT, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": g["step_ms"], "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv,
                   "head_dim": w.D, "prefix_tokens": int(inp.lens.sum()),
                   "tree_nodes": int(np.sum(n_nodes)), "tree": "dynamic" if inp.dynamic else "static",
                   "parallelism": "single GPU", "input_copies_rotated": g["copies"]},
        "roofline": {"bound": "mfma" if mfma_bound else "hbm",
                     "achieved": mfma_tflops if mfma_bound else achieved_gbs,
                     "peak": MFMA_BF16_PEAK_TFLOPS if mfma_bound else HBM_PEAK_GBS,
                     "unit": "TFLOP/s" if mfma_bound else "GB/s",
                     "frac": mfma_tflops / MFMA_BF16_PEAK_TFLOPS if mfma_bound
                     else achieved_gbs / HBM_PEAK_GBS,
                     "traffic": recorded_traffic(w.name),
                     "flop_per_byte": aflops / abytes,
                     "kernel": ("tree_verify_attn (attn_bf16 + attn_combine when split)"
                                if w.dtype == "bf16" else "tree_verify_attn (attn_f32)"),
                     "bytes_per_launch": abytes, "launch_ms": g["attn_ms"],
                     "launch_ms_p10_p50_p90": [g["attn_pct"][q] for q in ("p10", "p50", "p90")],
                     "hbm_gbs": achieved_gbs, "hbm_frac": achieved_gbs / HBM_PEAK_GBS,
                     "mfma_tflops": mfma_tflops, "mfma_frac": mfma_tflops / MFMA_BF16_PEAK_TFLOPS},
        "ms_per_step_wall": g["step_ms_wall"],
        "kv_compact": {"us_per_call": g["compact_ms"] * 1e3, "rows_per_call": g["compact_rows"],
                       "bytes_per_call": g["compact_bytes"],
                       "GB/s": g["compact_bytes"] / (g["compact_ms"] * 1e-3) / 1e9},
    }
    if g["stochastic"] is not None:
        line["accept_stochastic"] = g["stochastic"]
    line["candidate_head"] = g["candidates"]
    if args.cpu_seconds > 0:
        line["cpu_baseline"] = cpu_leg(args, inp, g["tree"])
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
