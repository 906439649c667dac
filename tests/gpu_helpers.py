"""Shared plumbing of the GPU parity tests: numpy <-> device tensors, and running the
HIP pipeline through the C ABI binding."""

import numpy as np
import torch

import tree_attention_verify_ancestor_amd as tv

DEV = "cuda"
ATOL = 2e-2          # absolute bound on |out - oracle|
RTOL_OF_MAX = 1e-2   # bound on max|out - oracle| / max|oracle|


def dev_i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def dev_i64(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(DEV)


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_input(a, dtype):
    """bf16 bit patterns (uint16) or float32 values -> device tensor of that dtype."""
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(DEV).view(torch.bfloat16)
    return dev_f32(a)


def host(t):
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy()
    return t.cpu().numpy()


def anc_u64(t):
    return t.cpu().numpy().view(np.uint64)


def attn_device_inputs(inp):
    return dict(q=dev_input(inp.q, inp.dtype), k_tree=dev_input(inp.k_tree, inp.dtype),
                v_tree=dev_input(inp.v_tree, inp.dtype), k_prefix=dev_input(inp.k_prefix, inp.dtype),
                v_prefix=dev_input(inp.v_prefix, inp.dtype), offsets=dev_i64(inp.prefix_offsets))


def run_attn(dinp, parent, n_nodes, max_prefix_len):
    """tree_build then tree_verify_attn on the device; returns (out, lse, status, anc)."""
    par = dev_i32(parent)
    nn = dev_i32(n_nodes)
    anc, depth, pos, st = tv.tree_build(par, nn)
    out, lse, ast = tv.tree_verify_attn(dinp["q"], dinp["k_tree"], dinp["v_tree"],
                                        dinp["k_prefix"], dinp["v_prefix"], dinp["offsets"], nn,
                                        anc, max_prefix_len)
    torch.cuda.synchronize()
    return out, lse, ast, anc


def attn_close(got, ref, what=""):
    """The attention tolerance: max abs error <= 2e-2 and <= 1e-2 of max |oracle|."""
    err = float(np.max(np.abs(got.astype(np.float64) - ref))) if ref.size else 0.0
    scale = float(np.max(np.abs(ref))) if ref.size else 0.0
    ok = err <= ATOL and (scale == 0.0 or err <= RTOL_OF_MAX * scale)
    return ok, f"{what} max_abs={err:.3e} max_ref={scale:.3e}"


def run_expand(levels, k, m, root_token, n_max=64, m_per_seq=None, budget_log=None):
    """All levels of tree_expand_rerank on the device; returns the outputs and the
    frontier tokens after each level."""
    B = levels[0].shape[0]
    S = len(levels)
    ws = tv.expand_workspace(B, k, S)
    out = tv.ExpandOutputs(B, n_max, k, DEV)
    roots = dev_i32(root_token)
    mps = None if m_per_seq is None else dev_i32(m_per_seq)
    bud = None if budget_log is None else dev_f32(budget_log)
    fronts = []
    for s in range(S):
        lg = dev_f32(levels[s])
        final = (m if np.isscalar(m) else 64) if s == S - 1 else 0
        tv.tree_expand_rerank(ws, s + 1, lg, k, S, final_m=int(final), m_per_seq=mps,
                              root_token=roots, n_max=n_max, out=out, budget_log=bud)
        fronts.append(out.frontier_token.cpu().numpy().copy())
    torch.cuda.synchronize()
    return out, fronts
