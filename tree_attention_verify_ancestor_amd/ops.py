"""Python binding of the treeverify C ABI: argument marshalling only.

Every function takes torch tensors already on the GPU, checks their dtype, shape and
layout, allocates the outputs it returns with torch (device memory is torch's job),
and calls the library on torch's current stream.  All arithmetic of every step runs
in the HIP kernels of libtreeverify.so; nothing here computes on the host.
"""

import ctypes

import torch

from . import _lib
from ._lib import check, lib

_DT = {torch.float32: _lib.TV_F32, torch.bfloat16: _lib.TV_BF16}


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t, name, dtype, ndim=None, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    return t


def abi_version():
    return lib().tv_abi_version()


def tree_build(parent, n_nodes, prefix_len=None, with_pos=True):
    """(anc int64 [B][n_max] holding the uint64 bit patterns, depth, pos, seq_status)."""
    _need(parent, "parent", torch.int32, 2)
    B, n_max = parent.shape
    _need(n_nodes, "n_nodes", torch.int32, shape=(B,))
    if prefix_len is not None:
        _need(prefix_len, "prefix_len", torch.int32, shape=(B,))
    dev = parent.device
    anc = torch.empty((B, n_max), dtype=torch.int64, device=dev)
    depth = torch.empty((B, n_max), dtype=torch.int32, device=dev)
    pos = torch.empty((B, n_max), dtype=torch.int32, device=dev) if with_pos else None
    status = torch.empty((B,), dtype=torch.int32, device=dev)
    check("tree_build", lib().tree_build(B, n_max, _ptr(parent), _ptr(n_nodes), _ptr(prefix_len),
                                         _ptr(anc), _ptr(depth), _ptr(pos), _ptr(status),
                                         _stream()))
    return anc, depth, pos, status


def expand_workspace(B, k, max_steps, device="cuda"):
    n = lib().tree_expand_workspace_size(B, k, max_steps)
    if n == 0:
        raise ValueError(f"unsupported expansion shape B={B} k={k} max_steps={max_steps}")
    return torch.empty((n,), dtype=torch.uint8, device=device)


class ExpandOutputs:
    """Outputs of the last expansion level (tree in output order) plus per-call state."""

    def __init__(self, B, n_max, k, device):
        self.parent = torch.empty((B, n_max), dtype=torch.int32, device=device)
        self.token = torch.empty((B, n_max), dtype=torch.int32, device=device)
        self.score = torch.empty((B, n_max), dtype=torch.float32, device=device)
        self.n_nodes = torch.empty((B,), dtype=torch.int32, device=device)
        self.frontier_token = torch.empty((B, k), dtype=torch.int32, device=device)
        self.seq_status = torch.empty((B,), dtype=torch.int32, device=device)


def tree_expand_rerank(ws, step, logits, k, max_steps, final_m=0, m_per_seq=None,
                       root_token=None, n_max=64, out=None, budget_log=None):
    """One EAGLE-2 level.  logits: fp32 [B][1 if step == 1 else k][vocab].  budget_log:
    optional fp32 [64] device tensor of per-place bars (see budget_thresholds)."""
    _need(ws, "ws", torch.uint8, 1)
    _need(logits, "logits", torch.float32, 3)
    B, rows, vocab = logits.shape
    if rows != (1 if step == 1 else k):
        raise ValueError(f"step {step} needs {1 if step == 1 else k} logit rows, got {rows}")
    if m_per_seq is not None:
        _need(m_per_seq, "m_per_seq", torch.int32, shape=(B,))
    if root_token is not None:
        _need(root_token, "root_token", torch.int32, shape=(B,))
    if budget_log is not None:
        _need(budget_log, "budget_log", torch.float32, shape=(64,))
    if out is None:
        out = ExpandOutputs(B, n_max, k, logits.device)
    check("tree_expand_rerank", lib().tree_expand_rerank(
        _ptr(ws), ws.numel(), B, k, max_steps, step, vocab, _ptr(logits), final_m,
        _ptr(m_per_seq), _ptr(budget_log), _ptr(root_token), n_max, _ptr(out.parent), _ptr(out.token),
        _ptr(out.score), _ptr(out.n_nodes), _ptr(out.frontier_token), _ptr(out.seq_status),
        _stream()))
    return out


def tree_draft_continue(ws, B, k, max_steps, m=0, m_per_seq=None, budget_log=None, more=None):
    """The per-level stop after a tree_expand_rerank level on workspace `ws`: int32 [B],
    1 where drafting that sequence further may still change its reranked tree."""
    _need(ws, "ws", torch.uint8, 1)
    if m_per_seq is not None:
        _need(m_per_seq, "m_per_seq", torch.int32, shape=(B,))
    if budget_log is not None:
        _need(budget_log, "budget_log", torch.float32, shape=(64,))
    if more is None:
        more = torch.empty((B,), dtype=torch.int32, device=ws.device)
    check("tree_draft_continue", lib().tree_draft_continue(
        _ptr(ws), ws.numel(), B, k, max_steps, m, _ptr(m_per_seq), _ptr(budget_log), _ptr(more),
        _stream()))
    return more


def tree_candidate_logits(h, A, Bm, W, C, logits=None, cand=None, ws=None):
    """The low-rank candidate head: bf16 h [rows][d], A [r][d], Bm [vocab][r], W [vocab][d]
    -> (fp32 logits [rows][vocab], int32 candidates [rows][C])."""
    _need(h, "h", torch.bfloat16, 2)
    rows, d = h.shape
    _need(A, "A", torch.bfloat16, 2)
    r = A.shape[0]
    _need(Bm, "Bm", torch.bfloat16, 2)
    vocab = Bm.shape[0]
    _need(W, "W", torch.bfloat16, shape=(vocab, d))
    if A.shape[1] != d or Bm.shape[1] != r:
        raise ValueError("A must be [r][d] and Bm [vocab][r]")
    dev = h.device
    if logits is None:
        logits = torch.empty((rows, vocab), dtype=torch.float32, device=dev)
    if cand is None:
        cand = torch.empty((rows, C), dtype=torch.int32, device=dev)
    if ws is None:
        ws = torch.empty((max(16, lib().tree_candidate_workspace_size(rows, r, vocab)),), dtype=torch.uint8,
                         device=dev)
    check("tree_candidate_logits", lib().tree_candidate_logits(
        rows, d, r, vocab, C, _ptr(h), _ptr(A), _ptr(Bm), _ptr(W), _ptr(logits), _ptr(cand),
        _ptr(ws), ws.numel(), _stream()))
    return logits, cand


def budget_thresholds(cost_us, threshold):
    """Per-place bars of the verify budget from a cost table: cost_us[N-1] = latency of
    one tree_verify_attn call with N nodes per tree (N = 1..n_max).  Returns a host
    float32 array [64] (computed by the library's host helper)."""
    import numpy as np
    c = np.ascontiguousarray(cost_us, dtype=np.float32)
    out = np.empty(64, dtype=np.float32)
    check("tree_budget_thresholds", lib().tree_budget_thresholds(
        c.ctypes.data, int(c.shape[0]), float(threshold), out.ctypes.data))
    return out


def cost_lookup(batch, context, nodes, cost_us, B, L, n_max=64):
    """Latency [n_max] (host float32) at batch B and context L from a cost table measured
    over the grid batch x context x nodes (cost_us float32 [len(batch)][len(context)]
    [len(nodes)]); the interpolation is the library's host helper."""
    import numpy as np
    ax = [np.ascontiguousarray(a, dtype=np.int32) for a in (batch, context, nodes)]
    c = np.ascontiguousarray(cost_us, dtype=np.float32)
    if c.shape != tuple(len(a) for a in ax):
        raise ValueError(f"cost table shape {c.shape} does not match the axes")
    out = np.empty(n_max, dtype=np.float32)
    check("tree_cost_lookup", lib().tree_cost_lookup(
        ax[0].ctypes.data, len(ax[0]), ax[1].ctypes.data, len(ax[1]), ax[2].ctypes.data,
        len(ax[2]), c.ctypes.data, int(B), int(L), int(n_max), out.ctypes.data))
    return out


def attn_workspace(dtype, B, n_max, Hq, Hkv, D, max_prefix_len, device="cuda"):
    n = lib().tree_verify_attn_workspace_size(_DT[dtype], B, n_max, Hq, Hkv, D, max_prefix_len)
    return torch.empty((max(n, 16),), dtype=torch.uint8, device=device)


def attn_plan(B, n_max, Hq, Hkv, D, max_prefix_len, dtype=torch.bfloat16):
    """The launch plan of tree_verify_attn for these sizes, as a dict (host only)."""
    plan = (ctypes.c_int32 * 8)()
    check("tree_verify_attn_plan", lib().tree_verify_attn_plan(_DT[dtype], B, n_max, Hq, Hkv, D,
                                                                max_prefix_len, plan))
    keys = ("waves", "row_groups", "key_splits", "tiles_per_wave", "rows_per_wg", "chunk_keys",
            "n_chunks", "grid")
    return dict(zip(keys, list(plan)))


def tree_verify_attn(q, k_tree, v_tree, k_prefix, v_prefix, prefix_offsets, n_nodes, anc,
                     max_prefix_len, scale=0.0, out=None, lse=None, ws=None, seq_status=None,
                     want_lse=True):
    """Tree-masked attention.  q [B][n_max][Hq][D]; tree K/V [B][n_max][Hkv][D];
    prefix K/V packed [total][Hkv][D] with int64 offsets [B+1]; anc int64 [B][n_max]."""
    if q.dtype not in _DT:
        raise TypeError(f"q must be float32 or bfloat16, got {q.dtype}")
    dt = q.dtype
    _need(q, "q", dt, 4)
    B, n_max, Hq, D = q.shape
    _need(k_tree, "k_tree", dt, 4)
    Hkv = k_tree.shape[2]
    _need(k_tree, "k_tree", dt, shape=(B, n_max, Hkv, D))
    _need(v_tree, "v_tree", dt, shape=(B, n_max, Hkv, D))
    _need(k_prefix, "k_prefix", dt, 3)
    _need(v_prefix, "v_prefix", dt, shape=tuple(k_prefix.shape))
    if k_prefix.shape[1:] != (Hkv, D):
        raise ValueError(f"k_prefix must be [total][{Hkv}][{D}], got {tuple(k_prefix.shape)}")
    _need(prefix_offsets, "prefix_offsets", torch.int64, shape=(B + 1,))
    _need(n_nodes, "n_nodes", torch.int32, shape=(B,))
    _need(anc, "anc", torch.int64, shape=(B, n_max))
    dev = q.device
    if out is None:
        out = torch.empty((B, n_max, Hq, D), dtype=dt, device=dev)
    _need(out, "out", dt, shape=(B, n_max, Hq, D))
    if lse is None and want_lse:
        lse = torch.empty((B, n_max, Hq), dtype=torch.float32, device=dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, shape=(B, n_max, Hq))
    if ws is None:
        ws = attn_workspace(dt, B, n_max, Hq, Hkv, D, max_prefix_len, dev)
    if seq_status is None:
        seq_status = torch.empty((B,), dtype=torch.int32, device=dev)
    kp = k_prefix if k_prefix.numel() else None
    vp = v_prefix if v_prefix.numel() else None
    check("tree_verify_attn", lib().tree_verify_attn(
        _DT[dt], B, Hq, Hkv, D, n_max, int(max_prefix_len), float(scale), _ptr(q), _ptr(k_tree),
        _ptr(v_tree), _ptr(kp), _ptr(vp), _ptr(prefix_offsets), _ptr(n_nodes), _ptr(anc),
        _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _ptr(seq_status), _stream()))
    return out, lse, seq_status


def tree_verify_attn_noalloc(q, k_tree, v_tree, k_prefix, v_prefix, prefix_offsets, n_nodes, anc,
                             max_prefix_len, out, seq_status, lse=None, scale=0.0):
    """tree_verify_attn without a workspace: the library's fixed per-GPU scratch holds
    the chunk partials.  The caller passes every output (out, seq_status, optional lse),
    so this call allocates nothing."""
    dt = q.dtype
    if dt not in _DT:
        raise TypeError(f"q must be float32 or bfloat16, got {q.dtype}")
    _need(q, "q", dt, 4)
    B, n_max, Hq, D = q.shape
    _need(k_tree, "k_tree", dt, 4)
    Hkv = k_tree.shape[2]
    _need(k_tree, "k_tree", dt, shape=(B, n_max, Hkv, D))
    _need(v_tree, "v_tree", dt, shape=(B, n_max, Hkv, D))
    _need(k_prefix, "k_prefix", dt, 3)
    _need(v_prefix, "v_prefix", dt, shape=tuple(k_prefix.shape))
    if k_prefix.shape[1:] != (Hkv, D):
        raise ValueError(f"k_prefix must be [total][{Hkv}][{D}], got {tuple(k_prefix.shape)}")
    _need(prefix_offsets, "prefix_offsets", torch.int64, shape=(B + 1,))
    _need(n_nodes, "n_nodes", torch.int32, shape=(B,))
    _need(anc, "anc", torch.int64, shape=(B, n_max))
    _need(out, "out", dt, shape=(B, n_max, Hq, D))
    _need(seq_status, "seq_status", torch.int32, shape=(B,))
    if lse is not None:
        _need(lse, "lse", torch.float32, shape=(B, n_max, Hq))
    kp = k_prefix if k_prefix.numel() else None
    vp = v_prefix if v_prefix.numel() else None
    check("tree_verify_attn_noalloc", lib().tree_verify_attn_noalloc(
        _DT[dt], B, Hq, Hkv, D, n_max, int(max_prefix_len), float(scale), _ptr(q), _ptr(k_tree),
        _ptr(v_tree), _ptr(kp), _ptr(vp), _ptr(prefix_offsets), _ptr(n_nodes), _ptr(anc),
        _ptr(out), _ptr(lse), _ptr(seq_status), _stream()))
    return out, lse, seq_status


def tree_accept(parent, depth, anc, n_nodes, token, target_next, want_path=True):
    """(accept_len, best_node, bonus_token, path) -- int32 tensors."""
    _need(parent, "parent", torch.int32, 2)
    B, n_max = parent.shape
    _need(depth, "depth", torch.int32, shape=(B, n_max))
    _need(anc, "anc", torch.int64, shape=(B, n_max))
    _need(n_nodes, "n_nodes", torch.int32, shape=(B,))
    _need(token, "token", torch.int32, shape=(B, n_max))
    _need(target_next, "target_next", torch.int32, shape=(B, n_max))
    dev = parent.device
    alen = torch.empty((B,), dtype=torch.int32, device=dev)
    best = torch.empty((B,), dtype=torch.int32, device=dev)
    bonus = torch.empty((B,), dtype=torch.int32, device=dev)
    path = torch.empty((B, n_max), dtype=torch.int32, device=dev) if want_path else None
    check("tree_accept", lib().tree_accept(B, n_max, _ptr(parent), _ptr(depth), _ptr(anc),
                                           _ptr(n_nodes), _ptr(token), _ptr(target_next),
                                           _ptr(alen), _ptr(best), _ptr(bonus), _ptr(path),
                                           _stream()))
    return alen, best, bonus, path


def tree_kv_compact(k_tree, v_tree, path, accept_len, k_dst, v_dst, dst_row):
    """Writes each sequence's accepted continuation (root, then the accepted path) from
    the per-node K/V [B][n_max][Hkv][D] into rows dst_row[b] .. dst_row[b] + accept_len[b]
    of k_dst / v_dst [rows][Hkv][D], in place."""
    if k_tree.dtype not in _DT:
        raise TypeError(f"k_tree must be float32 or bfloat16, got {k_tree.dtype}")
    dt = k_tree.dtype
    _need(k_tree, "k_tree", dt, 4)
    B, n_max, Hkv, D = k_tree.shape
    _need(v_tree, "v_tree", dt, shape=(B, n_max, Hkv, D))
    _need(path, "path", torch.int32, shape=(B, n_max))
    _need(accept_len, "accept_len", torch.int32, shape=(B,))
    _need(k_dst, "k_dst", dt, 3)
    if k_dst.shape[1:] != (Hkv, D):
        raise ValueError(f"k_dst must be [rows][{Hkv}][{D}], got {tuple(k_dst.shape)}")
    _need(v_dst, "v_dst", dt, shape=tuple(k_dst.shape))
    _need(dst_row, "dst_row", torch.int64, shape=(B,))
    check("tree_kv_compact", lib().tree_kv_compact(
        _DT[dt], B, n_max, Hkv, D, _ptr(k_tree), _ptr(v_tree), _ptr(path), _ptr(accept_len),
        _ptr(k_dst), _ptr(v_dst), _ptr(dst_row), int(k_dst.shape[0]), _stream()))
    return k_dst, v_dst


def tree_accept_stochastic(parent, anc, n_nodes, token, p_target, q_draft, u_accept, u_bonus,
                           want_path=True, split=True):
    """(accept_len, best_node, bonus_token, path): rejection-sampling acceptance.
    p_target, q_draft float32 [B][n_max][vocab]; u_accept [B][n_max], u_bonus [B].
    split: pass a workspace, so that each sequence's vocabulary is spread over several
    workgroups when the library's size query asks for one; False: one workgroup per
    sequence."""
    _need(parent, "parent", torch.int32, 2)
    B, n_max = parent.shape
    _need(anc, "anc", torch.int64, shape=(B, n_max))
    _need(n_nodes, "n_nodes", torch.int32, shape=(B,))
    _need(token, "token", torch.int32, shape=(B, n_max))
    _need(p_target, "p_target", torch.float32, 3)
    V = p_target.shape[2]
    _need(p_target, "p_target", torch.float32, shape=(B, n_max, V))
    _need(q_draft, "q_draft", torch.float32, shape=(B, n_max, V))
    _need(u_accept, "u_accept", torch.float32, shape=(B, n_max))
    _need(u_bonus, "u_bonus", torch.float32, shape=(B,))
    dev = parent.device
    alen = torch.empty((B,), dtype=torch.int32, device=dev)
    best = torch.empty((B,), dtype=torch.int32, device=dev)
    bonus = torch.empty((B,), dtype=torch.int32, device=dev)
    path = torch.empty((B, n_max), dtype=torch.int32, device=dev) if want_path else None
    need = lib().tree_accept_stochastic_workspace_size(B, n_max, V) if split else 0
    ws = torch.empty((need,), dtype=torch.uint8, device=dev) if need > 0 else None
    check("tree_accept_stochastic", lib().tree_accept_stochastic(
        B, n_max, V, _ptr(parent), _ptr(anc), _ptr(n_nodes), _ptr(token), _ptr(p_target),
        _ptr(q_draft), _ptr(u_accept), _ptr(u_bonus), _ptr(alen), _ptr(best), _ptr(bonus),
        _ptr(path), _ptr(ws), need, _stream()))
    return alen, best, bonus, path
