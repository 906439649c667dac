"""The C-ABI library on a machine without a GPU: it loads, exports what the header
declares, and rejects malformed host arguments with the documented status before
making any device call (so these tests never touch a GPU)."""

import ctypes
import os
import re

import pytest

import tree_attention_verify_ancestor_amd as tv
from tree_attention_verify_ancestor_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "treeverify.h")

OK, NULL, SHAPE, DTYPE, UNSUP, WS = 0, 1, 2, 3, 4, 5
P = ctypes.c_void_p(4096)        # a non-NULL, 16-byte aligned stand-in; never dereferenced
Z = None


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:tv_status|size_t|int|const char\*)\s+(\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.skip("libtreeverify.so not built")
    return tv.lib()


def test_every_declared_symbol_is_exported(L):
    names = declared_functions()
    assert set(names) == set(_lib.EXPORTS)
    for n in names:
        assert hasattr(L, n), n


def test_identity(L):
    assert L.tv_abi_version() == 3
    assert L.tv_status_string(0) == b"ok"
    assert b"workspace" in L.tv_status_string(WS)


def test_tree_build_validation(L):
    assert L.tree_build(1, 64, Z, P, Z, P, P, Z, Z, Z) == NULL
    assert L.tree_build(1, 64, P, P, Z, Z, P, Z, Z, Z) == NULL
    assert L.tree_build(0, 64, P, P, Z, P, P, Z, Z, Z) == SHAPE
    assert L.tree_build(1, 65, P, P, Z, P, P, Z, Z, Z) == SHAPE
    assert L.tree_build(1, 0, P, P, Z, P, P, Z, Z, Z) == SHAPE


def test_tree_accept_validation(L):
    assert L.tree_accept(1, 64, Z, P, P, P, P, P, P, P, P, Z, Z) == NULL
    assert L.tree_accept(1, 64, P, P, P, P, P, P, P, P, Z, Z, Z) == NULL
    assert L.tree_accept(2, 65, P, P, P, P, P, P, P, P, P, Z, Z) == SHAPE
    assert L.tree_accept(0, 8, P, P, P, P, P, P, P, P, P, Z, Z) == SHAPE


def _expand(L, ws=P, ws_bytes=1 << 30, B=2, k=4, max_steps=3, step=1, vocab=100, logits=P,
            final_m=0, root=Z, n_max=64, parent=Z, token=Z, score=Z, n_nodes=Z):
    return L.tree_expand_rerank(ws, ws_bytes, B, k, max_steps, step, vocab, logits, final_m, Z,
                                Z, root, n_max, parent, token, score, n_nodes, Z, Z, Z)


def test_expand_validation(L):
    assert _expand(L, logits=Z) == NULL
    assert _expand(L, k=17) == SHAPE
    assert _expand(L, k=0) == SHAPE
    assert _expand(L, step=0) == SHAPE
    assert _expand(L, step=4) == SHAPE
    assert _expand(L, vocab=3) == SHAPE
    assert _expand(L, vocab=(1 << 20) + 1) == SHAPE
    assert _expand(L, final_m=65) == SHAPE
    assert _expand(L, final_m=-1) == SHAPE
    assert _expand(L, n_max=65) == SHAPE
    assert _expand(L, k=16, max_steps=20) == SHAPE            # pool beyond 4096 slots
    assert _expand(L, final_m=8, root=P, parent=Z, token=P, score=P, n_nodes=P) == NULL
    assert _expand(L, final_m=8, root=Z, parent=P, token=P, score=P, n_nodes=P) == NULL
    assert _expand(L, ws=Z) == WS
    need = L.tree_expand_workspace_size(2, 4, 3)
    assert need > 0
    assert _expand(L, ws_bytes=need - 1) == WS


def test_draft_continue_validation(L):
    need = L.tree_expand_workspace_size(2, 4, 3)
    f = lambda ws=P, ws_bytes=need, B=2, k=4, S=3, m=8, mps=Z, more=P: L.tree_draft_continue(
        ws, ws_bytes, B, k, S, m, mps, Z, more, Z)
    assert f(more=Z) == NULL
    assert f(B=0) == SHAPE
    assert f(k=17) == SHAPE
    assert f(S=0) == SHAPE
    assert f(m=65) == SHAPE
    assert f(m=0) == SHAPE                       # no m at all
    assert f(k=16, S=20) == SHAPE                # pool beyond 4096 slots
    assert f(ws=Z) == WS
    assert f(ws_bytes=need - 1) == WS


def test_candidate_logits_validation(L):
    need = L.tree_candidate_workspace_size(4, 64, 1000)
    # z (16 padded rows x r float64) then one uint32 maximum per row and 16-token group
    assert need == 16 * 64 * 8 + (4 * 63 * 4 + 255) // 256 * 256
    assert L.tree_candidate_workspace_size(4, 513, 1000) == 0
    assert L.tree_candidate_workspace_size(4, 64, 0) == 0
    assert L.tree_candidate_workspace_size(4, 64, 128256) > L.tree_candidate_workspace_size(4, 64, 32000)
    f = lambda rows=4, d=128, r=64, V=1000, C=8, h=P, ws=P, ws_bytes=need: L.tree_candidate_logits(
        rows, d, r, V, C, h, P, P, P, P, P, ws, ws_bytes, Z)
    assert f(h=Z) == NULL
    assert f(rows=0) == SHAPE
    assert f(d=12) == SHAPE
    assert f(r=40) == SHAPE                      # r % 32
    assert f(r=520) == SHAPE
    assert f(C=0) == SHAPE
    assert f(C=257) == SHAPE
    assert f(V=7) == SHAPE
    assert f(h=ctypes.c_void_p(4096 + 8)) == UNSUP
    assert f(ws=Z) == WS
    assert f(ws_bytes=need - 1) == WS


def test_expand_workspace_size(L):
    assert L.tree_expand_workspace_size(0, 4, 3) == 0
    assert L.tree_expand_workspace_size(1, 17, 3) == 0
    assert L.tree_expand_workspace_size(1, 16, 20) == 0
    one = L.tree_expand_workspace_size(1, 10, 7)
    assert one >= 16 * (10 + 6 * 100) and one % 256 == 0
    assert L.tree_expand_workspace_size(32, 10, 7) == 32 * one


def _attn(L, dt=1, B=2, Hq=8, Hkv=2, D=128, n_max=64, Lmax=100, q=P, kt=P, vt=P, kp=P, vp=P,
          offs=P, nn=P, anc=P, out=P, ws=P, ws_bytes=1 << 34):
    return L.tree_verify_attn(dt, B, Hq, Hkv, D, n_max, Lmax, 0.0, q, kt, vt, kp, vp, offs, nn,
                              anc, out, Z, ws, ws_bytes, Z, Z)


def test_attn_validation(L):
    assert _attn(L, dt=7) == DTYPE
    assert _attn(L, Hq=6, Hkv=4) == SHAPE
    assert _attn(L, B=0) == SHAPE
    assert _attn(L, n_max=65) == SHAPE
    assert _attn(L, Lmax=-1) == SHAPE
    assert _attn(L, D=96) == UNSUP
    assert _attn(L, D=256) == UNSUP
    assert _attn(L, dt=0, D=6) == UNSUP
    assert _attn(L, dt=0, D=260) == UNSUP
    assert _attn(L, q=Z) == NULL
    assert _attn(L, anc=Z) == NULL
    assert _attn(L, out=Z) == NULL
    assert _attn(L, kp=Z) == NULL
    assert _attn(L, q=ctypes.c_void_p(4098)) == UNSUP              # misaligned
    assert _attn(L, Lmax=4096, ws=Z) == WS
    need = L.tree_verify_attn_workspace_size(1, 2, 64, 8, 2, 128, 4096)
    assert need > 0
    assert _attn(L, Lmax=4096, ws_bytes=need - 1) == WS


def test_attn_workspace_size(L):
    assert L.tree_verify_attn_workspace_size(0, 1, 10, 1, 1, 64, 32) == 0      # fp32 needs none
    assert L.tree_verify_attn_workspace_size(1, 1, 64, 8, 3, 128, 10) == 0     # Hq % Hkv
    big = L.tree_verify_attn_workspace_size(1, 4, 64, 64, 8, 128, 32768)
    small = L.tree_verify_attn_workspace_size(1, 1, 64, 32, 32, 128, 2048)
    assert big > 0 and small > 0
    # at least one fp32 partial row of D plus (max, sum) per (sequence, node, head)
    assert small >= 64 * 32 * (128 * 4 + 8)
    # a prefix that fits in one key chunk needs no partials at all
    assert L.tree_verify_attn_workspace_size(1, 1, 64, 32, 32, 128, 64) == 0


def test_attn_plan(L):
    """The launch-plan query: host only; each row-count regime takes its shape (a 70B-shaped
    batch with 512 rows per KV head: eight waves of one 32-row tile, 256 rows a
    workgroup, eight chunks of 4096 keys)."""
    plan = (ctypes.c_int32 * 8)()
    assert L.tree_verify_attn_plan(1, 4, 64, 64, 8, 128, 32768, plan) == OK
    assert list(plan) == [8, 8, 1, 1, 256, 4096, 8, 512]
    assert L.tree_verify_attn_plan(1, 2, 32, 2, 2, 128, 3000, plan) == OK
    assert list(plan)[:5] == [4, 1, 4, 1, 32]
    assert L.tree_verify_attn_plan(1, 2, 64, 4, 2, 128, 3000, plan) == OK
    assert list(plan)[:5] == [8, 4, 2, 1, 128]
    assert L.tree_verify_attn_plan(1, 1, 64, 32, 8, 128, 4096, plan) == OK   # few 256-row units
    assert list(plan)[:5] == [4, 1, 4, 2, 64]
    assert L.tree_verify_attn_plan(1, 1, 64, 32, 8, 128, 0, plan) == OK      # no prefix: one chunk
    assert plan[6] == 1
    assert L.tree_verify_attn_plan(0, 1, 64, 32, 8, 64, 100, plan) == DTYPE
    assert L.tree_verify_attn_plan(1, 1, 64, 32, 8, 96, 100, plan) == UNSUP
    assert L.tree_verify_attn_plan(1, 1, 65, 32, 8, 128, 100, plan) == SHAPE
    assert L.tree_verify_attn_plan(1, 1, 64, 32, 5, 128, 100, plan) == SHAPE
    assert L.tree_verify_attn_plan(1, 1, 64, 32, 8, 128, 100, None) == NULL


def test_cost_lookup_closed_forms(L):
    """tree_cost_lookup: exact on a power law in batch and context at and between grid
    points, linear in N between node points, the nearest grid value outside the grid,
    never falling with N; malformed tables rejected."""
    import numpy as np
    Bs, Ls, Ns = [1, 4, 16], [1024, 4096, 32768], [1, 16, 64]
    law = lambda b, l, n: 2.5 * b ** 0.7 * l ** 0.9 * (1 + n / 32)
    c = np.array([[[law(b, l, n) for n in Ns] for l in Ls] for b in Bs], np.float32)
    for (b, l) in [(1, 1024), (4, 4096), (2, 2048), (8, 20000), (16, 32768)]:
        got = tv.cost_lookup(Bs, Ls, Ns, c, b, l)
        want = np.array([law(b, l, n) for n in (1, 16, 64)])
        assert np.allclose(got[[0, 15, 63]], want, rtol=2e-6), (b, l)
        mid = [law(b, l, 1) + (law(b, l, 16) - law(b, l, 1)) * (n - 1) / 15 for n in (5, 9)]
        assert np.allclose(got[[4, 8]], mid, rtol=2e-6)
    # outside the grid: the nearest grid value
    assert np.array_equal(tv.cost_lookup(Bs, Ls, Ns, c, 64, 100000), tv.cost_lookup(Bs, Ls, Ns, c, 16, 32768))
    assert np.array_equal(tv.cost_lookup(Bs, Ls, Ns, c, 1, 10), tv.cost_lookup(Bs, Ls, Ns, c, 1, 1024))
    # a measured dip in N is lifted to the running maximum
    d = c.copy()
    d[:, :, 1] = d[:, :, 0] * 0.5
    got = tv.cost_lookup(Bs, Ls, Ns, d, 4, 4096)
    assert np.all(np.diff(got) >= 0) and got[15] == got[0]
    out = np.empty(64, np.float32)

    def call(b, l, n, cc):
        arrs = [np.ascontiguousarray(a, np.int32) for a in (b, l, n)] + [np.ascontiguousarray(cc, np.float32)]
        return L.tree_cost_lookup(arrs[0].ctypes.data, len(b), arrs[1].ctypes.data, len(l),
                                  arrs[2].ctypes.data, len(n), arrs[3].ctypes.data, 4, 4096, 64,
                                  out.ctypes.data)
    assert call(Bs, Ls, Ns, c) == OK
    assert call([4, 1, 16], Ls, Ns, c) == SHAPE                              # not ascending
    assert call(Bs, Ls, [1, 16, 65], c) == SHAPE                             # past 64 nodes
    bad = c.copy()
    bad[1, 1, 1] = 0.0
    assert call(Bs, Ls, Ns, bad) == SHAPE                                    # not positive
    assert L.tree_cost_lookup(Z, 3, Z, 3, Z, 3, Z, 4, 4096, 64, Z) == NULL


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "LIB_PATH", "/nonexistent/libtreeverify.so")
    with pytest.raises(ImportError):
        _lib.lib()


def test_product_code_never_touches_the_oracle():
    pkg = os.path.join(ROOT, "tree_attention_verify_ancestor_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle", text, re.M), f
                assert "oracle/" not in text, f


def _compact(L, dt=1, B=2, n_max=64, Hkv=2, D=128, kt=P, vt=P, path=P, alen=P, kd=P, vd=P, dst=P,
             rows=100):
    return L.tree_kv_compact(dt, B, n_max, Hkv, D, kt, vt, path, alen, kd, vd, dst, rows, Z)


def test_kv_compact_validation(L):
    assert _compact(L, dt=7) == DTYPE
    assert _compact(L, B=0) == SHAPE
    assert _compact(L, n_max=65) == SHAPE
    assert _compact(L, Hkv=0) == SHAPE
    assert _compact(L, rows=-1) == SHAPE
    assert _compact(L, kt=Z) == NULL
    assert _compact(L, path=Z) == NULL
    assert _compact(L, alen=Z) == NULL
    assert _compact(L, dst=Z) == NULL
    assert _compact(L, kd=Z) == NULL
    assert _compact(L, Hkv=1, D=4) == UNSUP                          # 8 B rows
    assert _compact(L, kd=ctypes.c_void_p(4104)) == UNSUP            # misaligned
    assert _compact(L, kd=Z, vd=Z, rows=0) == OK                     # nothing to write: no launch


def _stoch(L, B=2, n_max=64, V=1000, p=P):
    return L.tree_accept_stochastic(B, n_max, V, P, P, P, P, p, P, P, P, P, P, P, Z, Z, 0, Z)


def test_accept_stochastic_validation(L):
    assert _stoch(L, p=Z) == NULL
    assert _stoch(L, B=0) == SHAPE
    assert _stoch(L, n_max=65) == SHAPE
    assert _stoch(L, V=0) == SHAPE
    assert _stoch(L, V=-5) == SHAPE
    # no slices for bad shapes; without a device the query finds no compute units and
    # asks for no workspace (one workgroup per sequence)
    for B, n_max, V in ((0, 64, 1000), (2, 65, 1000), (2, 0, 1000), (2, 64, 0)):
        assert L.tree_accept_stochastic_workspace_size(B, n_max, V) == 0
    assert L.tree_accept_stochastic_workspace_size(4, 64, 128256) == 0


def test_budget_thresholds(L):
    import numpy as np
    out = np.empty(64, np.float32)
    cost = np.array([10, 10, 11, 13, 12, 20], np.float32)           # N = 1..6 nodes
    assert L.tree_budget_thresholds(cost.ctypes.data, 6, 0.5, out.ctypes.data) == OK
    assert np.isneginf(out[0]) and np.isneginf(out[1]) and np.isneginf(out[4])   # free, cheaper
    assert out[2] == np.float32(np.log(0.5 * 1.0)) and out[3] == np.float32(np.log(0.5 * 2.0))
    assert out[5] == np.float32(np.log(0.5 * 8.0)) and np.all(np.isneginf(out[6:]))
    assert L.tree_budget_thresholds(cost.ctypes.data, 6, 0.0, out.ctypes.data) == OK
    assert np.all(np.isneginf(out))
    assert L.tree_budget_thresholds(Z, 6, 0.5, out.ctypes.data) == NULL
    assert L.tree_budget_thresholds(cost.ctypes.data, 65, 0.5, out.ctypes.data) == SHAPE
