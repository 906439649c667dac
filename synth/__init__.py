"""Seeded synthetic inputs for draft-tree verification workloads.

This module is the only code both the oracle side (tests, CPU baseline) and the
HIP side (tests, bench) consume.  It draws random numbers and lays them out; it
holds none of the method's arithmetic (no masks, softmax, ranking or acceptance).

Every stream is ``numpy.random.default_rng(SeedSequence([workload_id, tensor_id]))``
with fixed tensor ids: 0 Q, 1 prefix K, 2 prefix V, 3 tree K, 4 tree V, 5 draft
logits, 6 tree shape / lengths, 7 token ids.  Half-precision inputs are drawn in
float32 and rounded to bfloat16 (round to nearest even); the oracle receives the
exact float32 upcast of the very same bits.

Workloads (ids 1..5) follow the five verification configurations studied: a tiny
float32 case, a Llama-7B-shaped MHA layer with a static tree, an EAGLE-2 dynamic
tree with GQA, a 70B-shaped long-context layer and a ragged serving batch.  The
pages fix none of these sizes; they only fix the structure (a depth-3, 10-token
example tree; left-heavy static trees; top-k expansion; greedy acceptance).
"""

from dataclasses import dataclass, field
from typing import Optional

import numpy as np

T_Q, T_KP, T_VP, T_KT, T_VT, T_LOGITS, T_TREE, T_TOKENS = range(8)

# Static trees (parent arrays, root = node 0).  The 10-node tree is the reading of
# the depth-3, 10-token draft-tree example of the "EAGLE" notes (root with three
# children, then two / one / none, the left subtree deepest).  The 26-node tree is
# a depth-5 left-heavy tree with level sizes 1/4/7/7/4/3.
EAGLE1_EXAMPLE_TREE = [-1, 0, 0, 0, 1, 1, 2, 4, 4, 5]
STATIC_TREE_26 = [-1, 0, 0, 0, 0, 1, 1, 1, 2, 2, 3, 4, 5, 5, 5, 6, 6, 7, 8, 12, 12, 13, 14,
                  19, 19, 20]


@dataclass
class Workload:
    wid: int
    name: str
    B: int
    Hq: int
    Hkv: int
    D: int
    dtype: str                      # "f32" or "bf16"
    prefix: object                  # int, or (lo, hi) inclusive uniform per sequence
    tree: object                    # list (static parent array) or "dynamic"
    qkv_std: float = 1.0
    S: int = 0                      # expansion levels (dynamic trees)
    k: int = 0                      # top-k per expanded node / frontier width
    V: int = 32000                  # vocabulary
    m: object = 0                   # kept nodes incl. root: int, or (lo, hi) per sequence
    q_match: Optional[float] = None  # per-node match probability of target ids; None = uniform ids
    logit_std: float = 2.0
    n_max: int = 64


WORKLOADS = {
    1: Workload(1, "tiny_f32_d64_L32_tree10", B=1, Hq=1, Hkv=1, D=64, dtype="f32", prefix=32,
                tree=EAGLE1_EXAMPLE_TREE, qkv_std=1.0, q_match=None),
    2: Workload(2, "llama7b_mha32_d128_L2048_static26", B=1, Hq=32, Hkv=32, D=128, dtype="bf16",
                prefix=2048, tree=STATIC_TREE_26, qkv_std=0.5, q_match=0.8),
    3: Workload(3, "eagle2_gqa32x8_d128_L4096_dyn60", B=1, Hq=32, Hkv=8, D=128, dtype="bf16",
                prefix=4096, tree="dynamic", qkv_std=0.5, S=6, k=10, V=32000, m=60, q_match=0.8),
    4: Workload(4, "llama70b_gqa64x8_d128_B4_L32768_dyn64", B=4, Hq=64, Hkv=8, D=128, dtype="bf16",
                prefix=32768, tree="dynamic", qkv_std=0.5, S=8, k=8, V=128256, m=64, q_match=0.8),
    5: Workload(5, "serving_gqa32x8_d128_B32_L512-8192_dyn16-64", B=32, Hq=32, Hkv=8, D=128,
                dtype="bf16", prefix=(512, 8192), tree="dynamic", qkv_std=0.5, S=7, k=10,
                V=32000, m=(16, 64), q_match=0.75),
}


def rng_for(wid, tensor_id, sub=None):
    key = [int(wid), int(tensor_id)] + ([] if sub is None else [int(sub)])
    return np.random.default_rng(np.random.SeedSequence(key))


def bf16_bits(x):
    """float32 array -> uint16 bfloat16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return rounded.astype(np.uint16)


def bf16_to_f32(bits):
    """uint16 bfloat16 bit patterns -> exact float32 values."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal(wid, tensor_id, shape, std, dtype):
    """Seeded N(0, std^2) tensor: float32 values, or bf16 bits when dtype == "bf16"."""
    x = rng_for(wid, tensor_id).standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return bf16_bits(x) if dtype == "bf16" else x


def prefix_lengths(w):
    if isinstance(w.prefix, tuple):
        lo, hi = w.prefix
        return rng_for(w.wid, T_TREE).integers(lo, hi + 1, size=w.B).astype(np.int64)
    return np.full(w.B, int(w.prefix), dtype=np.int64)


def kept_counts(w):
    """Nodes per tree (root included): static tree size, or the kept-node count m."""
    if isinstance(w.tree, list):
        return np.full(w.B, len(w.tree), dtype=np.int32)
    if isinstance(w.m, tuple):
        lo, hi = w.m
        return rng_for(w.wid, T_TREE, 1).integers(lo, hi + 1, size=w.B).astype(np.int32)
    return np.full(w.B, int(w.m), dtype=np.int32)


@dataclass
class AttnInputs:
    """Verification-attention inputs.  Half-precision tensors are uint16 bf16 bits."""
    dtype: str
    q: np.ndarray                 # [B][n_max][Hq][D]
    k_tree: np.ndarray            # [B][n_max][Hkv][D]
    v_tree: np.ndarray
    k_prefix: np.ndarray          # [sum L][Hkv][D]
    v_prefix: np.ndarray
    prefix_offsets: np.ndarray    # int64 [B+1]
    extras: dict = field(default_factory=dict)

    def f32(self, name):
        a = getattr(self, name)
        return bf16_to_f32(a) if self.dtype == "bf16" else a


def attention_inputs(w, wid=None):
    """Q, tree K/V and packed prefix K/V of a workload (seeded by its id)."""
    wid = w.wid if wid is None else wid
    lens = prefix_lengths(w)
    offs = np.zeros(w.B + 1, dtype=np.int64)
    offs[1:] = np.cumsum(lens)
    tot = int(offs[-1])
    return AttnInputs(
        dtype=w.dtype,
        q=normal(wid, T_Q, (w.B, w.n_max, w.Hq, w.D), w.qkv_std, w.dtype),
        k_tree=normal(wid, T_KT, (w.B, w.n_max, w.Hkv, w.D), w.qkv_std, w.dtype),
        v_tree=normal(wid, T_VT, (w.B, w.n_max, w.Hkv, w.D), w.qkv_std, w.dtype),
        k_prefix=normal(wid, T_KP, (tot, w.Hkv, w.D), w.qkv_std, w.dtype),
        v_prefix=normal(wid, T_VP, (tot, w.Hkv, w.D), w.qkv_std, w.dtype),
        prefix_offsets=offs,
    )


def static_tree(w):
    """(parent int32 [B][n_max], n_nodes int32 [B]) of a static-tree workload."""
    n = len(w.tree)
    parent = np.full((w.B, w.n_max), -1, dtype=np.int32)
    parent[:, :n] = np.asarray(w.tree, dtype=np.int32)
    return parent, np.full(w.B, n, dtype=np.int32)


def draft_logits(w):
    """Per level s = 1..S: float32 [B][1 if s == 1 else k][V], entries logit_std * N(0, 1)."""
    r = rng_for(w.wid, T_LOGITS)
    out = []
    for s in range(w.S):
        rows = 1 if s == 0 else w.k
        x = r.standard_normal(size=(w.B, rows, w.V), dtype=np.float32)
        x *= np.float32(w.logit_std)
        out.append(x)
    return out


def root_tokens(w):
    return rng_for(w.wid, T_TOKENS).integers(0, w.V, size=w.B).astype(np.int32)


def static_draft_tokens(w):
    """Draft token ids of a static tree: uniform in [0, V); node 0 holds the root token."""
    r = rng_for(w.wid, T_TOKENS)
    roots = r.integers(0, w.V, size=w.B).astype(np.int32)
    tok = r.integers(0, w.V, size=(w.B, w.n_max)).astype(np.int32)
    tok[:, 0] = roots
    return tok


def target_ids(w, parent, token, n_nodes, stream=T_TOKENS + 100):
    """Target greedy ids per node.

    With ``q_match`` None: independent uniform ids.  Otherwise, for each node with
    children: with probability q_match the id equals the token of one of its
    children chosen uniformly, else it is a uniform id equal to none of them;
    leaves get uniform ids.  (The tree is an input here; nothing is accepted.)
    """
    r = rng_for(w.wid, stream)
    B, n_max = parent.shape
    tgt = r.integers(0, w.V, size=(B, n_max)).astype(np.int32)
    if w.q_match is None:
        return tgt
    for b in range(B):
        n = int(n_nodes[b])
        kids = [[] for _ in range(n)]
        for i in range(1, n):
            p = int(parent[b, i])
            if 0 <= p < n:
                kids[p].append(i)
        for p in range(n):
            if not kids[p]:
                continue
            toks = {int(token[b, c]) for c in kids[p]}
            if r.random() < w.q_match:
                tgt[b, p] = int(token[b, kids[p][int(r.integers(0, len(kids[p])))]])
            else:
                t = int(r.integers(0, w.V))
                while t in toks:
                    t = int(r.integers(0, w.V))
                tgt[b, p] = t
    return tgt


# ---------------------------------------------------------------- small random cases

def random_parents(rng, n, shape="random"):
    """A valid parent array of n nodes: "random", "chain", "star" or "broom"."""
    p = np.full(n, -1, dtype=np.int32)
    for i in range(1, n):
        if shape == "chain":
            p[i] = i - 1
        elif shape == "star":
            p[i] = 0
        elif shape == "broom":        # a chain of half the nodes, then a fan on its tip
            p[i] = i - 1 if i <= n // 2 else n // 2
        else:
            p[i] = int(rng.integers(0, i))
    return p


def random_attention_case(seed, B, Hq, Hkv, D, prefix_lens, n_nodes, dtype="bf16", std=0.5,
                          n_max=64, shapes=None):
    """Seeded inputs for one small verification-attention case, plus its trees."""
    rng = np.random.default_rng(np.random.SeedSequence([1000, int(seed)]))
    lens = np.asarray(prefix_lens, dtype=np.int64)
    offs = np.zeros(B + 1, dtype=np.int64)
    offs[1:] = np.cumsum(lens)
    tot = int(offs[-1])

    def draw(shape):
        x = rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)
        return bf16_bits(x) if dtype == "bf16" else x

    inp = AttnInputs(dtype=dtype, q=draw((B, n_max, Hq, D)), k_tree=draw((B, n_max, Hkv, D)),
                     v_tree=draw((B, n_max, Hkv, D)), k_prefix=draw((tot, Hkv, D)),
                     v_prefix=draw((tot, Hkv, D)), prefix_offsets=offs)
    parent = np.full((B, n_max), -1, dtype=np.int32)
    for b in range(B):
        shape = "random" if shapes is None else shapes[b % len(shapes)]
        parent[b, :n_nodes[b]] = random_parents(rng, int(n_nodes[b]), shape)
    return inp, parent, np.asarray(n_nodes, dtype=np.int32)
