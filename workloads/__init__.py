"""Seeded synthetic inputs for prefix-shared tree decode attention.

This module only draws trees and random numbers.  It holds none of the
attention arithmetic: the tree index, the plan, the scores and the merge live
in the library (``prefix_shared_tree_amd``) and, independently, in the CPU
oracle (``oracle``).  Both consume exactly what this module produces.

A tree is given the way the KV-cache forest of the CoDec page describes it
(CoDec: Prefix-Shared Decoding Kernel for LLMs, section KV缓存管理 / KV-cache
management): nodes hold contiguous runs of K/V tokens, ``parent[i]`` is the
node whose tokens are the prefix of node ``i`` (``-1`` = child of the virtual
root), every query sits on a node and sees the tokens of every node on its
root-to-node path.  A node may be *masked*: then each query that sits on it
sees only the tokens whose bit is set in its 64-bit mask (bit j = token j),
the bit causal mask of the DEFT page (DEFT: Decoding with Flash
Tree-Attention, section 3.3 and Table 2).

Value distribution: Q, K, V ~ N(0, 1) drawn in float32, then rounded to
nearest-even bfloat16 for bf16 workloads.  Draw order per workload:
topology, lengths, query counts, masks (numpy PCG64 with ``seed``), then Q,
K and V (see :func:`make_tensors`).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

__all__ = [
    "TreeSpec",
    "config",
    "config_names",
    "random_tree",
    "make_tensors",
    "draft_tree_masks",
]


@dataclass
class TreeSpec:
    """A tree of KV nodes plus the decode queries that sit on it."""

    name: str
    parent: np.ndarray  # int32 [N], parent[i] < i, -1 = child of the virtual root
    kv_len: np.ndarray  # int32 [N], >= 1
    kv_offset: np.ndarray  # int64 [N], token offset of node i in the K/V pools
    query_node: np.ndarray  # int32 [B]
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    dtype: str  # "f32" or "bf16"
    seed: int
    query_mask: Optional[np.ndarray] = None  # uint64 [B] or None
    node_masked: Optional[np.ndarray] = None  # uint8 [N] or None
    total_tokens: int = field(init=False)

    def __post_init__(self):
        self.parent = np.ascontiguousarray(self.parent, dtype=np.int32)
        self.kv_len = np.ascontiguousarray(self.kv_len, dtype=np.int32)
        self.kv_offset = np.ascontiguousarray(self.kv_offset, dtype=np.int64)
        self.query_node = np.ascontiguousarray(self.query_node, dtype=np.int32)
        if self.query_mask is not None:
            self.query_mask = np.ascontiguousarray(self.query_mask, dtype=np.uint64)
        if self.node_masked is not None:
            self.node_masked = np.ascontiguousarray(self.node_masked, dtype=np.uint8)
        if len(self.kv_len):
            self.total_tokens = int((self.kv_offset + self.kv_len).max())
        else:
            self.total_tokens = 0

    @property
    def num_nodes(self) -> int:
        return int(self.parent.shape[0])

    @property
    def num_queries(self) -> int:
        return int(self.query_node.shape[0])

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def _offsets(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(len(lengths), dtype=np.int64)
    if len(lengths) > 1:
        off[1:] = np.cumsum(lengths)[:-1]
    return off


# ---------------------------------------------------------------------------
# The five named workloads
# ---------------------------------------------------------------------------

def _config1() -> TreeSpec:
    """Tiny two-level tree: one 256-token root, four 32-token leaves.

    The shape of DEFT's two-query cascade example (K_a = K0 || K1,
    K_b = K0 || K2; DEFT page, section 3.2) widened to four leaves.
    """
    parent = [-1, 0, 0, 0, 0]
    lens = [256, 32, 32, 32, 32]
    return TreeSpec("tiny-2level-f32", np.array(parent), np.array(lens), _offsets(lens),
                    np.array([1, 2, 3, 4]), 4, 4, 64, "f32", 1)


def _config2() -> TreeSpec:
    """Document-QA tree: a 32768-token shared root, 64 private 512-token leaves."""
    parent = [-1] + [0] * 64
    lens = [32768] + [512] * 64
    return TreeSpec("docqa-32k-64x512", np.array(parent), np.array(lens), _offsets(lens),
                    np.arange(1, 65), 32, 8, 128, "bf16", 2)


def _config3() -> TreeSpec:
    """Few-shot three-level tree: 4000-token root, 8 x 1024, 16 x 128 leaves under each."""
    parent = [-1]
    lens = [4000]
    for c in range(8):
        parent.append(0)
        lens.append(1024)
    # Leaves in breadth-first order: children of node 1 first, then node 2, ...
    leaves = []
    for c in range(8):
        for _ in range(16):
            parent.append(1 + c)
            lens.append(128)
            leaves.append(len(parent) - 1)
    return TreeSpec("fewshot-4000-8x1024-128x128", np.array(parent), np.array(lens),
                    _offsets(lens), np.array(leaves), 32, 8, 128, "bf16", 3)


def draft_tree_masks(parents: np.ndarray) -> np.ndarray:
    """Ancestor-or-self bit masks of a draft token tree stored in topological order.

    ``parents[j]`` is the parent token of draft token ``j`` inside the draft
    node (-1 for the draft root).  The query of draft token ``j`` sees its
    ancestors and itself: the tree mask of speculative verification (shared
    prefix blog, section 4.5.4), with bit j = token j (DEFT's 64-bit mask).
    """
    n = len(parents)
    assert n <= 64
    masks = np.zeros(n, dtype=np.uint64)
    for j in range(n):
        bits = 0
        t = j
        while t != -1:
            bits |= 1 << t
            t = int(parents[t])
        masks[j] = np.uint64(bits)
    return masks


def _config4() -> TreeSpec:
    """Speculative-decoding trees: 16 private prefixes, each topped by a 64-token draft tree.

    Draw order: for each request its draft topology (parent of token i uniform
    over the earlier tokens of depth < 8), then the 16 prefix lengths, integer
    uniform on [2048, 10240].
    """
    rng = np.random.default_rng(4)
    drafts = []
    for _ in range(16):
        par = np.full(64, -1, dtype=np.int64)
        depth = np.zeros(64, dtype=np.int64)
        depth[0] = 1
        for i in range(1, 64):
            cand = np.nonzero(depth[:i] < 8)[0]
            p = int(cand[rng.integers(0, len(cand))])
            par[i] = p
            depth[i] = depth[p] + 1
        drafts.append(par)
    prefix = rng.integers(2048, 10240, size=16, endpoint=True)
    parent, lens, masked = [], [], []
    qnode, qmask = [], []
    for r in range(16):
        pid = len(parent)
        parent.append(-1)
        lens.append(int(prefix[r]))
        masked.append(0)
        did = len(parent)
        parent.append(pid)
        lens.append(64)
        masked.append(1)
        m = draft_tree_masks(drafts[r])
        for j in range(64):
            qnode.append(did)
            qmask.append(m[j])
    return TreeSpec("specdec-16x(2k-10k)+64draft", np.array(parent), np.array(lens),
                    _offsets(lens), np.array(qnode), 32, 32, 128, "bf16", 4,
                    query_mask=np.array(qmask, dtype=np.uint64),
                    node_masked=np.array(masked))


def _attach(rng, num_children: int, num_parents: int) -> np.ndarray:
    """Parent index (0..num_parents-1) for each child: one per parent first, rest uniform."""
    assert num_children >= num_parents
    rest = rng.integers(0, num_parents, size=num_children - num_parents)
    par = np.concatenate([np.arange(num_parents), rest])
    return np.sort(par, kind="stable")  # breadth-first ids: grouped by parent


def _zipf_truncated(rng, s: float, kmax: int, size: int) -> np.ndarray:
    k = np.arange(1, kmax + 1, dtype=np.float64)
    p = k ** (-s)
    p /= p.sum()
    return rng.choice(np.arange(1, kmax + 1), size=size, p=p)


def _config5(kind: str) -> TreeSpec:
    """Skewed random tree: every root-to-leaf path has 4 nodes, 256 leaves.

    Level sizes: 1 root, c2 ~ U{2..16}, c3 ~ U{c2..64}, 256 leaves; children
    attach one per parent first, the rest uniformly; ids breadth-first.
    Node lengths log-uniform on [16, 65536]; queries per leaf truncated
    Zipf(1.2) on {1..16}.
    """
    rng = np.random.default_rng(5)
    c2 = int(rng.integers(2, 16, endpoint=True))
    c3 = int(rng.integers(c2, 64, endpoint=True))
    nleaf = 256
    parent = [-1]
    parent += [0] * c2
    lvl3 = _attach(rng, c3, c2)
    parent += [1 + int(p) for p in lvl3]
    lvl4 = _attach(rng, nleaf, c3)
    parent += [1 + c2 + int(p) for p in lvl4]
    n = len(parent)
    u = rng.random(n)
    lens = np.minimum(65536, np.floor(np.exp(math.log(16) + u * (math.log(65536) - math.log(16)))))
    lens = lens.astype(np.int64)
    nq = _zipf_truncated(rng, 1.2, 16, nleaf)
    first_leaf = 1 + c2 + c3
    qnode = np.repeat(np.arange(first_leaf, first_leaf + nleaf), nq)
    if kind == "mqa":
        hq, hkv = 32, 1
    elif kind == "mha":
        hq, hkv = 32, 32
    else:
        raise ValueError(kind)
    return TreeSpec(f"skewed-depth4-256leaf-{kind}", np.array(parent), lens, _offsets(lens),
                    qnode, hq, hkv, 128, "bf16", 5)


_CONFIGS = {
    "1": _config1,
    "2": _config2,
    "3": _config3,
    "4": _config4,
    "5-mqa": lambda: _config5("mqa"),
    "5-mha": lambda: _config5("mha"),
}


def config_names():
    return list(_CONFIGS)


def config(name) -> TreeSpec:
    """One of the named workloads: "1", "2", "3", "4", "5-mqa", "5-mha"."""
    return _CONFIGS[str(name)]()


# ---------------------------------------------------------------------------
# Random small trees for tests
# ---------------------------------------------------------------------------

def random_tree(seed: int, *, max_nodes: int = 6, max_len: int = 40, max_queries: int = 6,
                num_q_heads: int = 4, num_kv_heads: int = 2, head_dim: int = 64,
                dtype: str = "f32", masked_prob: float = 0.0, min_len: int = 1) -> TreeSpec:
    """A random forest (parents before children) with queries on random nodes.

    With ``masked_prob`` > 0 some nodes of at most 64 tokens are masked; each
    query on such a node gets a random non-empty mask of its tokens.
    """
    rng = np.random.default_rng(seed)
    n = int(rng.integers(1, max_nodes, endpoint=True))
    parent = np.array([-1] + [int(rng.integers(-1, i)) for i in range(1, n)], dtype=np.int32)
    lens = rng.integers(min_len, max_len, size=n, endpoint=True)
    # Shuffle the pool placement so node order and token order differ.
    perm = rng.permutation(n)
    off = np.zeros(n, dtype=np.int64)
    pos = 0
    for i in perm:
        off[i] = pos
        pos += int(lens[i]) + int(rng.integers(0, 3))  # small gaps between nodes
    b = int(rng.integers(1, max_queries, endpoint=True))
    qnode = rng.integers(0, n, size=b).astype(np.int32)
    node_masked = None
    qmask = None
    if masked_prob > 0:
        node_masked = ((rng.random(n) < masked_prob) & (lens <= 64)).astype(np.uint8)
        qmask = np.zeros(b, dtype=np.uint64)
        for r in range(b):
            node = qnode[r]
            if node_masked[node]:
                L = int(lens[node])
                bits = 0
                while bits == 0:
                    bits = int(sum(1 << j for j in range(L) if rng.random() < 0.5))
                qmask[r] = np.uint64(bits)
    return TreeSpec(f"random-{seed}", parent, lens, off, qnode, num_q_heads, num_kv_heads,
                    head_dim, dtype, seed, query_mask=qmask, node_masked=node_masked)


# ---------------------------------------------------------------------------
# Tensors
# ---------------------------------------------------------------------------

def make_tensors(spec: TreeSpec, device="cpu", *, kv_tokens: Optional[int] = None, q_scale: float = 1.0):
    """Q [B, H_q, d] and head-major K, V pools [H_kv, T, d], seeded by ``spec.seed``.

    On ``cpu`` numpy PCG64 draws the float32 normals; on a GPU device torch's
    device generator draws them head by head (pools of tens of GB are never
    staged on the host).  bf16 workloads round to nearest even.  The oracle
    always consumes the returned (rounded) values.  ``q_scale`` multiplies Q
    before rounding (a peaked-attention stress input).
    """
    import torch

    dt = torch.float32 if spec.dtype == "f32" else torch.bfloat16
    T = kv_tokens if kv_tokens is not None else spec.total_tokens
    B, hq, hkv, d = spec.num_queries, spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    dev = torch.device(device)
    if dev.type == "cpu":
        rng = np.random.default_rng([spec.seed, 1000])
        q = torch.from_numpy(rng.standard_normal((B, hq, d), dtype=np.float32) * np.float32(q_scale)).to(dt)
        k = torch.from_numpy(rng.standard_normal((hkv, T, d), dtype=np.float32)).to(dt)
        v = torch.from_numpy(rng.standard_normal((hkv, T, d), dtype=np.float32)).to(dt)
        return q.contiguous(), k.contiguous(), v.contiguous()
    g = torch.Generator(device=dev)
    g.manual_seed(spec.seed * 1000003 + 17)
    q = (torch.randn((B, hq, d), generator=g, device=dev, dtype=torch.float32) * q_scale).to(dt)
    k = torch.empty((hkv, T, d), device=dev, dtype=dt)
    v = torch.empty((hkv, T, d), device=dev, dtype=dt)
    for h in range(hkv):
        k[h] = torch.randn((T, d), generator=g, device=dev, dtype=torch.float32).to(dt)
        v[h] = torch.randn((T, d), generator=g, device=dev, dtype=torch.float32).to(dt)
    return q, k, v


def page_pools(spec: TreeSpec, k, v, page_size: int, *, spare_pages: int = 0, fill: float = float("nan"),
               scatter: bool = True):
    """A paged copy of the contiguous pools ``k``, ``v`` ([H_kv, T, d]).

    Node i gets ceil(kv_len[i] / page_size) + ``spare_pages`` pages.  The
    physical page numbers are a seeded draw without replacement from a range
    one eighth larger than needed, so pages are scattered and the pool has
    holes.  Rows not holding a token (page tails, holes) are set to ``fill``
    (NaN by default: a read past a node's end poisons the output).  With
    ``scatter`` False the pages are numbered in order without holes.  Returns
    ``({"page_size", "page_ptr", "page_idx"}, k_paged, v_paged)``; token j
    of node i is row ``page_idx[page_ptr[i] + j // P] * P + j % P``.  The
    oracle keeps reading the contiguous ``k``, ``v`` with ``spec.kv_offset``.
    """
    import torch

    P = int(page_size)
    kv_len = np.asarray(spec.kv_len, dtype=np.int64)
    npg = (kv_len + P - 1) // P + int(spare_pages)
    page_ptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    total = int(page_ptr[-1])
    rng = np.random.default_rng([spec.seed, 7919, P])
    if scatter:
        page_idx = rng.permutation(total + max(1, total // 8))[:total].astype(np.int32)
    else:
        page_idx = np.arange(total, dtype=np.int32)
    pool_rows = (int(page_idx.max()) + 1) * P if total else 0
    src = np.full(pool_rows, -1, dtype=np.int64)  # contiguous row feeding each paged row
    for i in range(spec.num_nodes):
        j = np.arange(int(kv_len[i]), dtype=np.int64)
        pages = page_idx[page_ptr[i]:page_ptr[i + 1]].astype(np.int64)
        src[pages[j // P] * P + j % P] = int(spec.kv_offset[i]) + j
    src_t = torch.from_numpy(src).to(k.device)
    valid = src_t >= 0
    out = []
    for x in (k, v):
        xp = torch.full((x.shape[0], pool_rows, x.shape[2]), fill, dtype=x.dtype, device=x.device)
        xp[:, valid] = x[:, src_t[valid]]
        out.append(xp)
    return {"page_size": P, "page_ptr": page_ptr, "page_idx": page_idx}, out[0], out[1]


# ---------------------------------------------------------------------------
# Tree shapes of the CoDec evaluation (binary 2T ... 5-ary 5T and a degenerate
# tree DT; CoDec page, 实验结果 section 1).  The page names the shapes and
# sweeps sequence length, batch and shared-prefix ratio without printing the
# trees, so the sizes below are a reading of them: every query's path holds
# `path_len` tokens, the root `shared` of them, the rest split evenly over
# the deeper levels; one query per leaf.
# ---------------------------------------------------------------------------

def kary_tree(k: int, depth: int, *, path_len: int = 4096, shared: float = 0.5, num_q_heads: int = 32,
              num_kv_heads: int = 8, head_dim: int = 128, dtype: str = "bf16", seed: int = 7) -> TreeSpec:
    """Full k-ary tree of `depth` levels (k^(depth-1) leaves, one query each)."""
    root = int(round(path_len * shared))
    per = max(1, (path_len - root) // max(1, depth - 1))
    parent, lens, level = [-1], [root], [0]
    for lv in range(1, depth):
        for p in [i for i, d in enumerate(level) if d == lv - 1]:
            for _ in range(k):
                parent.append(p)
                lens.append(per)
                level.append(lv)
    leaves = np.array([i for i, d in enumerate(level) if d == depth - 1], dtype=np.int32)
    return TreeSpec(f"{k}T-depth{depth}", np.array(parent), np.array(lens), _offsets(lens), leaves,
                    num_q_heads, num_kv_heads, head_dim, dtype, seed)


def degenerate_tree(queries: int, *, path_len: int = 4096, shared: float = 0.5, num_q_heads: int = 32,
                    num_kv_heads: int = 8, head_dim: int = 128, dtype: str = "bf16", seed: int = 7) -> TreeSpec:
    """Degenerate tree DT: a chain of `queries` nodes below the root, each with
    a leaf hanging off it, so query i shares the root and i chain nodes with
    the others and prefixes vary from shared to nearly private.  The chain
    splits the unshared part of the longest path evenly; every leaf tops its
    path up to `path_len` tokens."""
    root = int(round(path_len * shared))
    step = max(1, (path_len - root) // (queries + 1))
    parent, lens, leaves = [-1], [root], []
    chain = 0
    for i in range(queries):
        parent.append(chain)  # next chain node
        lens.append(step)
        chain = len(parent) - 1
        parent.append(chain)  # leaf of query i
        lens.append(max(1, path_len - root - (i + 1) * step))
        leaves.append(len(parent) - 1)
    return TreeSpec(f"DT-{queries}", np.array(parent), np.array(lens), _offsets(lens), np.array(leaves),
                    num_q_heads, num_kv_heads, head_dim, dtype, seed)
