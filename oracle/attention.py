"""Plain per-query tree decode attention in float64 (test infrastructure only).

Definition followed.  CoDec (CoDec: Prefix-Shared Decoding Kernel for LLMs),
section 背景知识与设计原则 (background): attention is
O = softmax(Q K^T / sqrt(d)) V; section KV缓存管理 (KV-cache management):
the KV cache is a forest of nodes joined under a virtual root, each edge
p -> c says p is a prefix of c, and a query attends to the tokens of the
nodes on its path, under a visibility mask; section 块内内核原语 (PAC): the
partial computation is "exactly ordinary attention".  DEFT (DEFT: Decoding
with Flash Tree-Attention), section 速读: the LSE of a query is the log of
the sum of exp(q k^T / sqrt(d)).

So for query r and q-head h: take the nodes from the virtual root down to the
query's node, concatenate their tokens in that order (for a masked query
node, only the tokens whose mask bit is set), and compute one full softmax
over all of them in float64 from the exact stored input values.

Readings where the pages are silent: kv head of q-head h is h // (H_q/H_kv)
(contiguous groups); scale 1/sqrt(d); the query's own node is visible in
full (its current token's K/V is already in the cache); mask bit j <->
token j of the node, set = visible.
"""
from __future__ import annotations

import numpy as np


def _as_f64(x):
    """Exact float64 copy of a numpy array or torch tensor (bf16/f32 upcast is lossless)."""
    if isinstance(x, np.ndarray):
        return x.astype(np.float64)
    import torch

    return x.detach().to("cpu", torch.float64).numpy()


def _path(parent, node):
    path = []
    n = int(node)
    while n != -1:
        path.append(n)
        n = int(parent[n])
    path.reverse()
    return path


def visible_tokens(spec, r) -> np.ndarray:
    """Pool positions of the tokens query ``r`` sees, in root-to-node order."""
    qn = int(spec.query_node[r])
    toks = []
    for node in _path(spec.parent, qn):
        base = int(spec.kv_offset[node])
        length = int(spec.kv_len[node])
        masked = (spec.node_masked is not None and spec.node_masked[node]
                  and node == qn and spec.query_mask is not None)
        if masked:
            bits = int(spec.query_mask[r])
            toks.extend(base + j for j in range(length) if (bits >> j) & 1)
        else:
            toks.extend(range(base, base + length))
    return np.asarray(toks, dtype=np.int64)


def _gather(pool, h, idx):
    """Rows ``idx`` of head ``h`` of a [H_kv, T, d] pool as float64."""
    if isinstance(pool, np.ndarray):
        return pool[h, idx].astype(np.float64)
    import torch

    t = torch.as_tensor(idx, dtype=torch.long)
    return pool[h].index_select(0, t.to(pool.device)).to("cpu", torch.float64).numpy()


def attend(spec, q, k, v, *, scale=None, queries=None):
    """O [n, H_q, d] and LSE [n, H_q] (natural log) for the listed queries.

    ``q`` is [B, H_q, d]; ``k``/``v`` are head-major pools [H_kv, T, d]
    (numpy arrays or torch tensors in any dtype; values are used exactly).
    """
    hq, hkv, d = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    g = hq // hkv
    if scale is None:
        scale = 1.0 / np.sqrt(d)
    if queries is None:
        queries = range(spec.num_queries)
    queries = list(queries)
    O = np.zeros((len(queries), hq, d))
    L = np.zeros((len(queries), hq))
    for qi, r in enumerate(queries):
        idx = visible_tokens(spec, r)
        if len(idx) == 0:
            raise ValueError(f"query {r} sees no token")
        qr = _as_f64(q[r])  # [H_q, d]
        for kh in range(hkv):
            K = _gather(k, kh, idx)  # [n, d]
            V = _gather(v, kh, idx)
            heads = slice(kh * g, (kh + 1) * g)
            s = scale * (qr[heads] @ K.T)  # [g, n]
            m = s.max(axis=1, keepdims=True)
            w = np.exp(s - m)
            z = w.sum(axis=1, keepdims=True)
            O[qi, heads] = (w @ V) / z
            L[qi, heads] = (m + np.log(z))[:, 0]
    return O, L


def partial_attend(qrows, K, V, scale):
    """Attention of query rows [R, d] over one token set K, V [n, d], all float64.

    Returns the normalised partial output O [R, d], the row maximum m [R],
    the sum of exponentials s [R] (relative to m) and LSE = m + ln s: the
    state a partial attention computation hands to the merge (CoDec, section
    块内内核原语, PAC and POR; DEFT, section A.4, phase 1 returns the partial
    attention plus its LogSumExp).  An empty token set yields O = 0,
    m = -inf, s = 0, LSE = -inf (it must carry no weight in a merge).
    """
    qrows = np.asarray(qrows, dtype=np.float64)
    R = qrows.shape[0]
    if K.shape[0] == 0:
        return (np.zeros((R, V.shape[1])), np.full(R, -np.inf), np.zeros(R), np.full(R, -np.inf))
    s = scale * (qrows @ K.T)
    m = s.max(axis=1)
    w = np.exp(s - m[:, None])
    z = w.sum(axis=1)
    O = (w @ V) / z[:, None]
    return O, m, z, m + np.log(z)
