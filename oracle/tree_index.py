"""Tree index in canonical order (test infrastructure only).

CoDec (CoDec: Prefix-Shared Decoding Kernel for LLMs), section KV缓存管理:
the memory manager keeps, for every KV node, the set of queries that share
it (so a partial computation can gather them), and for every query the nodes
that make up its prefix (so its partial results can be found and merged).
DEFT (DEFT: Decoding with Flash Tree-Attention), section A.8, Algorithm 1,
names the same two maps QMapKV and KVMapQ.

Canonical form built here (the bit-exact target for the library):

* ``depth[i]``: nodes on the path from the virtual root to ``i`` (roots: 1);
* ``n_q[i]``: number of queries whose path contains ``i``;
* query -> node CSR ``qn_ptr``/``qn_idx``: each query's path, root first;
* node -> query CSR ``nq_ptr``/``nq_idx``: each node's queries, ascending id;
  ``nq_mask`` beside it: the query's 64-bit mask where the node is the
  query's own masked node, else all ones;
* ``visible[r]``: tokens query ``r`` sees.

Validation (raises :class:`TreeError` with the library's error name):
parents come before children; lengths >= 1; offsets >= 0; queries sit on
existing nodes; masked nodes hold at most 64 tokens; no mask bit at or above
the node length; every query sees at least one token.
"""
from __future__ import annotations

import numpy as np

ALL_ONES = np.uint64(0xFFFFFFFFFFFFFFFF)


class TreeError(ValueError):
    def __init__(self, code, msg):
        super().__init__(f"{code}: {msg}")
        self.code = code


def build_index(spec):
    parent = np.asarray(spec.parent, dtype=np.int64)
    kv_len = np.asarray(spec.kv_len, dtype=np.int64)
    kv_off = np.asarray(spec.kv_offset, dtype=np.int64)
    qnode = np.asarray(spec.query_node, dtype=np.int64)
    N, B = len(parent), len(qnode)
    masked = (np.zeros(N, dtype=bool) if spec.node_masked is None
              else np.asarray(spec.node_masked).astype(bool))
    qmask = spec.query_mask
    for i in range(N):
        if not (-1 <= parent[i] < i):
            raise TreeError("PST_E_INVALID_TREE", f"parent[{i}]={parent[i]} not in [-1, {i})")
        if kv_len[i] < 1:
            raise TreeError("PST_E_INVALID_TREE", f"kv_len[{i}]={kv_len[i]} < 1")
        if kv_off[i] < 0:
            raise TreeError("PST_E_INVALID_TREE", f"kv_offset[{i}] < 0")
        if masked[i] and kv_len[i] > 64:
            raise TreeError("PST_E_INVALID_TREE", f"masked node {i} longer than 64")
    depth = np.zeros(N, dtype=np.int64)
    for i in range(N):
        depth[i] = 1 if parent[i] == -1 else depth[parent[i]] + 1

    paths = []
    visible = np.zeros(B, dtype=np.int64)
    for r in range(B):
        n = int(qnode[r])
        if not (0 <= n < N):
            raise TreeError("PST_E_INVALID_TREE", f"query_node[{r}]={n} out of range")
        path = []
        t = n
        while t != -1:
            path.append(t)
            t = int(parent[t])
        path.reverse()
        paths.append(path)
        vis = int(sum(kv_len[p] for p in path[:-1]))
        if masked[n] and qmask is not None:
            bits = int(qmask[r])
            if bits >> int(kv_len[n]):
                raise TreeError("PST_E_INVALID_TREE", f"mask of query {r} has bits past node length")
            vis += bin(bits).count("1")
        else:
            vis += int(kv_len[n])
        if vis == 0:
            raise TreeError("PST_E_INVALID_TREE", f"query {r} sees no token")
        visible[r] = vis

    qn_ptr = np.zeros(B + 1, dtype=np.int32)
    for r in range(B):
        qn_ptr[r + 1] = qn_ptr[r] + len(paths[r])
    qn_idx = np.array([n for p in paths for n in p], dtype=np.int32)

    members = [[] for _ in range(N)]
    for r in range(B):  # ascending query id by construction
        for n in paths[r]:
            members[n].append(r)
    nq_ptr = np.zeros(N + 1, dtype=np.int32)
    for i in range(N):
        nq_ptr[i + 1] = nq_ptr[i] + len(members[i])
    nq_idx = np.array([r for m in members for r in m], dtype=np.int32)
    nq_mask = np.full(len(nq_idx), ALL_ONES, dtype=np.uint64)
    e = 0
    for i in range(N):
        for r in members[i]:
            if masked[i] and qmask is not None and int(qnode[r]) == i:
                nq_mask[e] = np.uint64(int(qmask[r]))
            e += 1
    n_q = np.diff(nq_ptr).astype(np.int32)
    return {
        "depth": depth.astype(np.int32),
        "n_q": n_q,
        "qn_ptr": qn_ptr,
        "qn_idx": qn_idx,
        "nq_ptr": nq_ptr,
        "nq_idx": nq_idx,
        "nq_mask": nq_mask,
        "visible": visible,
    }
