"""Flattened tree KV splitting (test infrastructure only).

Source: DEFT (DEFT: Decoding with Flash Tree-Attention), section 3.3 (tree
KV splitting and load balance, remark 3.1, Fig. 3(c)) and appendix A.9
(DEFT-Flatten, phase 1).  The tree's KV is laid out in depth-first order as
one logical sequence (no data moves) and cut into chunks of equal token
count, at most S_t each; each chunk is grouped with every query that shares
any of its KV, and a 64-bit bit causal mask per (query, 64 tokens) records
which tokens of the chunk the query sees.  Phase 2 is the partial attention
of every group under its mask, then the same per-query reduction as for
node-grouped partials.

The pages fix neither the traversal order among siblings, nor how groups go
to processors, nor the mask's word layout.  The reading implemented here,
identically in the library:

1. depth-first pre-order from the roots in increasing node id, children in
   increasing node id; nodes that no query sees are left out;
2. chunk c = flattened tokens [c S_t, (c+1) S_t) (the last one shorter);
   S_t is a multiple of 128 tokens;
3. the group of chunk c: the queries that see at least one of its tokens,
   in increasing query id (one "entry" each);
4. the mask of an entry: W = S_t / 64 words; bit j of word w is set when
   the query sees token 64 w + j of the chunk (a token of a node on its
   path, and for its own masked node the query's mask bit); bits past the
   chunk's end are clear;
5. row groups of whole entries, at most E_max = min(floor(R_max / g),
   floor(1024 / W)) entries each (rows = entries x GQA group; the masks of
   one row group fit 8 KB): gq = ceil(entries / E_max) groups of
   ceil(entries / gq) entries, the last one shorter;
6. the groups go to m blocks by longest-processing-time list scheduling on
   the cost table C(rows, chunk tokens), sorted by (cost desc, chunk, row
   group), each to the block with the smallest (load, block id);
7. query r's partial slots: one per chunk in its groups, in chunk order,
   from slot_ptr[r];
8. token rows: the pool row of every chunk token (contiguous: offset + j;
   paged: page_idx[page_ptr[i] + j // P] * P + j % P), -1 past the end.
"""
from __future__ import annotations

import numpy as np

from .planner import _ceil, _lpt

FLAG_FLAT = 2


def dfs_order(parent, n_q):
    """Step 1: nodes in depth-first pre-order (roots and children by id)."""
    parent = np.asarray(parent, dtype=np.int64)
    N = len(parent)
    children = [[] for _ in range(N)]
    roots = []
    for i in range(N):
        (roots if parent[i] < 0 else children[int(parent[i])]).append(i)
    order = []
    stack = list(reversed(roots))
    while stack:
        i = stack.pop()
        if n_q[i] == 0:
            continue
        order.append(i)
        stack.extend(reversed(children[i]))
    return order


def token_row(i, j, kv_offset=None, page_size=0, page_ptr=None, page_idx=None):
    """Step 8: pool row of token j of node i."""
    if page_size:
        return int(page_idx[int(page_ptr[i]) + j // page_size]) * page_size + j % page_size
    return int(kv_offset[i]) + j


def flatten_plan(index, parent, kv_len, node_masked, g, table, m, *, chunk=256, r_max=256, kv_offset=None,
                 page_size=0, page_ptr=None, page_idx=None):
    if chunk <= 0 or chunk % 128:
        raise ValueError("chunk must be a positive multiple of 128")
    kv_len = np.asarray(kv_len, dtype=np.int64)
    N = len(kv_len)
    masked = np.zeros(N, dtype=bool) if node_masked is None else np.asarray(node_masked).astype(bool)
    nq_ptr, nq_idx, nq_mask = index["nq_ptr"], index["nq_idx"], index["nq_mask"]
    B = len(index["qn_ptr"]) - 1
    W = chunk // 64
    e_max = min(r_max // g, 1024 // W)
    if e_max < 1:
        raise ValueError("the GQA group does not fit one row group")

    order = dfs_order(parent, index["n_q"])
    flat = [(i, j) for i in order for j in range(int(kv_len[i]))]
    nchunks = _ceil(len(flat), chunk)

    rows = np.full(nchunks * chunk, -1, dtype=np.int32)
    for t, (i, j) in enumerate(flat):
        rows[t] = token_row(i, j, kv_offset, page_size, page_ptr, page_idx)

    flat_ptr = np.zeros(nchunks + 1, dtype=np.int32)
    flat_query, flat_mask = [], []
    chunk_len = []
    for c in range(nchunks):
        toks = flat[c * chunk:(c + 1) * chunk]
        chunk_len.append(len(toks))
        words = {}  # query -> W mask words (Python ints)
        for t, (i, j) in enumerate(toks):
            for e in range(int(nq_ptr[i]), int(nq_ptr[i + 1])):
                r = int(nq_idx[e])
                if masked[i] and not (int(nq_mask[e]) >> j) & 1:
                    continue
                w = words.setdefault(r, [0] * W)
                w[t // 64] |= 1 << (t % 64)
        for r in sorted(words):
            flat_query.append(r)
            flat_mask.extend(words[r])
        flat_ptr[c + 1] = len(flat_query)

    items = []
    groups = {}
    for c in range(nchunks):
        ne = int(flat_ptr[c + 1] - flat_ptr[c])
        gq = _ceil(ne, e_max)
        epg = _ceil(ne, gq)
        groups[c] = epg
        for k in range(gq):
            n_ent = min(epg, ne - k * epg)
            items.append((table.lookup(n_ent * g, chunk_len[c]), c, k, 0))
    bins, loads = _lpt(items, m)

    tasks = []
    bin_ptr = np.zeros(m + 1, dtype=np.int32)
    for b in range(m):
        for cost, c, k, _ in bins[b]:
            ne = int(flat_ptr[c + 1] - flat_ptr[c])
            epg = groups[c]
            n_ent = min(epg, ne - k * epg)
            tasks.append((c, 0, c * chunk, chunk_len[c], k * epg * g, n_ent * g, FLAG_FLAT))
        bin_ptr[b + 1] = len(tasks)

    # Step 7: slots per query in chunk order.
    count = np.zeros(B, dtype=np.int64)
    for r in flat_query:
        count[r] += 1
    slot_ptr = np.zeros(B + 1, dtype=np.int64)
    slot_ptr[1:] = np.cumsum(count)
    cursor = slot_ptr[:-1].copy()
    flat_slot = np.zeros(len(flat_query), dtype=np.int64)
    for e, r in enumerate(flat_query):  # entries are in chunk order
        flat_slot[e] = cursor[r]
        cursor[r] += 1

    return {
        "tasks": np.array(tasks, dtype=np.int32).reshape(-1, 7),
        "bin_ptr": bin_ptr,
        "slot_ptr": slot_ptr,
        "bin_load": np.array(loads, dtype=np.int64),
        "makespan": int(max(loads)) if loads else 0,
        "num_slots": int(slot_ptr[-1]),
        "chunk": chunk,
        "flat_ptr": flat_ptr,
        "flat_query": np.array(flat_query, dtype=np.int32),
        "flat_mask": np.array(flat_mask, dtype=np.uint64),
        "flat_slot": flat_slot,
        "flat_rows": rows,
    }
