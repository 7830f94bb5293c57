"""Task partitioner for the partial-attention launch (test infrastructure only).

Source: CoDec (CoDec: Prefix-Shared Decoding Kernel for LLMs), section
工作负载平衡 (workload balance) and the min-max objective in section 速读.
Each KV node i is a task T[i] = (n_q[i], n[i]); it may be cut along the query
axis (b_q) and the KV axis (b_k); an assignment A of the pieces to m blocks
minimises the largest block cost  max_i sum_j C[j] A[i, j].  The heuristic
takes b_q = 1 (query rows stay together so the KV is read once), finds a
lower bound cost_l of the per-block cost by binary search from two facts
(the pieces of a task cost at least the task; the largest block costs at
least the average), bounds b_k[i] <= ceil(C_est(n_q[i], n[i]) / cost_l), and
grid-searches the split per node.  The assignment step is list scheduling
(Graham, "Bounds for certain multiprocessing anomalies", 1966, cited there);
the longest-processing-time order is used.

The pages fix no constants, tie-breaks or piece geometry.  This is the
reading taken here, implemented identically in the library, all in integers:

1. rows r_i = n_q[i] * g (queries x GQA group).  If r_i > R_max the rows are
   cut into gq_i = ceil(r_i / R_max) row groups of ceil(r_i / gq_i) rows (the
   last one shorter): one block only holds R_max rows (this departs from
   b_q = 1 only where a node has more rows than a block holds).  The
   query-guided (FlashDecoding-style) baseline is the same procedure with
   R_max = g: one query per group, so shared KV is read once per query.
2. piece geometry for b pieces: Lp = roundup(ceil(n/b), G), b_eff = ceil(n/Lp),
   piece k = [k Lp, min((k+1) Lp, n)); bmax = ceil(n/G).
3. cost(i, b) = sum over row groups and pieces of C(rows, piece length).
4. b_i(T) = the smallest b in [1, bmax] whose longest piece of the largest
   row group costs <= T, else bmax.  W(T) = sum_i min over b in
   [b_i(T), bmax_i] of cost(i, b): the least total cost of any splits whose
   pieces all cost <= T (every b >= b_i(T) qualifies, the piece length
   shrinking with b).  A makespan of T needs m T >= W(T) (the largest block
   costs at least the average), so the smallest such T is the section's
   lower bound cost_l; W is non-increasing in T, so the binary search finds
   it.  (cost(i, b) is not monotone in b under every table: taking
   cost(i, b_i(T)) alone made W jump up with T and the search miss the
   smallest T.)
5. cost_l = smallest T in [lo, hi] with m T >= W(T) by binary search, with
   lo = max_i C(rows_i, min(n_i, G)) and hi = sum_i cost(i, 1).
6. ub_i = min(bmax_i, max(1, ceil(C(rows_i, n_i) / cost_l))).
7. grid search k = 0..K: T_k = cost_l + (cost_l k) // K, b_i = min(ub_i, b_i(T_k));
   7b (an addition to the pages' procedure): one candidate per uniform piece length
   U = G x 1, 2, 3, 4, 6, 8, 12, 16, ... (every node cut into pieces of U,
   the last shorter), up to the first U that holds the longest node, as
   k = K+1, K+2, ...; for every candidate the pieces (per row group) are
   sorted by (cost desc, node, row group, piece) and each goes to the block
   with the smallest (load, block id).
8. keep the k with the smallest makespan; ties: fewer pieces, then smaller k.
9. tasks are emitted block by block in assignment order.  The partial slot
   of (query r, node i, piece p) is slot_ptr[r] + (pieces of the nodes before
   i on r's path) + p.
"""
from __future__ import annotations

import heapq

import numpy as np

FLAG_LAST_PIECE = 1


def _ceil(a, b):
    return -(-a // b)


class _Node:
    __slots__ = ("i", "n", "rows", "gq", "rpg", "last_rows", "bmax")


def _geom(n, b, G):
    Lp = _ceil(_ceil(n, b), G) * G
    return Lp, _ceil(n, Lp)


def _cost_with_lp(table, nd, Lp):
    beff = _ceil(nd.n, Lp)
    last_len = nd.n - (beff - 1) * Lp
    full_groups = nd.gq - 1
    c = 0
    for rows, count in ((nd.rpg, full_groups), (nd.last_rows, 1)):
        if count == 0:
            continue
        c += count * ((beff - 1) * table.lookup(rows, Lp) + table.lookup(rows, last_len))
    return c


def _b_of_T(table, nd, T, G):
    def f(b):
        Lp, _ = _geom(nd.n, b, G)
        return table.lookup(nd.rpg, min(Lp, nd.n))

    if f(nd.bmax) > T:
        return nd.bmax
    lo, hi = 1, nd.bmax
    while lo < hi:
        mid = (lo + hi) // 2
        if f(mid) <= T:
            hi = mid
        else:
            lo = mid + 1
    return lo


def _lpt(items, m):
    """items: list of (cost, node, group, piece).  Returns per-bin lists and loads."""
    items = sorted(items, key=lambda t: (-t[0], t[1], t[2], t[3]))
    heap = [(0, b) for b in range(m)]
    bins = [[] for _ in range(m)]
    for it in items:
        load, b = heapq.heappop(heap)
        bins[b].append(it)
        heapq.heappush(heap, (load + it[0], b))
    loads = [0] * m
    for load, b in heap:
        loads[b] = load
    return bins, loads


def plan(index, kv_len, g, table, m, *, r_max=256, tile=64, grid_steps=8,
         query_guided=False, no_split=False, fixed_chunk=0):
    """Plan for one tree.  ``index`` is :func:`oracle.tree_index.build_index` output."""
    if m < 1:
        raise ValueError("m >= 1")
    G = int(tile)
    if query_guided:
        r_max = g
    n_q = np.asarray(index["n_q"], dtype=np.int64)
    kv_len = np.asarray(kv_len, dtype=np.int64)
    N = len(kv_len)
    nodes = []
    for i in range(N):
        if n_q[i] == 0:
            continue
        nd = _Node()
        nd.i = i
        nd.n = int(kv_len[i])
        nd.rows = int(n_q[i]) * g
        nd.gq = _ceil(nd.rows, r_max)
        nd.rpg = _ceil(nd.rows, nd.gq)
        nd.last_rows = nd.rows - (nd.gq - 1) * nd.rpg
        nd.bmax = _ceil(nd.n, G)
        nodes.append(nd)

    # Piece length per node for a given choice of b (or a fixed geometry).
    def lp_for(nd, b):
        return _geom(nd.n, b, G)[0]

    info = {"cost_l": 0, "chosen_k": 0, "ub": {}}
    if not nodes:
        candidates = []
    elif no_split or fixed_chunk > 0:
        lps = {}
        for nd in nodes:
            lps[nd.i] = fixed_chunk if fixed_chunk > 0 else lp_for(nd, 1)
        candidates = [lps]
    else:
        # Per node, the least cost over splits into b or more pieces:
        # least[nd.i][b] = min over b' in [b, bmax] of cost(i, b').
        least = {}
        for nd in nodes:
            suf = [0] * (nd.bmax + 2)
            suf[nd.bmax + 1] = None
            for b in range(nd.bmax, 0, -1):
                c = _cost_with_lp(table, nd, lp_for(nd, b))
                suf[b] = c if suf[b + 1] is None else min(c, suf[b + 1])
            least[nd.i] = suf

        def W(T):
            return sum(least[nd.i][_b_of_T(table, nd, T, G)] for nd in nodes)

        lo = max(table.lookup(nd.rpg, min(nd.n, G)) for nd in nodes)
        hi = sum(_cost_with_lp(table, nd, lp_for(nd, 1)) for nd in nodes)
        while lo < hi:
            mid = lo + (hi - lo) // 2
            if m * mid >= W(mid):
                hi = mid
            else:
                lo = mid + 1
        cost_l = lo
        info["cost_l"] = cost_l
        ub = {}
        for nd in nodes:
            ub[nd.i] = min(nd.bmax, max(1, _ceil(table.lookup(nd.rpg, nd.n), cost_l)))
        info["ub"] = ub
        candidates = []
        for k in range(grid_steps + 1):
            T = cost_l + (cost_l * k) // grid_steps
            lps = {}
            for nd in nodes:
                b = min(ub[nd.i], _b_of_T(table, nd, T, G))
                lps[nd.i] = lp_for(nd, b)
            candidates.append(lps)
        # Step 7b: one piece length U for every node, U = G x 1, 2, 3, 4, 6,
        # 8, 12, ... up to the first U that holds the longest node.
        nmax = max(nd.n for nd in nodes)
        factors = []
        p = 1
        while True:
            factors.append(2 * p)  # in halves of G: U = G * f / 2
            if G * p >= nmax:
                break
            if p >= 2:
                factors.append(3 * p)
                if G * p * 3 // 2 >= nmax:
                    break
            p *= 2
        for f in factors:
            u = G * f // 2
            candidates.append({nd.i: u for nd in nodes})

    best = None
    if nodes:
        for k, lps in enumerate(candidates):
            items = []
            for nd in nodes:
                Lp = lps[nd.i]
                beff = _ceil(nd.n, Lp)
                for gidx in range(nd.gq):
                    rows = nd.rpg if gidx < nd.gq - 1 else nd.last_rows
                    for p in range(beff):
                        plen = min(Lp, nd.n - p * Lp)
                        items.append((table.lookup(rows, plen), nd.i, gidx, p))
            bins, loads = _lpt(items, m)
            key = (max(loads), len(items), k)
            if best is None or key < best[0]:
                best = (key, lps, bins, loads, k)
        _, lps, bins, loads, chosen_k = best
        info["chosen_k"] = chosen_k
    else:
        lps, bins, loads = {}, [[] for _ in range(m)], [0] * m

    by_id = {nd.i: nd for nd in nodes}
    piece_len = np.zeros(N, dtype=np.int32)
    b_eff = np.zeros(N, dtype=np.int32)
    rpg = np.zeros(N, dtype=np.int32)
    for nd in nodes:
        piece_len[nd.i] = lps[nd.i]
        b_eff[nd.i] = _ceil(nd.n, lps[nd.i])
        rpg[nd.i] = nd.rpg

    tasks = []
    bin_ptr = np.zeros(m + 1, dtype=np.int32)
    for b in range(m):
        for cost, i, gidx, p in bins[b]:
            nd = by_id[i]
            Lp = int(piece_len[i])
            kv_begin = p * Lp
            kv_n = min(Lp, nd.n - kv_begin)
            row_begin = gidx * nd.rpg
            row_count = min(nd.rpg, nd.rows - row_begin)
            flags = FLAG_LAST_PIECE if p == b_eff[i] - 1 else 0
            tasks.append((i, p, kv_begin, kv_n, row_begin, row_count, flags))
        bin_ptr[b + 1] = len(tasks)

    qn_ptr, qn_idx = index["qn_ptr"], index["qn_idx"]
    nq_ptr = index["nq_ptr"]
    B = len(qn_ptr) - 1
    slot_ptr = np.zeros(B + 1, dtype=np.int64)
    entry_slot = np.zeros(int(nq_ptr[-1]), dtype=np.int64)
    cursor = np.array(nq_ptr[:-1], dtype=np.int64).copy()
    for r in range(B):
        off = int(slot_ptr[r])
        for t in range(int(qn_ptr[r]), int(qn_ptr[r + 1])):
            i = int(qn_idx[t])
            entry_slot[cursor[i]] = off
            cursor[i] += 1
            off += int(b_eff[i])
        slot_ptr[r + 1] = off

    return {
        "tasks": np.array(tasks, dtype=np.int32).reshape(-1, 7),
        "bin_ptr": bin_ptr,
        "slot_ptr": slot_ptr,
        "entry_slot": entry_slot,
        "piece_len": piece_len,
        "b_eff": b_eff,
        "rows_per_group": rpg,
        "bin_load": np.array(loads, dtype=np.int64),
        "makespan": int(max(loads)) if loads else 0,
        "cost_l": int(info["cost_l"]),
        "chosen_k": int(info["chosen_k"]),
        "num_slots": int(slot_ptr[-1]),
    }
