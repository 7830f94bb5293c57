"""The planner oracle against a brute force written from the reading alone.

CoDec (CoDec: Prefix-Shared Decoding Kernel for LLMs), section 工作负载平衡:
cost_l is found by binary search from "the pieces of a task cost at least
the task" and "the largest block costs at least the average"; every node's
split is capped by ceil(C_est(n_q, n) / cost_l); the splits are grid
searched and the pieces placed on the blocks.  The pages leave the details
open; the planner takes the reading stated in ``oracle/planner.py`` and
``include/pst.h`` (rows in row groups of at most R_max, pieces of
roundup(ceil(n / b), G) tokens, b(T) the smallest split whose longest piece
of the largest row group costs at most T, cost_l the smallest T with
m T >= W(T), K + 1 threshold candidates plus one candidate per uniform piece
length, LPT placement, the candidate with the smallest (makespan, pieces,
k)).

Nothing here comes from ``oracle.planner`` or ``oracle.cost``: the cost
lookup, the piece lists, b(T), W(T), cost_l, the caps, the candidates, the
placement and the choice are written out again, the slow way (linear scans,
explicit piece lists, the exact smallest feasible T over every breakpoint of
W), on trees small enough for that: at most 4 nodes, 600 tokens per node,
4 bins.  ``oracle.plan`` must give the same plan, task for task.
"""
import math

import numpy as np
import pytest

import oracle

ROWS = [1, 2, 4, 8, 16, 32, 64, 128, 256]
LENS = [16 << i for i in range(13)]
G = 64


def lookup(table, rows, length):
    """C(rows, len): rows -> the first grid point >= rows (the last beyond the
    grid); len -> the first column below the grid, the straight line through
    the two grid points around it (floor), the line through the last two
    points beyond the grid."""
    ri = next((i for i, r in enumerate(ROWS) if r >= rows), len(ROWS) - 1)
    row = table[ri]
    if length <= LENS[0]:
        return row[0]
    if length >= LENS[-1]:
        x0, x1, y0, y1 = LENS[-2], LENS[-1], row[-2], row[-1]
    else:
        j = max(i for i, L in enumerate(LENS) if L <= length)
        x0, x1, y0, y1 = LENS[j], LENS[j + 1], row[j], row[j + 1]
    return y0 + (y1 - y0) * (length - x0) // (x1 - x0)


def row_groups(rows, r_max):
    """Row counts of the groups of a node with `rows` rows."""
    gq = -(-rows // r_max)
    per = -(-rows // gq)
    return [min(per, rows - k * per) for k in range(gq)]


def pieces(n, b):
    """Piece lengths of a node of n tokens cut in b: every piece Lp =
    roundup(ceil(n / b), G) tokens, the last one what is left."""
    Lp = -(-(-(-n // b)) // G) * G
    out, start = [], 0
    while start < n:
        out.append(min(Lp, n - start))
        start += Lp
    return Lp, out


def node_cost(table, groups, lens):
    return sum(lookup(table, r, L) for r in groups for L in lens)


def b_of(table, n, groups, T):
    """Linear scan: the smallest b in 1..bmax whose longest piece, with the
    rows of the largest row group, costs at most T; bmax if none does."""
    bmax = -(-n // G)
    for b in range(1, bmax + 1):
        _, lens = pieces(n, b)
        if lookup(table, max(groups), max(lens)) <= T:
            return b
    return bmax


def brute_plan(parent, kv_len, query_node, g, table, m, r_max=256, K=8):
    N = len(kv_len)
    n_q = [0] * N
    for qn in query_node:
        n = int(qn)
        while n >= 0:
            n_q[n] += 1
            n = int(parent[n])
    nodes = [i for i in range(N) if n_q[i] > 0]
    groups = {i: row_groups(n_q[i] * g, r_max) for i in nodes}
    n = {i: int(kv_len[i]) for i in nodes}

    def W(T):
        """The least total cost of splits whose pieces, with the rows of
        the largest row group, all cost <= T: every b from b(T) up."""
        total = 0
        for i in nodes:
            bmax = -(-n[i] // G)
            total += min(node_cost(table, groups[i], pieces(n[i], b)[1]) for b in range(b_of(table, n[i], groups[i], T),
                                                                                      bmax + 1))
        return total

    lo = max(lookup(table, max(groups[i]), min(n[i], G)) for i in nodes)
    hi = sum(node_cost(table, groups[i], [n[i]]) for i in nodes)
    # W is constant between consecutive values C(largest group, longest piece
    # of some split): check each such stretch for its smallest T with m T >= W.
    breaks = sorted({lo, hi} | {lookup(table, max(groups[i]), max(pieces(n[i], b)[1]))
                                for i in nodes for b in range(1, -(-n[i] // G) + 1)})
    breaks = [t for t in breaks if lo <= t <= hi]
    cost_l = None
    for a, nxt in zip(breaks, breaks[1:] + [hi + 1]):
        w = W(a)
        t = max(a, -(-w // m))
        if t < nxt:
            cost_l = t
            break
    assert cost_l is not None
    ub = {i: min(-(-n[i] // G), max(1, -(-lookup(table, max(groups[i]), n[i]) // cost_l))) for i in nodes}
    cands = []
    for k in range(K + 1):
        T = cost_l + cost_l * k // K
        cands.append({i: pieces(n[i], min(ub[i], b_of(table, n[i], groups[i], T)))[0] for i in nodes})
    longest = max(n.values())
    # Uniform piece lengths G x {1, 2, 3, 4, 6, 8, 12, 16, ...} (the powers of
    # two, and 1.5 times each from 2 on), up to the first that holds the
    # longest node.
    us = []
    p = 1
    while True:
        us.append(G * p)
        if G * p >= longest:
            break
        if p >= 2:
            us.append(G * p * 3 // 2)
            if G * p * 3 // 2 >= longest:
                break
        p *= 2
    cands += [{i: u for i in nodes} for u in us]
    best = None
    for k, lps in enumerate(cands):
        items = []
        for i in nodes:
            lens = []
            start = 0
            while start < n[i]:
                lens.append(min(lps[i], n[i] - start))
                start += lps[i]
            for gi, rows in enumerate(groups[i]):
                for pi, L in enumerate(lens):
                    items.append((lookup(table, rows, L), i, gi, pi))
        items.sort(key=lambda it: (-it[0], it[1], it[2], it[3]))
        load = [0] * m
        placed = [[] for _ in range(m)]
        for it in items:
            b = min(range(m), key=lambda x: (load[x], x))
            placed[b].append(it)
            load[b] += it[0]
        key = (max(load), len(items), k)
        if best is None or key < best[0]:
            best = (key, k, lps, placed, load)
    (span, count, _), k, lps, placed, load = best
    tasks = []
    for b in range(m):
        for cost, i, gi, pi in placed[b]:
            beff = -(-n[i] // lps[i])
            start = pi * lps[i]
            per = groups[i][0]
            tasks.append((i, pi, start, min(lps[i], n[i] - start), gi * per, groups[i][gi],
                          1 if pi == beff - 1 else 0))
    return {"tasks": tasks, "cost_l": cost_l, "chosen_k": k, "makespan": span, "bin_load": load,
            "ub": ub, "num_pieces": count}


def random_table(rng, jumpy):
    """A valid table (>= 1, non-decreasing along both axes); `jumpy` tables
    have rare large steps, so piece costs are far from affine."""
    if jumpy:
        inc = rng.integers(0, 30, size=(9, 13)) + (rng.random((9, 13)) < 0.2) * rng.integers(0, 3000, size=(9, 13))
    else:
        inc = rng.integers(1, 60, size=(9, 13))
    return (np.cumsum(np.cumsum(inc, axis=0), axis=1) + rng.integers(1, 500)).tolist()


def random_case(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 5))
    parent = [-1] + [int(rng.integers(-1, i)) for i in range(1, N)]
    kv_len = [int(rng.integers(1, 601)) for _ in range(N)]
    B = int(rng.integers(1, 7))
    query_node = [int(rng.integers(0, N)) for _ in range(B)]
    g = int(rng.choice([1, 2, 8, 32, 64]))
    m = int(rng.integers(1, 5))
    r_max = int(rng.choice([256, 64, 16]))
    return parent, kv_len, query_node, g, m, r_max, random_table(rng, jumpy=seed % 2 == 1)


def _spec(parent, kv_len, query_node, g):
    import workloads

    off = np.concatenate([[0], np.cumsum(kv_len)[:-1]])
    return workloads.TreeSpec("bf", np.array(parent), np.array(kv_len), off, np.array(query_node), g, 1, 128,
                              "bf16", 0)


@pytest.mark.parametrize("seed", range(400))
def test_planner_matches_brute_force(seed):
    parent, kv_len, query_node, g, m, r_max, table = random_case(seed)
    if g > r_max:
        r_max = 256
    want = brute_plan(parent, kv_len, query_node, g, table, m, r_max=r_max)
    spec = _spec(parent, kv_len, query_node, g)
    got = oracle.plan(oracle.build_index(spec), spec.kv_len, g, oracle.CostTable(ROWS, LENS, table), m,
                      r_max=r_max)
    assert got["cost_l"] == want["cost_l"]
    assert got["chosen_k"] == want["chosen_k"]
    assert got["makespan"] == want["makespan"]
    assert got["bin_load"].tolist() == want["bin_load"]
    assert [tuple(int(x) for x in t) for t in got["tasks"]] == want["tasks"]


def test_brute_force_pieces_and_groups():
    """The brute force's own building blocks on hand-checked values."""
    assert pieces(600, 1) == (640, [600])
    assert pieces(600, 2) == (320, [320, 280])
    assert pieces(600, 3) == (256, [256, 256, 88])
    assert pieces(600, 10) == (64, [64] * 9 + [24])
    assert pieces(65, 2) == (64, [64, 1])
    assert row_groups(256, 256) == [256]
    assert row_groups(257, 256) == [129, 128]
    assert row_groups(512, 256) == [256, 256]
    assert row_groups(40, 16) == [14, 14, 12]
    t = [[10 * (r + 1) + L for L in range(13)] for r in range(9)]
    assert lookup(t, 1, 16) == 10 and lookup(t, 3, 16) == 30 and lookup(t, 300, 16) == 90
    assert lookup(t, 1, 24) == 10 + (11 - 10) * 8 // 16
    assert lookup(t, 1, 65536 + 65536) == 22 + (22 - 21) * 65536 // 32768
