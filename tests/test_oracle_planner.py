"""Pins of the oracle's cost lookup and task partitioner (CPU only).

The pages leave the partitioner's exact steps open, so its quality is parity
unpinned; its structure is pinned here by:
* closed forms of the integer lookup on an affine table;
* tiling invariants (pieces and row groups cover every node exactly once,
  every (query, path node) owns exactly b_eff consecutive slots, bin loads
  add up);
* the IO identities of CoDec's complexity analysis (KV-guided: every node's
  KV once; query-guided: once per query);
* Graham's bound for LPT list scheduling (makespan <= (4/3 - 1/(3m)) OPT)
  against the brute-force optimum of tiny instances;
* the binary search for cost_l against a linear scan.
"""
import itertools

import numpy as np
import pytest

import oracle
import workloads
from oracle.planner import _lpt

ROWS = [1, 2, 4, 8, 16, 32, 64, 128, 256]
LENS = [16 << i for i in range(13)]


def affine_table(a=900, b=3, c=2):
    return oracle.CostTable(ROWS, LENS, [[a + b * r + c * L for L in LENS] for r in ROWS])


def random_table(seed):
    rng = np.random.default_rng(seed)
    t = np.cumsum(np.cumsum(rng.integers(1, 50, size=(len(ROWS), len(LENS))), axis=0), axis=1) + 500
    return oracle.CostTable(ROWS, LENS, t)


def test_affine_lookup_closed_form():
    t = affine_table()
    for rows in [1, 3, 4, 5, 17, 255, 256]:
        rg = next(x for x in ROWS if x >= rows)
        for L in [1, 16, 17, 100, 1000, 4000, 32768, 40000, 65536, 70000, 200000]:
            assert t.lookup(rows, L) == 900 + 3 * rg + 2 * max(L, 16)


def test_table_validation():
    with pytest.raises(ValueError):
        oracle.CostTable(ROWS, LENS, [[5] * 13] * 8)
    bad = [[900 + L for L in LENS] for _ in ROWS]
    bad[3][4] = 1
    with pytest.raises(ValueError):
        oracle.CostTable(ROWS, LENS, bad)


def _check_plan(spec, ix, p, table, m, g, r_max):
    tasks = p["tasks"]
    kv_len = spec.kv_len
    n_q = ix["n_q"]
    # Pieces and row groups tile each node exactly once.
    cover = {}
    for node, piece, kb, kn, rb, rc, flags in tasks:
        cover.setdefault(node, []).append((kb, kn, rb, rc))
        assert kn >= 1 and rc >= 1 and rc <= max(r_max, 1)
        assert kb == piece * p["piece_len"][node]
        assert bool(flags & 1) == (piece == p["b_eff"][node] - 1)
    for i in range(spec.num_nodes):
        if n_q[i] == 0:
            assert i not in cover
            continue
        grid = np.zeros((int(n_q[i]) * g, int(kv_len[i])), dtype=np.int32)
        for kb, kn, rb, rc in cover[i]:
            grid[rb:rb + rc, kb:kb + kn] += 1
        assert (grid == 1).all()
        assert p["b_eff"][i] == -(-int(kv_len[i]) // int(p["piece_len"][i]))
    # Bins: loads add up to the cost of their tasks.
    bp = p["bin_ptr"]
    assert bp[0] == 0 and bp[-1] == len(tasks) and len(bp) == m + 1
    for b in range(m):
        load = sum(table.lookup(int(t[5]), int(t[3])) for t in tasks[bp[b]:bp[b + 1]])
        assert load == p["bin_load"][b]
    assert p["makespan"] == max(p["bin_load"])
    # Slots: each (query, path node) owns b_eff consecutive slots, in path order.
    sp = p["slot_ptr"]
    for r in range(spec.num_queries):
        path = ix["qn_idx"][ix["qn_ptr"][r]:ix["qn_ptr"][r + 1]]
        assert sp[r + 1] - sp[r] == sum(int(p["b_eff"][i]) for i in path)
        off = sp[r]
        for i in path:
            ents = range(ix["nq_ptr"][i], ix["nq_ptr"][i + 1])
            e = next(e for e in ents if ix["nq_idx"][e] == r)
            assert p["entry_slot"][e] == off
            off += p["b_eff"][i]


@pytest.mark.parametrize("seed", range(12))
@pytest.mark.parametrize("m", [1, 3, 16])
def test_plan_invariants_random(seed, m):
    spec = workloads.random_tree(seed, max_nodes=8, max_len=700, max_queries=12, num_q_heads=8, num_kv_heads=2)
    ix = oracle.build_index(spec)
    table = random_table(seed) if seed % 2 else affine_table()
    r_max = [256, 16, 8][seed % 3]
    p = oracle.plan(ix, spec.kv_len, spec.group, table, m, r_max=r_max)
    _check_plan(spec, ix, p, table, m, spec.group, r_max)
    if m == 1:
        assert p["bin_ptr"][1] == len(p["tasks"])


@pytest.mark.parametrize("name", ["1", "2", "3", "4"])
def test_plan_invariants_configs(name):
    spec = workloads.config(name)
    ix = oracle.build_index(spec)
    table = affine_table()
    r_max = 16 if spec.dtype == "f32" else 256
    p = oracle.plan(ix, spec.kv_len, spec.group, table, 32, r_max=r_max)
    _check_plan(spec, ix, p, table, 32, spec.group, r_max)


def test_kv_guided_reads_each_node_once_query_guided_once_per_query():
    spec = workloads.config("3")
    ix = oracle.build_index(spec)
    t = affine_table()
    kvg = oracle.plan(ix, spec.kv_len, spec.group, t, 64, r_max=512)
    qg = oracle.plan(ix, spec.kv_len, spec.group, t, 64, query_guided=True)
    read = lambda p: int(p["tasks"][:, 3].astype(np.int64).sum())
    assert read(kvg) == int(spec.kv_len.sum())
    assert read(qg) == int((ix["n_q"].astype(np.int64) * spec.kv_len).sum())
    assert (qg["tasks"][:, 5] == spec.group).all()


def test_equal_tasks_one_per_bin():
    spec = workloads.TreeSpec("eq", np.full(6, -1), np.full(6, 64), np.arange(6) * 64, np.arange(6), 4, 4, 64, "f32", 0)
    ix = oracle.build_index(spec)
    p = oracle.plan(ix, spec.kv_len, 1, affine_table(), 8)
    counts = np.diff(p["bin_ptr"])
    assert sorted(counts.tolist()) == [0, 0, 1, 1, 1, 1, 1, 1]


def _opt_makespan(costs, m):
    best = None
    for assign in itertools.product(range(m), repeat=len(costs)):
        if assign and assign[0] != 0:
            continue  # symmetry
        loads = [0] * m
        for c, b in zip(costs, assign):
            loads[b] += c
        best = max(loads) if best is None else min(best, max(loads))
    return best


@pytest.mark.parametrize("seed", range(40))
def test_lpt_graham_bound(seed):
    rng = np.random.default_rng(seed)
    m = int(rng.integers(2, 4))
    n = int(rng.integers(m + 1, 8))
    costs = [int(c) for c in rng.integers(1, 100, size=n)]
    items = [(c, i, 0, 0) for i, c in enumerate(costs)]
    _, loads = _lpt(items, m)
    opt = _opt_makespan(costs, m)
    assert max(loads) * 3 * m <= (4 * m - 1) * opt
    assert sum(loads) == sum(costs)


@pytest.mark.parametrize("seed", range(6))
def test_cost_l_is_first_feasible_bound(seed):
    """With an affine table W(T) is non-increasing, so the binary search must
    land on the smallest T with m T >= W(T); checked by scanning every T."""
    from oracle.planner import _Node, _b_of_T, _cost_with_lp, _geom

    spec = workloads.random_tree(100 + seed, max_nodes=5, max_len=900, max_queries=6, num_q_heads=4, num_kv_heads=4)
    ix = oracle.build_index(spec)
    t = affine_table(a=300, b=1, c=1)
    m = 7
    p = oracle.plan(ix, spec.kv_len, 1, t, m)
    nodes = []
    for i in range(spec.num_nodes):
        if ix["n_q"][i] == 0:
            continue
        nd = _Node()
        nd.i, nd.n, nd.rows = i, int(spec.kv_len[i]), int(ix["n_q"][i])
        nd.gq, nd.rpg, nd.last_rows, nd.bmax = 1, nd.rows, nd.rows, -(-nd.n // 64)
        nodes.append(nd)
    W = lambda T: sum(_cost_with_lp(t, nd, _geom(nd.n, _b_of_T(t, nd, T, 64), 64)[0]) for nd in nodes)
    lo = max(t.lookup(nd.rpg, min(nd.n, 64)) for nd in nodes)
    T = lo
    while m * T < W(T):
        T += 1
    assert p["cost_l"] == T
