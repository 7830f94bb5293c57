"""Property-based checks on random tiny trees (hypothesis; CPU only).

Trees are drawn directly (parents before children, lengths, queries, masked
nodes with non-empty masks), so the shapes include single nodes, long
chains, many queries on one node and 64-token masked nodes.  Properties:
* the library's index equals the oracle's, bit for bit;
* the library's cost-model plan and its flattened plan equal the oracle's;
* the oracle's tree attention equals attention over each query's
  concatenated visible tokens written out by hand (root-to-node order, own
  node's mask bits), in float64.
"""
import numpy as np
import pytest
from hypothesis import HealthCheck, given, settings
from hypothesis import strategies as st

import oracle
import prefix_shared_tree_amd as pst
import workloads
from oracle.flatten import flatten_plan

ROWS = [1, 2, 4, 8, 16, 32, 64, 128, 256]
LENS = [16 << i for i in range(13)]
TABLE = [[700 + 5 * r + 3 * L for L in LENS] for r in ROWS]
SETTINGS = settings(max_examples=150, deadline=None, derandomize=True,
                    suppress_health_check=[HealthCheck.too_slow, HealthCheck.data_too_large])


@st.composite
def trees(draw, max_nodes=10, max_len=300, max_queries=8, g_choices=(1, 2, 4)):
    n = draw(st.integers(1, max_nodes))
    parent = [-1] + [draw(st.integers(-1, i - 1)) for i in range(1, n)]
    lens = [draw(st.integers(1, max_len)) for _ in range(n)]
    masked = [1 if (lens[i] <= 64 and draw(st.booleans()) and draw(st.booleans())) else 0 for i in range(n)]
    b = draw(st.integers(1, max_queries))
    qnode = [draw(st.integers(0, n - 1)) for _ in range(b)]
    qmask = []
    for r in range(b):
        L = lens[qnode[r]]
        if masked[qnode[r]]:
            bits = draw(st.integers(1, (1 << L) - 1))
        else:
            bits = 0
        qmask.append(bits)
    hkv = draw(st.sampled_from([1, 2]))
    g = draw(st.sampled_from(g_choices))
    off = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
    return workloads.TreeSpec("prop", np.array(parent), np.array(lens), off, np.array(qnode), hkv * g, hkv, 64, "f32",
                              0, query_mask=np.array(qmask, dtype=np.uint64) if any(masked) else None,
                              node_masked=np.array(masked, dtype=np.uint8) if any(masked) else None)


@SETTINGS
@given(trees())
def test_index_matches_oracle(spec):
    got = pst.Tree.from_spec(spec, host_only=True).index()
    want = oracle.build_index(spec)
    for key in want:
        assert np.array_equal(got[key], want[key].astype(got[key].dtype)), key


@SETTINGS
@given(trees(), st.integers(1, 12), st.sampled_from([4, 8, 16]))
def test_cost_model_plan_matches_oracle(spec, m, r_max):
    if spec.group > r_max:
        r_max = 16
    tree = pst.Tree.from_spec(spec, host_only=True)
    got = pst.Plan(tree, pst.CostModel(ROWS, LENS, TABLE), num_bins=m, max_rows=r_max, host_only=True).view()
    want = oracle.plan(oracle.build_index(spec), spec.kv_len, spec.group, oracle.CostTable(ROWS, LENS, TABLE), m,
                       r_max=r_max)
    assert np.array_equal(got["tasks"][:, :7], want["tasks"])
    for key in ("bin_ptr", "slot_ptr", "entry_slot", "piece_len", "b_eff", "bin_load"):
        assert np.array_equal(got[key], want[key].astype(got[key].dtype)), key


@SETTINGS
@given(trees(), st.integers(1, 12), st.sampled_from([128, 256, 384]))
def test_flattened_plan_matches_oracle(spec, m, chunk):
    tree = pst.Tree.from_spec(spec, host_only=True)
    got = pst.Plan(tree, pst.CostModel(ROWS, LENS, TABLE), num_bins=m, max_rows=16, flatten=chunk,
                   host_only=True).view()
    want = flatten_plan(oracle.build_index(spec), spec.parent, spec.kv_len, spec.node_masked, spec.group,
                        oracle.CostTable(ROWS, LENS, TABLE), m, chunk=chunk, r_max=16, kv_offset=spec.kv_offset)
    assert np.array_equal(got["tasks"][:, :7], want["tasks"])
    for key in ("bin_ptr", "slot_ptr", "flat_ptr", "flat_query", "flat_mask", "flat_rows"):
        assert np.array_equal(got[key], want[key].astype(got[key].dtype)), key
    assert np.array_equal(got["entry_slot"], want["flat_slot"])


@settings(max_examples=60, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(trees(max_nodes=6, max_len=40, max_queries=4), st.integers(0, 2 ** 31 - 1))
def test_tree_attention_is_attention_over_the_visible_sequence(spec, seed):
    rng = np.random.default_rng(seed)
    T = int(spec.total_tokens)
    q = rng.standard_normal((spec.num_queries, spec.num_q_heads, 64))
    k = rng.standard_normal((spec.num_kv_heads, T, 64))
    v = rng.standard_normal((spec.num_kv_heads, T, 64))
    O, L = oracle.attend(spec, q, k, v)
    for r in range(spec.num_queries):
        # Visible rows by hand: walk up from the query's node, prepend each node.
        rows, i, own = [], int(spec.query_node[r]), int(spec.query_node[r])
        while i >= 0:
            n0, n = int(spec.kv_offset[i]), int(spec.kv_len[i])
            if i == own and spec.node_masked is not None and spec.node_masked[i]:
                part = [n0 + j for j in range(n) if (int(spec.query_mask[r]) >> j) & 1]
            else:
                part = list(range(n0, n0 + n))
            rows = part + rows
            i = int(spec.parent[i])
        for h in range(spec.num_q_heads):
            kv = h // spec.group
            s = (k[kv, rows] @ q[r, h]) / 8.0
            w = np.exp(s - s.max())
            assert np.allclose(O[r, h], (w @ v[kv, rows]) / w.sum(), rtol=0, atol=1e-12)
            assert np.isclose(L[r, h], s.max() + np.log(w.sum()), rtol=0, atol=1e-12)


@settings(max_examples=40, deadline=None, derandomize=True, suppress_health_check=[HealthCheck.too_slow])
@given(st.lists(st.tuples(st.sampled_from("abp"), st.integers(0, 1000), st.integers(1, 3)), min_size=1, max_size=14))
def test_decode_session_random_operations(ops):
    """Random appends, forks and finishes on a host-only decode session, each
    followed by the full consistency check against a node model (tree arrays,
    every token's pool row, page accounting, index and plan bit-exact)."""
    import torch

    from prefix_shared_tree_amd.decode_loop import DecodeSession
    from test_lib_cpu import _session_model_check

    P, max_new = 8, 16
    parent = np.array([-1, 0, 0])
    lens = np.array([30, 5, 12])
    off = np.array([0, 30, 35])
    spec = workloads.TreeSpec("session", parent, lens, off, np.array([1, 2]), 4, 2, 64, "f32", 0)
    T = int(lens.sum())
    ids = torch.arange(1, T + 1, dtype=torch.float32)
    k = torch.zeros((2, T, 64))
    v = torch.zeros((2, T, 64))
    k[:, :, 0] = ids
    v[:, :, 3] = -ids
    cm_lib, cm_or = pst.CostModel(ROWS, LENS, TABLE), oracle.CostTable(ROWS, LENS, TABLE)
    sess = DecodeSession(spec, k, v, page_size=P, max_new_tokens=max_new, extra_pages=60, host_only=True,
                         plan_kw=dict(cost=cm_lib, num_bins=5, max_rows=16))
    nodes = [[int(parent[i]), list(range(int(off[i]) + 1, int(off[i] + lens[i]) + 1)), True] for i in range(3)]
    queries = [1, 2]
    nxt, appends = T + 1, 0
    _session_model_check(sess, nodes, queries, P, cm_or)
    for op, x, n in ops:
        B = len(queries)
        planned = True
        if op == "a":
            if appends >= max_new - 1:
                continue
            kn, vn = torch.zeros((B, 2, 64)), torch.zeros((B, 2, 64))
            for r, mnode in enumerate(queries):
                kn[r, :, 0], vn[r, :, 3] = nxt, -nxt
                nodes[mnode][1].append(nxt)
                nxt += 1
            sess.append(kn, vn)
            appends += 1
            planned = False
        elif op == "b":
            qi = x % B
            kn, vn = torch.zeros((n, 2, 64)), torch.zeros((n, 2, 64))
            new = []
            for j in range(n):
                kn[j, :, 0], vn[j, :, 3] = nxt, -nxt
                nodes.append([queries[qi], [nxt], True])
                new.append(len(nodes) - 1)
                nxt += 1
            try:
                sess.branch(qi, kn, vn)
            except ValueError:  # pool exhausted: nothing changed
                del nodes[-n:]
                nxt -= n
                continue
            queries[qi] = new[0]
            queries += new[1:]
        else:
            if B < 2:
                continue
            qi = x % B
            del queries[qi]
            live = set()
            for mnode in queries:
                while mnode >= 0:
                    live.add(mnode)
                    mnode = nodes[mnode][0]
            for i, nd in enumerate(nodes):
                nd[2] = nd[2] and i in live
            sess.prune(qi)
        _session_model_check(sess, nodes, queries, P, cm_or, planned=planned)
