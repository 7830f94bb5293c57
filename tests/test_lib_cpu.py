"""The C-ABI library on the host (no GPU): exports, bit-exact index and plan
against the oracle, and every error path that can be forced from the host."""
import os
import re

import numpy as np
import pytest

import oracle
import prefix_shared_tree_amd as pst
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROWS = [1, 2, 4, 8, 16, 32, 64, 128, 256]
LENS = [16 << i for i in range(13)]


def test_exports_every_declared_symbol():
    with open(os.path.join(ROOT, "include", "pst.h")) as f:
        header = f.read()
    declared = set(re.findall(r"\b(pst_[a-z_]+)\s*\(", header))
    assert declared, "no declarations found"
    for name in sorted(declared):
        assert hasattr(pst._lib, name), name
    assert declared == set(pst.EXPORTS)


def _tree(spec, **kw):
    return pst.Tree.from_spec(spec, host_only=True, **kw)


def _specs():
    out = [workloads.random_tree(s, max_nodes=9, max_len=300, max_queries=10, num_q_heads=8, num_kv_heads=2,
                                 masked_prob=0.4 if s % 3 == 0 else 0.0) for s in range(25)]
    out += [workloads.config(n) for n in ("1", "2", "3", "4", "5-mqa")]
    return out


@pytest.mark.parametrize("spec", _specs(), ids=lambda s: s.name)
def test_index_bit_exact(spec):
    got = _tree(spec).index()
    want = oracle.build_index(spec)
    for key in want:
        assert np.array_equal(got[key], want[key].astype(got[key].dtype)), key


def _table(kind, seed=0):
    if kind == "affine":
        t = [[900 + 3 * r + 2 * L for L in LENS] for r in ROWS]
    else:
        rng = np.random.default_rng(seed)
        t = (np.cumsum(np.cumsum(rng.integers(1, 60, size=(9, 13)), axis=0), axis=1) + 400).tolist()
    return t


PLAN_CASES = [
    dict(m=32, r_max=256),
    dict(m=7, r_max=16),
    dict(m=1, r_max=256),
    dict(m=64, r_max=8),
    dict(m=16, query_guided=True),
    dict(m=16, no_split=True),
    dict(m=16, fixed_chunk=128),
    dict(m=40, r_max=64, grid_steps=3),
]


@pytest.mark.parametrize("case", range(len(PLAN_CASES)))
@pytest.mark.parametrize("spec", _specs()[::3] + _specs()[-5:], ids=lambda s: s.name)
@pytest.mark.parametrize("tkind", ["affine", "random"])
def test_plan_bit_exact(spec, case, tkind):
    c = dict(PLAN_CASES[case])
    if spec.dtype == "f32" and not c.get("query_guided"):
        c["r_max"] = min(c.get("r_max", 16), 16)
    if spec.dtype == "f32" and c.get("query_guided") and spec.group > 16:
        pytest.skip("f32 rows per workgroup capped at 16")
    table = _table(tkind, seed=case)
    cm = pst.CostModel(ROWS, LENS, table)
    tree = _tree(spec)
    plan = pst.Plan(tree, cm, num_bins=c["m"], max_rows=c.get("r_max", 0), grid_steps=c.get("grid_steps", 0),
                    fixed_chunk=c.get("fixed_chunk", 0), query_guided=c.get("query_guided", False),
                    no_split=c.get("no_split", False), host_only=True)
    got = plan.view()
    ix = oracle.build_index(spec)
    want = oracle.plan(ix, spec.kv_len, spec.group, oracle.CostTable(ROWS, LENS, table), c["m"],
                       r_max=c.get("r_max", 256), grid_steps=c.get("grid_steps", 8),
                       query_guided=c.get("query_guided", False), no_split=c.get("no_split", False),
                       fixed_chunk=c.get("fixed_chunk", 0))
    assert np.array_equal(got["tasks"][:, :7], want["tasks"])
    for key in ("bin_ptr", "slot_ptr", "entry_slot", "piece_len", "b_eff", "rows_per_group", "bin_load"):
        assert np.array_equal(got[key], want[key].astype(got[key].dtype)), key
    for key in ("makespan", "cost_l", "chosen_k", "num_slots"):
        assert got[key] == want[key], key


def test_cost_lookup_matches_oracle():
    table = _table("random", seed=3)
    cm = pst.CostModel(ROWS, LENS, table)
    ot = oracle.CostTable(ROWS, LENS, table)
    for rows in [1, 2, 3, 5, 16, 17, 200, 256, 300]:
        for L in [1, 15, 16, 17, 63, 64, 65, 1000, 4000, 65535, 65536, 65537, 10 ** 6]:
            assert cm.lookup(rows, L) == ot.lookup(rows, L)


# ---------------------------------------------------------------------------
# Error paths (forced from the host)
# ---------------------------------------------------------------------------

def _raises(code, fn, *a, **kw):
    with pytest.raises(pst.PstError) as e:
        fn(*a, **kw)
    assert e.value.code == code, str(e.value)
    return e.value


BAD_TREES = {
    "parent_after_child": dict(parent=[-1, 2, 0]),
    "zero_length": dict(kv_len=[4, 0, 3]),
    "negative_offset": dict(kv_offset=[0, -1, 9]),
    "query_on_missing_node": dict(query_node=[1, 5]),
    "masked_node_too_long": dict(kv_len=[4, 65, 3], node_masked=[0, 1, 0], query_mask=[1, 0]),
    "mask_bit_past_length": dict(node_masked=[0, 1, 0], query_mask=[1 << 2, 0]),
    "query_sees_nothing": dict(parent=[-1, -1, 0], node_masked=[0, 1, 0], query_mask=[0, 0]),
    "node_outside_pool": dict(pool_tokens=8),
}


@pytest.mark.parametrize("case", sorted(BAD_TREES))
def test_invalid_tree(case):
    base = dict(parent=[-1, 0, 0], kv_len=[4, 2, 3], kv_offset=[0, 4, 6], query_node=[1, 2], node_masked=None,
                query_mask=None, pool_tokens=0)
    base.update(BAD_TREES[case])
    _raises("PST_E_INVALID_TREE", pst.Tree, base["parent"], base["kv_offset"], base["kv_len"], base["query_node"],
            num_q_heads=2, num_kv_heads=1, head_dim=64, dtype="f32", node_masked=base["node_masked"],
            query_mask=base["query_mask"], pool_tokens=base["pool_tokens"], host_only=True)


@pytest.mark.parametrize("hq,hkv,d,dt,odt", [(3, 2, 64, "f32", None), (4, 4, 96, "f32", None),
                                             (4, 4, 64, "f32", "bf16"), (512, 1, 128, "bf16", None)])
def test_unsupported_shape(hq, hkv, d, dt, odt):
    _raises("PST_E_UNSUPPORTED", pst.Tree, [-1], [0], [5], [0], num_q_heads=hq, num_kv_heads=hkv, head_dim=d,
            dtype=dt, out_dtype=odt, host_only=True)


@pytest.mark.parametrize("stride,ok", [((1 << 22) - 4, True), (1 << 22, False)])
def test_token_stride_limit(stride, ok):
    """Token strides of 16 MiB or more are refused (the kernels' per-tile offsets are 32-bit)."""
    mk = lambda: pst.Tree([-1], [0], [5], [0], num_q_heads=2, num_kv_heads=1, head_dim=64, dtype="f32",
                          kv_stride_token=stride, kv_stride_head=64, host_only=True)
    if ok:
        mk().free()
    else:
        _raises("PST_E_INVALID_ARG", mk)


def test_bad_cost_tables():
    _raises("PST_E_INVALID_ARG", pst.CostModel, ROWS, LENS, [[0] * 13] * 9)
    bad = _table("affine")
    bad[2][5] = 1
    _raises("PST_E_INVALID_ARG", pst.CostModel, ROWS, LENS, bad)
    _raises("PST_E_INVALID_ARG", pst.CostModel, [1, 1], LENS, _table("affine")[:2])


def test_bad_plan_options():
    t = _tree(workloads.config("1"))
    _raises("PST_E_INVALID_ARG", pst.Plan, t, tile=100, host_only=True)
    _raises("PST_E_INVALID_ARG", pst.Plan, t, max_rows=512, host_only=True)
    _raises("PST_E_INVALID_ARG", pst.Plan, t, fixed_chunk=70, host_only=True)
    _raises("PST_E_UNSUPPORTED", pst.Plan, t, max_rows=64, host_only=True)  # float32 rows > 16


def _a256(n):
    return -(-n // 256) * 256


@pytest.mark.parametrize("odt", ["f32", "bf16"])
@pytest.mark.parametrize("dot_small", [False, True])
def test_workspace_layout(odt, dot_small):
    """The workspace holds the partial outputs and their LSE: float32 partials
    and float32 LSE, or, when input and output are bf16 and every piece runs on
    the matrix cores, fp16 partials and (LSE, exponent) pairs; each array
    256-byte aligned (the layout include/pst.h states)."""
    spec = workloads.config("3")
    t = _tree(spec, out_dtype=odt)
    plan = pst.Plan(t, num_bins=32, host_only=True, dot_small=dot_small)
    S, H, D = plan.view()["num_slots"], spec.num_q_heads, spec.head_dim
    f16 = odt == "bf16" and not dot_small
    want = _a256(S * H * D * (2 if f16 else 4)) + _a256(S * H * (8 if f16 else 4))
    assert plan.workspace_bytes == want
    t32 = _tree(workloads.config("1"))
    p32 = pst.Plan(t32, num_bins=4, host_only=True)
    v = p32.view()
    assert p32.workspace_bytes == _a256(v["num_slots"] * 4 * 64 * 4) + _a256(v["num_slots"] * 4 * 4)


def test_engine_threshold():
    """bf16 plans put every piece on the matrix cores unless PST_PLAN_DOT_SMALL asks for the
    dot-product path below 16 rows; float32 plans never use them."""
    t = _tree(workloads.config("3"))
    assert pst.Plan(t, num_bins=8, host_only=True).view()["mfma_min_rows"] == 1
    assert pst.Plan(t, num_bins=8, host_only=True, dot_small=True).view()["mfma_min_rows"] == 16
    t1 = _tree(workloads.config("1"))
    assert pst.Plan(t1, num_bins=4, host_only=True).view()["mfma_min_rows"] == 2**31 - 1


def test_host_only_objects_cannot_launch():
    import ctypes as C

    t = _tree(workloads.config("1"))
    p = pst.Plan(t, num_bins=4, host_only=True)
    dummy = C.c_void_p(4096)  # never dereferenced: the call fails before any launch
    st = pst._lib.pst_decode_attn(p._h, dummy, dummy, dummy, dummy, None, dummy, 1 << 20, None)
    assert pst.STATUS[st] == "PST_E_NO_DEVICE"
    assert "host-only" in pst._lib.pst_last_error().decode()


def test_binding_rejects_host_tensors():
    import torch

    t = _tree(workloads.config("1"))
    p = pst.Plan(t, num_bins=4, host_only=True)
    x = torch.zeros(4 * 4 * 64)
    with pytest.raises(ValueError):
        pst.decode_attn(p, x, x, x, out=x, lse=None, ws=torch.zeros(4096, dtype=torch.uint8))


def test_free_order_and_lengths():
    spec = workloads.config("3")
    t = _tree(spec)
    p = pst.Plan(t, num_bins=8, host_only=True)
    _raises("PST_E_INVALID_ARG", t.free)  # a plan still borrows the tree
    shorter = spec.kv_len.copy()
    shorter[5] -= 1
    _raises("PST_E_INVALID_ARG", t.set_lengths, shorter)
    longer = spec.kv_len.copy()
    longer[-1] += 10
    _raises("PST_E_INVALID_TREE", t.set_lengths, longer)  # leaves the pool (pool = exact size)
    p.free()
    t.free()


def test_growth_keeps_plan_and_updates_visible():
    spec = workloads.config("2")
    pool = spec.total_tokens + 1000
    # Leaves are contiguous: give the last leaf room to grow inside a larger pool.
    t = pst.Tree.from_spec(spec, host_only=True, pool_tokens=pool)
    p = pst.Plan(t, num_bins=32, host_only=True)
    before = p.view()
    lens = spec.kv_len.copy()
    lens[-1] += 7
    t.set_lengths(lens)
    assert t.index()["visible"][-1] == 32768 + 512 + 7
    assert np.array_equal(p.view()["tasks"], before["tasks"])  # the plan is reused as is


def test_empty_batch():
    t = pst.Tree([-1], [0], [10], [], num_q_heads=4, num_kv_heads=4, head_dim=64, dtype="f32", host_only=True)
    p = pst.Plan(t, num_bins=4, host_only=True)
    v = p.view()
    assert v["tasks"].shape == (0, 8) and v["num_slots"] == 0 and p.workspace_bytes == 0


def _paged_tree(**kw):
    base = dict(parent=[-1, 0, 0], kv_len=[20, 9, 3], query_node=[1, 2], page_size=8,
                page_ptr=[0, 3, 5, 6], page_idx=[7, 2, 9, 0, 4, 11], pool_tokens=0)
    base.update(kw)
    return pst.Tree(base["parent"], None, base["kv_len"], base["query_node"], num_q_heads=2, num_kv_heads=1,
                    head_dim=64, dtype="f32", page_size=base["page_size"], page_ptr=base["page_ptr"],
                    page_idx=base["page_idx"], pool_tokens=base["pool_tokens"], host_only=True)


def test_paged_index_view_and_extent():
    t = _paged_tree()
    ix = t.index()
    assert ix["page_size"] == 8
    assert ix["page_ptr"].tolist() == [0, 3, 5, 6] and ix["page_idx"].tolist() == [7, 2, 9, 0, 4, 11]
    assert ix["visible"].tolist() == [29, 23]
    assert t.kv_extent == 12 * 8 * 64  # (largest page + 1) pages of 8 rows of 64 channels
    p = pst.Plan(t, num_bins=2, host_only=True)
    assert p.view()["tasks"].shape[0] == 3  # one piece per node (plan is layout-independent)


@pytest.mark.parametrize("kw,code", [
    (dict(page_size=12), "PST_E_INVALID_ARG"),                  # not a power of two
    (dict(page_size=4), "PST_E_INVALID_ARG"),                   # below 8 tokens
    (dict(page_ptr=[1, 3, 5, 6]), "PST_E_INVALID_TREE"),        # page_ptr[0] != 0
    (dict(page_ptr=[0, 3, 2, 6]), "PST_E_INVALID_TREE"),        # decreasing
    (dict(page_ptr=[0, 2, 4, 6]), "PST_E_INVALID_TREE"),        # node 0: 20 tokens in 2 pages of 8
    (dict(page_idx=[7, 2, -1, 0, 4, 11]), "PST_E_INVALID_TREE"),  # negative page
    (dict(pool_tokens=64), "PST_E_INVALID_TREE"),               # page 11 lies outside 64 rows
    (dict(pool_tokens=1 << 31), "PST_E_INVALID_ARG"),           # rows beyond 31 bits
])
def test_paged_invalid(kw, code):
    _raises(code, _paged_tree, **kw)


def test_paged_growth_within_pages():
    t = _paged_tree()
    p = pst.Plan(t, num_bins=2, host_only=True)
    t.set_lengths([24, 16, 8])  # every node fills its pages exactly
    assert t.index()["visible"].tolist() == [40, 32]
    _raises("PST_E_INVALID_TREE", t.set_lengths, [25, 16, 8])  # node 0 would outgrow its 3 pages
    p.free()
    t.free()


def _session_model_check(sess, nodes, queries, P, cm, planned=True):
    """The session against a plain model: ``nodes`` is a list of [parent, token ids, alive]
    (never reordered), ``queries`` the model node of each query.  ``planned``: the plan was
    made for the current lengths (else it is the one made before the last growth)."""
    import torch

    alive = [i for i, n in enumerate(nodes) if n[2]]
    rank = {m: r for r, m in enumerate(alive)}
    par = [rank[nodes[m][0]] if nodes[m][0] >= 0 else -1 for m in alive]
    assert sess.parent.tolist() == par
    assert sess.kv_len.tolist() == [len(nodes[m][1]) for m in alive]
    assert sess.query_node.tolist() == [rank[m] for m in queries]
    # Pages: live nodes own disjoint pages that, with the free list, cover the pool once.
    owned = [p for pg in sess.pages for p in pg]
    assert sorted(owned + sess.free) == list(range(sess.pool_pages))
    for i, m in enumerate(alive):
        assert len(sess.pages[i]) * P >= len(nodes[m][1])
    # Every token sits in the pool where the page table says.
    parent, kv_len, off, qn, k, v = sess.contiguous()
    want = [t for m in alive for t in nodes[m][1]]
    assert k[0, :, 0].tolist() == want and v[1, :, 3].tolist() == [-t for t in want]
    # Index and plan of the rebuilt tree, bit-exact against the oracle.
    spec = workloads.TreeSpec("session", parent, kv_len, off, qn, 4, 2, 64, "f32", 0)
    ix = oracle.build_index(spec)
    got = sess.tree.index()
    for key in ix:
        assert np.array_equal(got[key], ix[key].astype(got[key].dtype)), key
    paths = []
    for m in queries:
        s, n = 0, m
        while n >= 0:
            s += len(nodes[n][1])
            n = nodes[n][0]
        paths.append(s)
    assert got["visible"].tolist() == paths
    if planned:
        sess._planned_lens = kv_len
    spec.kv_len = sess._planned_lens
    want_plan = oracle.plan(oracle.build_index(spec), sess._planned_lens, spec.group, cm, 5, r_max=16)
    assert np.array_equal(sess.plan.view()["tasks"][:, :7], want_plan["tasks"])


def test_decode_session_branch_prune_bookkeeping():
    """Append, branch and prune on a host-only session: the tree, the page
    pool and the plan stay consistent with a model that never moves nodes."""
    import torch

    from prefix_shared_tree_amd.decode_loop import DecodeSession

    P, max_new = 8, 24
    parent = np.array([-1, 0, 0, 1])
    lens = np.array([40, 17, 5, 9])
    off = np.concatenate([[0], np.cumsum(lens)[:-1]])
    qnode = np.array([2, 3])
    spec = workloads.TreeSpec("session", parent, lens, off, qnode, 4, 2, 64, "f32", 0)
    T = int(lens.sum())
    ids = torch.arange(1, T + 1, dtype=torch.float32)
    k = torch.zeros((2, T, 64))
    v = torch.zeros((2, T, 64))
    k[:, :, 0] = ids
    v[:, :, 3] = -ids
    table = _table("affine")
    cm_lib, cm_or = pst.CostModel(ROWS, LENS, table), oracle.CostTable(ROWS, LENS, table)
    sess = DecodeSession(spec, k, v, page_size=P, max_new_tokens=max_new, extra_pages=64, host_only=True,
                         plan_kw=dict(cost=cm_lib, num_bins=5, max_rows=16))
    nodes = [[int(parent[i]), list(range(int(off[i]) + 1, int(off[i] + lens[i]) + 1)), True] for i in range(4)]
    queries = [2, 3]
    nxt = T + 1
    rng = np.random.default_rng(5)
    _session_model_check(sess, nodes, queries, P, cm_or)
    appends = 0
    for op in ["a", "b", "a", "a", "b", "p", "a", "b", "p", "a", "p", "b", "a", "a", "p", "b", "a"]:
        B = len(queries)
        if op == "a" and appends < max_new - 1:
            kn = torch.zeros((B, 2, 64))
            vn = torch.zeros((B, 2, 64))
            for r, m in enumerate(queries):
                kn[r, :, 0] = nxt
                vn[r, :, 3] = -nxt
                nodes[m][1].append(nxt)
                nxt += 1
            sess.append(kn, vn)
            appends += 1
            _session_model_check(sess, nodes, queries, P, cm_or, planned=False)
            continue
        elif op == "b":
            qi, n = int(rng.integers(B)), int(rng.integers(1, 4))
            kn = torch.zeros((n, 2, 64))
            vn = torch.zeros((n, 2, 64))
            new = []
            for j in range(n):
                kn[j, :, 0] = nxt
                vn[j, :, 3] = -nxt
                nodes.append([queries[qi], [nxt], True])
                new.append(len(nodes) - 1)
                nxt += 1
            got = sess.branch(qi, kn, vn)
            assert got == list(range(B, B + n - 1))
            queries[qi] = new[0]
            queries += new[1:]
        elif op == "p" and B > 1:
            qi = int(rng.integers(B))
            del queries[qi]
            live = set()
            for m in queries:
                while m >= 0:
                    live.add(m)
                    m = nodes[m][0]
            for i, n in enumerate(nodes):
                n[2] = n[2] and i in live
            sess.prune(qi)
        _session_model_check(sess, nodes, queries, P, cm_or)
    with pytest.raises(ValueError):
        sess.branch(0, torch.zeros((200, 2, 64)), torch.zeros((200, 2, 64)))  # more pages than the pool has
    _session_model_check(sess, nodes, queries, P, cm_or, planned=False)  # a refused branch changes nothing


FLAT_CASES = [(128, 256, 5), (256, 16, 3), (512, 256, 32), (1024, 8, 7), (640, 64, 1)]


@pytest.mark.parametrize("chunk,r_max,m", FLAT_CASES)
@pytest.mark.parametrize("spec", _specs()[::2] + [workloads.config("4")], ids=lambda s: s.name)
def test_flatten_plan_bit_exact(spec, chunk, r_max, m):
    """DEFT-Flatten partition: the library's tasks, bins, entries, masks, row
    table and slots equal the oracle's."""
    from oracle.flatten import flatten_plan

    if spec.dtype == "f32":
        r_max = min(r_max, 16)
    if spec.group > r_max:
        pytest.skip("GQA group larger than a row group")
    table = _table("random", seed=chunk)
    cm = pst.CostModel(ROWS, LENS, table)
    plan = pst.Plan(_tree(spec), cm, num_bins=m, max_rows=r_max, flatten=chunk, host_only=True)
    got = plan.view()
    ix = oracle.build_index(spec)
    want = flatten_plan(ix, spec.parent, spec.kv_len, spec.node_masked, spec.group,
                        oracle.CostTable(ROWS, LENS, table), m, chunk=chunk, r_max=r_max, kv_offset=spec.kv_offset)
    assert got["flat_chunk"] == chunk
    assert np.array_equal(got["tasks"][:, :7], want["tasks"])
    for key in ("bin_ptr", "slot_ptr", "bin_load", "flat_ptr", "flat_query", "flat_mask", "flat_rows"):
        assert np.array_equal(got[key], want[key].astype(got[key].dtype)), key
    assert np.array_equal(got["entry_slot"], want["flat_slot"])
    assert got["makespan"] == want["makespan"] and got["num_slots"] == want["num_slots"]


@pytest.mark.parametrize("page", [8, 32])
def test_flatten_plan_paged_bit_exact(page):
    from oracle.flatten import flatten_plan

    spec = workloads.config("3")
    paged = _paged_tables(spec, page)
    tree = pst.Tree.from_paged(spec, paged, host_only=True)
    table = _table("affine")
    plan = pst.Plan(tree, pst.CostModel(ROWS, LENS, table), num_bins=16, flatten=256, host_only=True)
    got = plan.view()
    ix = oracle.build_index(spec)
    want = flatten_plan(ix, spec.parent, spec.kv_len, None, spec.group, oracle.CostTable(ROWS, LENS, table), 16,
                        chunk=256, page_size=page, page_ptr=paged["page_ptr"], page_idx=paged["page_idx"])
    for key in ("flat_rows", "flat_mask", "flat_query"):
        assert np.array_equal(got[key], want[key].astype(got[key].dtype)), key
    assert np.array_equal(got["tasks"][:, :7], want["tasks"])


def _paged_tables(spec, page):
    """Page tables with scattered page numbers (no K/V needed on the host)."""
    rng = np.random.default_rng(page)
    npg = (np.asarray(spec.kv_len, dtype=np.int64) + page - 1) // page
    page_ptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
    page_idx = rng.permutation(int(page_ptr[-1]) + 7)[:int(page_ptr[-1])].astype(np.int32)
    return {"page_size": page, "page_ptr": page_ptr, "page_idx": page_idx}


def test_flatten_options_and_growth():
    spec = workloads.config("1")
    t = _tree(spec)
    _raises("PST_E_INVALID_ARG", pst.Plan, t, num_bins=4, flatten=192, host_only=True)  # not a multiple of 128
    _raises("PST_E_INVALID_ARG", pst.Plan, t, num_bins=4, flatten=256, no_split=True, host_only=True)
    _raises("PST_E_INVALID_ARG", pst.Plan, t, num_bins=4, flatten=256, query_guided=True, host_only=True)
    _raises("PST_E_UNSUPPORTED", pst.Plan, t, num_bins=4, flatten=128 * 1024, host_only=True)  # masks exceed 8 KB
    p = pst.Plan(t, num_bins=4, flatten=256, host_only=True)
    before = t.index()["visible"].copy()
    longer = spec.kv_len.copy()
    _raises("PST_E_UNSUPPORTED", t.set_lengths, longer)  # refused while a flattened plan is live
    assert np.array_equal(t.index()["visible"], before)
    p.free()
    t.set_lengths(longer)  # allowed again
    t.free()


def test_paged_block_tables_of_the_pages_example():
    """The shared-prefix blog's paged example (section 4.3, tests/golden): a
    96-token prefix in pages 0-5 and two 4-token suffixes in pages 6 and 7.
    The per-request block tables, their indptr, last-page lengths and every
    token's pool row follow from the tree's page table and the query paths."""
    import json

    with open(os.path.join(ROOT, "tests", "golden", "flashinfer_paged_prefix_96_4_4.json")) as f:
        g = json.load(f)
    tr, P = g["tree"], g["page_size"]
    t = pst.Tree(tr["parent"], None, tr["kv_len"], tr["query_node"], num_q_heads=4, num_kv_heads=1, head_dim=64,
                 dtype="f32", page_size=P, page_ptr=tr["page_ptr"], page_idx=tr["page_idx"], host_only=True)
    ix = t.index()
    assert ix["visible"].tolist() == g["expect"]["visible"]
    tables, last = [], []
    for r in range(len(tr["query_node"])):
        path = ix["qn_idx"][ix["qn_ptr"][r]:ix["qn_ptr"][r + 1]]
        pages = [int(p) for i in path for p in ix["page_idx"][ix["page_ptr"][i]:ix["page_ptr"][i + 1]]]
        tables.append(pages)
        last.append(int(tr["kv_len"][path[-1]]) % P or P)
        # Token j of the request's sequence: pool row from the block table
        # (the page's view) equals the row through the node that holds it.
        rows_block = [pages[j // P] * P + j % P for j in range(int(ix["visible"][r]))]
        rows_tree = [int(ix["page_idx"][ix["page_ptr"][i] + j // P]) * P + j % P
                     for i in path for j in range(int(tr["kv_len"][i]))]
        assert rows_block == rows_tree
    assert [0] + list(np.cumsum([len(x) for x in tables])) == g["expect"]["paged_kv_indptr"]
    assert [p for x in tables for p in x] == g["expect"]["paged_kv_indices"]
    assert last == g["expect"]["paged_kv_last_page_len"]


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus N > 1 exits with a message, before touching a device."""
    import subprocess
    import sys

    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def test_build_script_loads_without_the_package():
    """build() must work on a fresh checkout, where the package refuses to
    import because libpst.so does not exist yet: the build script is loaded
    by path and imports nothing from the package."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = (
        "import importlib.util, os, sys\n"
        f"spec = importlib.util.spec_from_file_location('_b', os.path.join({root!r}, 'prefix_shared_tree_amd', 'build.py'))\n"
        "m = importlib.util.module_from_spec(spec); spec.loader.exec_module(m)\n"
        "assert callable(m.build)\n"
        "assert 'prefix_shared_tree_amd' not in sys.modules\n"
    )
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, cwd="/")
    assert r.returncode == 0, r.stderr
    src = open(os.path.join(root, "__graft_entry__.py")).read()
    assert "spec_from_file_location" in src and "from prefix_shared_tree_amd.build" not in src


# ---------------------------------------------------------------------------
# Fitted cost tables as shipped: the JSON loader and the plans the bench runs
# ---------------------------------------------------------------------------

TABLE_DIR = os.path.join(ROOT, "prefix_shared_tree_amd", "cost_tables")
SHIPPED = sorted(f for f in os.listdir(TABLE_DIR) if f.startswith("gfx950_") and f.endswith(".json"))


def _json_table(name):
    import json

    with open(os.path.join(TABLE_DIR, name)) as f:
        d = json.load(f)
    return d["rows_grid"], d["len_grid"], d["table_ns"]


@pytest.mark.parametrize("name", SHIPPED)
def test_cost_model_load_matches_the_file(name):
    """pst_cost_model_load reads the shipped table: every lookup (grid points,
    between them, below and beyond the grids) equals the oracle's lookup on
    the arrays Python's own JSON reader finds in the file."""
    lib = pst.CostModel.load(os.path.join(TABLE_DIR, name))
    rg, lg, tb = _json_table(name)
    ot = oracle.CostTable(rg, lg, tb)
    for rows in [1, 2, 3, 7, 16, 31, 32, 100, 255, 256, 257, 1000]:
        for L in [1, 15, 16, 17, 100, 1023, 1024, 1025, 40000, 65536, 65537, 300000]:
            assert lib.lookup(rows, L) == ot.lookup(rows, L), (rows, L)


@pytest.mark.parametrize("text,why", [
    ("", "not an object"),
    ("[1, 2]", "not an object"),
    ('{"rows_grid": [1, 2], "len_grid": [16, 32]}', "no table"),
    ('{"rows_grid": [1], "len_grid": [16, 32], "table_ns": [[5, 6]]} x', "trailing characters"),
    ('{"rows_grid": [1], "len_grid": [16, 32], "table_ns": [[5, 6.5]]}', "fractional cost"),
    ('{"rows_grid": [1, 2], "len_grid": [16, 32], "table_ns": [[5, 6]]}', "one table row missing"),
    ('{"rows_grid": [1], "len_grid": [16, 32], "table_ns": [[5]]}', "short table row"),
    ('{"rows_grid": [1], "len_grid": [16, 32], "table_ns": [[6, 5]]}', "decreasing costs"),
    ('{"rows_grid": [2, 1], "len_grid": [16, 32], "table_ns": [[5, 6], [5, 6]]}', "rows grid not ascending"),
    ('{"rows_grid": [1], "len_grid": [16, 32], "table_ns": [[5, 6]]', "unterminated object"),
    ('{"rows_grid": [1], "len_grid": [16, 32], "table_ns": [[5, 6]], "note": "\\q"}', "bad escape"),
])
def test_cost_model_load_rejects(tmp_path, text, why):
    path = tmp_path / "t.json"
    path.write_text(text)
    e = _raises("PST_E_INVALID_ARG", pst.CostModel.load, str(path))
    assert "t.json" in str(e), why


def test_cost_model_load_missing_file_and_extra_keys(tmp_path):
    _raises("PST_E_INVALID_ARG", pst.CostModel.load, str(tmp_path / "absent.json"))
    path = tmp_path / "ok.json"
    path.write_text('{"note": {"a": [true, false, null, -1.5e3, "x\\u00e9"]}, "rows_grid": [1],'
                    ' "len_grid": [16, 32], "table_ns": [[5, 9]], "raw_ns": [[1.25, 2]]}')
    cm = pst.CostModel.load(str(path))
    assert cm.lookup(1, 24) == 7 and cm.lookup(4, 48) == 13


@pytest.mark.parametrize("name", SHIPPED)
@pytest.mark.parametrize("cfg", ["1", "2", "3", "4", "5-mqa", "5-mha"])
def test_plan_bit_exact_under_shipped_tables(name, cfg):
    """The plans of the workloads under each shipped gfx950 table, with the
    bins an MI355X gives (256 compute units, one PAC workgroup each, per kv
    head), equal the oracle's plans bit for bit."""
    spec = workloads.config(cfg)
    m = max(1, 256 // spec.num_kv_heads)
    r_max = 16 if spec.dtype == "f32" else 256
    lib = pst.Plan(_tree(spec), pst.CostModel.load(os.path.join(TABLE_DIR, name)), num_bins=m, host_only=True)
    got = lib.view()
    want = oracle.plan(oracle.build_index(spec), spec.kv_len, spec.group, oracle.CostTable(*_json_table(name)), m,
                       r_max=r_max)
    assert np.array_equal(got["tasks"][:, :7], want["tasks"])
    for key in ("bin_ptr", "slot_ptr", "entry_slot", "piece_len", "b_eff", "rows_per_group", "bin_load"):
        assert np.array_equal(got[key], want[key].astype(got[key].dtype)), key
    for key in ("makespan", "cost_l", "chosen_k", "num_slots"):
        assert got[key] == want[key], key


def test_baseline_entry_needs_a_device_tree():
    import ctypes as C

    t = _tree(workloads.config("1"))
    dummy = C.c_void_p(4096)  # never dereferenced: the call fails before any launch
    st = pst._lib.pst_decode_attn_baseline(t._h, None, dummy, dummy, dummy, dummy, None, dummy, 1 << 20, None)
    assert pst.STATUS[st] == "PST_E_NO_DEVICE"
    n = C.c_size_t()
    assert pst.STATUS[pst._lib.pst_baseline_workspace_size(t._h, None, None, C.byref(n))] == "PST_E_NO_DEVICE"


def test_pac_and_por_check_their_tensors():
    """The per-phase calls check sizes, dtypes and devices like decode_attn:
    the kernels size their reads from the plan, not from the tensors."""
    import torch

    t = _tree(workloads.config("1"))
    p = pst.Plan(t, num_bins=4, host_only=True)
    x = torch.zeros(4 * 4 * 64)
    ws = torch.zeros(1 << 16, dtype=torch.uint8)
    with pytest.raises(ValueError):
        pst.pac(p, x, x, x, ws)
    with pytest.raises(ValueError):
        pst.por(p, x, None, ws)


def test_set_lengths_needs_one_length_per_node():
    spec = workloads.config("3")
    t = _tree(spec)
    with pytest.raises(ValueError):
        t.set_lengths(spec.kv_len[:-1])
    with pytest.raises(ValueError):
        t.set_lengths(np.concatenate([spec.kv_len, [5]]))


def test_noalloc_limit_and_host_only_plans():
    """The binding's copy of PST_NOALLOC_SCRATCH_BYTES is the header's, and the
    allocation-free entry point refuses host-only plans before any device call."""
    import ctypes as C

    with open(os.path.join(ROOT, "include", "pst.h")) as f:
        m = re.search(r"#define PST_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", f.read())
    assert m and int(m.group(1)) << int(m.group(2)) == pst.NOALLOC_SCRATCH_BYTES
    t = _tree(workloads.config("1"))
    p = pst.Plan(t, num_bins=4, host_only=True)
    dummy = C.c_void_p(4096)  # never dereferenced
    st = pst._lib.pst_decode_attn_noalloc(p._h, dummy, dummy, dummy, dummy, None, None)
    assert pst.STATUS[st] == "PST_E_NO_DEVICE"
