"""GPU parity: the HIP path (through the C ABI) against the float64 oracle.

Tolerances (max-abs, float32 outputs): 1e-5 for float32 inputs, 2e-3 for
bfloat16 inputs with float32 accumulation.  bfloat16 outputs are checked to
be the round-to-nearest-even of an output within that tolerance (within one
bf16 ulp of the oracle plus 2e-3).  Full-size workloads are checked on
sampled queries (every head of each sampled query).
"""
import math
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import oracle  # noqa: E402
import workloads  # noqa: E402

pytestmark = pytest.mark.gpu

if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("needs a GPU", allow_module_level=True)

import prefix_shared_tree_amd as pst  # noqa: E402

TOL = {"f32": 1e-5, "bf16": 2e-3}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def run(spec, *, out_dtype="f32", q_scale=1.0, tensors=None, **plan_kw):
    q, k, v = tensors if tensors is not None else workloads.make_tensors(spec, "cuda", q_scale=q_scale)
    tree = pst.Tree.from_spec(spec, out_dtype=out_dtype)
    plan = pst.Plan(tree, **plan_kw)
    out, lse = pst.decode_attn(plan, q, k, v)
    torch.cuda.synchronize()
    return (q, k, v), plan, out, lse


def check(spec, tensors, out, lse, queries=None, tol=None, lse_tol=None, by_node=False):
    """Max-abs errors of ``out`` and ``lse`` on ``queries`` against the oracle.

    ``by_node``: at full size, the oracle's answer is formed per path node
    (see :func:`oracle_by_node`) instead of per query."""
    q, k, v = tensors
    if queries is None:
        queries = list(range(spec.num_queries))
    if by_node:
        O, L = oracle_by_node(spec, q, k, v, queries)
    else:
        O, L = oracle.attend(spec, q, k, v, queries=queries)
    got = out[queries].double().cpu().numpy()
    tol = TOL[spec.dtype] if tol is None else tol
    lse_tol = max(tol, 1e-5) * 4 if lse_tol is None else lse_tol
    lerr = np.abs(lse[queries].double().cpu().numpy() - L).max() if len(queries) else 0.0
    if out.dtype == torch.bfloat16:
        # A bf16 output is the rounding to nearest of a value within `tol`:
        # allow one bf16 ulp of the oracle's value on top (bf16 keeps 8
        # significant bits).
        ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(O), 1e-38))) - 7)
        excess = (np.abs(got - O) - ulp).max() if len(queries) else 0.0
        err = np.abs(got - O).max() if len(queries) else 0.0
        say(f"  {spec.name}: bf16 out, max|dO| = {err:.3e} (beyond one ulp {excess:.3e}), "
            f"max|dLSE| = {lerr:.3e} over {len(queries)} queries")
        assert excess <= tol, excess
        assert lerr <= lse_tol, lerr
        return err
    err = np.abs(got - O).max() if len(queries) else 0.0
    say(f"  {spec.name}: max|dO| = {err:.3e}, max|dLSE| = {lerr:.3e} over {len(queries)} queries")
    assert err <= tol, err
    assert lerr <= lse_tol, lerr
    return err


def oracle_by_node(spec, q, k, v, queries):
    """The oracle for ``queries`` of an unmasked tree whose K/V are too large
    to gather once per query: each node on the queries' paths is copied from
    the device once, every checked query's partial attention over it comes
    from ``oracle.partial_attend`` in float64, and each query's partials are
    merged with ``oracle.lse_merge`` (the split-and-merge identity the CPU
    tests pin against one full softmax to 1e-12)."""
    assert spec.node_masked is None or not np.asarray(spec.node_masked).any()
    hq, hkv, d = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    g = hq // hkv
    scale = 1.0 / math.sqrt(d)
    paths = []
    for r in queries:
        path, n = [], int(spec.query_node[r])
        while n >= 0:
            path.append(n)
            n = int(spec.parent[n])
        paths.append(path[::-1])
    through = {}
    for qi, path in enumerate(paths):
        for n in path:
            through.setdefault(n, []).append(qi)
    qh = q[queries].cpu().double().numpy()  # [n, hq, d]
    parts = [dict() for _ in queries]  # node -> (O [hq, d], LSE [hq])
    for n in sorted(through):
        rs = through[n]
        a, L = int(spec.kv_offset[n]), int(spec.kv_len[n])
        O = np.zeros((len(rs), hq, d))
        lse = np.zeros((len(rs), hq))
        for kh in range(hkv):
            K = k[kh, a:a + L].cpu().double().numpy()
            V = v[kh, a:a + L].cpu().double().numpy()
            heads = slice(kh * g, (kh + 1) * g)
            rows = qh[rs][:, heads].reshape(-1, d)
            Oh, _, _, lh = oracle.partial_attend(rows, K, V, scale)
            O[:, heads] = Oh.reshape(len(rs), g, d)
            lse[:, heads] = lh.reshape(len(rs), g)
        for j, qi in enumerate(rs):
            parts[qi][n] = (O[j], lse[j])
    Oall = np.zeros((len(queries), hq, d))
    Lall = np.zeros((len(queries), hq))
    for qi, path in enumerate(paths):
        Oall[qi], Lall[qi] = oracle.lse_merge([parts[qi][n][0] for n in path], [parts[qi][n][1] for n in path])
    return Oall, Lall


def per_leaf_queries(spec):
    """One query (the lowest id) per node some query sits on: every node of
    the tree, and so every piece of every node, lies on a checked path."""
    first = {}
    for r, n in enumerate(spec.query_node):
        first.setdefault(int(n), r)
    return sorted(first.values())


def sample(n, k, seed=0):
    if n <= k:
        return list(range(n))
    rng = np.random.default_rng(seed)
    return sorted(rng.choice(n, size=k, replace=False).tolist())


@pytest.mark.parametrize("name", ["1", "3"])
def test_config_full(name):
    spec = workloads.config(name)
    say(f"config {name}: {spec.name}")
    t, plan, out, lse = run(spec)
    check(spec, t, out, lse)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_config2_all_queries(out_dtype):
    """The document-QA tree, every query (every head): the root's pieces and
    every leaf; with a bf16 output the partials travel in fp16."""
    spec = workloads.config("2")
    say(f"config 2: {spec.name}, {out_dtype} output")
    t, plan, out, lse = run(spec, out_dtype=out_dtype)
    check(spec, t, out, lse, by_node=True)


def config4_queries(spec, extra=32, seed=1):
    """One query per request (its deepest draft node, so the request's prefix
    and its masked draft node are both checked) plus seeded random others."""
    per_request = {}
    for r, n in enumerate(spec.query_node):
        per_request.setdefault(int(spec.parent[int(n)]), []).append(r)
    chosen = set()
    for rs in per_request.values():
        chosen.add(max(rs, key=lambda r: bin(int(spec.query_mask[r])).count("1")))
    chosen.update(sample(spec.num_queries, extra, seed))
    return sorted(chosen)


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_config4_every_request(out_dtype):
    spec = workloads.config("4")
    say(f"config 4: {spec.name}, {out_dtype} output")
    t, plan, out, lse = run(spec, out_dtype=out_dtype)
    queries = config4_queries(spec)
    assert len({int(spec.parent[int(spec.query_node[r])]) for r in queries}) == 16
    check(spec, t, out, lse, queries=queries)


def test_config5_mqa_every_leaf():
    spec = workloads.config("5-mqa")
    say(f"config 5-mqa: {spec.name}")
    t, plan, out, lse = run(spec)
    check(spec, t, out, lse, queries=per_leaf_queries(spec), by_node=True)


def test_config5_mha_every_leaf():
    """The largest workload (MHA 32/32, ~38 GB of K/V: pool offsets beyond
    2^32 bytes), in the launch configuration the bench times, on one query per
    leaf (every head): every node and every piece lies on a checked path."""
    spec = workloads.config("5-mha")
    say(f"config 5-mha: {spec.name}, {spec.total_tokens} tokens")
    t, plan, out, lse = run(spec)
    queries = per_leaf_queries(spec)
    say(f"  checking {len(queries)} queries (one per leaf)")
    check(spec, t, out, lse, queries=queries, by_node=True)
    del t


@pytest.mark.parametrize("seed", range(24))
def test_random_trees(seed):
    """Random forests spanning the dot-product / matrix-core switch (rows 1..300)."""
    rng = np.random.default_rng(seed)
    dtype = "f32" if seed % 4 == 0 else "bf16"
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 4, 8, 32]))
    d = 64 if seed % 5 == 0 else 128
    spec = workloads.random_tree(1000 + seed, max_nodes=8, max_len=int(rng.choice([40, 300, 2000])),
                                 max_queries=int(rng.choice([3, 12, 40])), num_q_heads=hkv * g, num_kv_heads=hkv,
                                 head_dim=d, dtype=dtype, masked_prob=0.3 if seed % 3 == 0 else 0.0)
    if dtype == "f32" and g > 16:
        spec = workloads.random_tree(1000 + seed, max_nodes=8, max_len=300, max_queries=12, num_q_heads=hkv * 4,
                                     num_kv_heads=hkv, head_dim=d, dtype=dtype)
    say(f"random tree seed {seed}: dtype {spec.dtype} H {spec.num_q_heads}/{spec.num_kv_heads} d {spec.head_dim} "
        f"N {spec.num_nodes} B {spec.num_queries}")
    t, plan, out, lse = run(spec, num_bins=int(rng.choice([0, 3, 17])), dot_small=seed % 2 == 1)
    check(spec, t, out, lse)


@pytest.mark.parametrize("rows", [1, 2, 4, 8, 12, 15, 16, 17, 31, 32, 33, 48, 63, 64, 65, 100, 128, 129, 200, 256])
def test_row_counts_single_node(rows):
    """One node shared by `rows` MQA rows (g = rows, one query): every row bucket and a ragged tail."""
    spec = workloads.TreeSpec(f"rows{rows}", np.array([-1]), np.array([1000]), np.array([0]), np.array([0]),
                              rows, 1, 128, "bf16", 77)
    say(f"rows {rows}")
    t, plan, out, lse = run(spec, num_bins=5)
    check(spec, t, out, lse)


@pytest.mark.parametrize("rows", [3, 16, 33, 40, 64, 100, 128, 200, 256])
def test_row_counts_head_dim_64(rows):
    """Head dim 64: 128-token tiles, so every wavefront runs several 32-token sub-steps per tile."""
    spec = workloads.TreeSpec(f"rows{rows}-d64", np.array([-1]), np.array([1000]), np.array([0]), np.array([0]),
                              rows, 1, 64, "bf16", 79)
    say(f"rows {rows} at head dim 64")
    t, plan, out, lse = run(spec, num_bins=5)
    check(spec, t, out, lse)


@pytest.mark.parametrize("rows", [1, 2, 4, 8, 12, 15])
def test_row_counts_dot_path(rows):
    """The wavefront dot-product path for bf16 pieces below 16 rows (PST_PLAN_DOT_SMALL)."""
    spec = workloads.TreeSpec(f"rows{rows}-dot", np.array([-1]), np.array([1000]), np.array([0]), np.array([0]),
                              rows, 1, 128, "bf16", 78)
    say(f"rows {rows} on the dot-product path")
    t, plan, out, lse = run(spec, num_bins=5, dot_small=True)
    assert plan.view()["mfma_min_rows"] == 16
    check(spec, t, out, lse)


@pytest.mark.parametrize("rows", [16, 100, 256])
def test_reference_raised_mid_piece(rows):
    """K grows eightfold along one 1000-token piece, so the running maximum of
    every row rises by more than 2^8 several times after the first tile: the
    rescale of O and of the P still waiting for its products, in the
    branch-free (16, 100 rows) and the per-lane-test (256 rows) layouts."""
    spec = workloads.TreeSpec(f"ramp{rows}", np.array([-1]), np.array([1000]), np.array([0]), np.array([0]),
                              rows, 1, 128, "bf16", 81)
    q, k, v = workloads.make_tensors(spec, "cuda")
    ramp = torch.linspace(1.0, 8.0, 1000, device="cuda", dtype=torch.float32)
    k = (k.float() * ramp[None, :, None]).to(torch.bfloat16).contiguous()
    say(f"rows {rows}, K ramped x1 -> x8")
    t, plan, out, lse = run(spec, tensors=(q, k, v), num_bins=1)
    assert plan.view()["b_eff"][0] == 1  # one piece: every raise happens inside it
    check(spec, t, out, lse)


# (seed, dtype, kv heads, group, head dim, page size, dot_small, masked fraction, max rows per node)
PAGED_CASES = [
    (0, "bf16", 2, 4, 128, 16, False, 0.0, 40),
    (1, "bf16", 1, 32, 128, 64, False, 0.0, 12),   # many rows: the one-slab-per-wave layout
    (2, "bf16", 2, 4, 64, 8, False, 0.3, 40),      # head dim 64 (8 tokens per DMA block), masked nodes
    (3, "f32", 2, 4, 64, 16, False, 0.0, 12),      # float32 dot path
    (4, "f32", 1, 4, 128, 32, False, 0.3, 12),     # float32, 512-byte rows (2 tokens per DMA block)
    (5, "bf16", 4, 1, 128, 8, True, 0.3, 40),      # bf16 dot path below 16 rows
    (6, "bf16", 1, 8, 128, 128, False, 0.0, 40),   # pages longer than a tile
]


@pytest.mark.parametrize("case", PAGED_CASES, ids=[f"paged{c[0]}" for c in PAGED_CASES])
def test_paged_kv(case):
    """Paged K/V: pages scattered with holes, page tails and holes filled
    with NaN (a read past a node's end would poison the output), one spare
    page per node; the oracle reads the contiguous layout."""
    seed, dtype, hkv, g, d, P, dot_small, masked, maxq = case
    spec = workloads.random_tree(2000 + seed, max_nodes=8, max_len=700, max_queries=maxq, num_q_heads=hkv * g,
                                 num_kv_heads=hkv, head_dim=d, dtype=dtype, masked_prob=masked)
    say(f"paged case {seed}: page {P} dtype {dtype} H {hkv * g}/{hkv} d {d} N {spec.num_nodes} B {spec.num_queries}")
    q, k, v = workloads.make_tensors(spec, "cuda")
    paged, kp, vp = workloads.page_pools(spec, k, v, P, spare_pages=1)
    tree = pst.Tree.from_paged(spec, paged, out_dtype="f32")
    plan = pst.Plan(tree, num_bins=5, dot_small=dot_small)
    out, lse = pst.decode_attn(plan, q, kp, vp)
    torch.cuda.synchronize()
    check(spec, (q, k, v), out, lse)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_paged_pages_example(dtype):
    """The shared-prefix blog's paged layout (section 4.3; tests/golden): the
    96-token prefix in pages 0-5, the suffixes in pages 6 and 7 of a 16-token
    page pool, one decode query per request."""
    import json
    import os

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    with open(os.path.join(root, "tests", "golden", "flashinfer_paged_prefix_96_4_4.json")) as f:
        g = json.load(f)
    tr, P = g["tree"], g["page_size"]
    lens = np.array(tr["kv_len"])
    spec = workloads.TreeSpec("pages-example", np.array(tr["parent"]), lens, np.concatenate([[0], np.cumsum(lens)[:-1]]),
                              np.array(tr["query_node"]), 8, 2, 128, dtype, 43)
    q, k, v = workloads.make_tensors(spec, "cuda")
    # The pool as the page lays it out: node i's token j at page_idx[page_ptr[i] + j // P] * P + j % P.
    kp = torch.full((2, 8 * P, 128), float("nan"), dtype=k.dtype, device="cuda")
    vp = torch.full_like(kp, float("nan"))
    for i in range(3):
        for j in range(int(lens[i])):
            row = tr["page_idx"][tr["page_ptr"][i] + j // P] * P + j % P
            kp[:, row] = k[:, int(spec.kv_offset[i]) + j]
            vp[:, row] = v[:, int(spec.kv_offset[i]) + j]
    tree = pst.Tree(tr["parent"], None, tr["kv_len"], tr["query_node"], num_q_heads=8, num_kv_heads=2, head_dim=128,
                    dtype=dtype, out_dtype="f32", page_size=P, page_ptr=tr["page_ptr"], page_idx=tr["page_idx"])
    for kw in ({}, {"flatten": 128}):
        plan = pst.Plan(tree, num_bins=2, **kw)
        out, lse = pst.decode_attn(plan, q, kp, vp)
        torch.cuda.synchronize()
        check(spec, (q, k, v), out, lse)


@pytest.mark.parametrize("P", [128, 256, 1024])
@pytest.mark.parametrize("dot_small", [False, True])
def test_paged_tiles_off_page_boundaries(P, dot_small):
    """Head dim 64 (128-token tiles) over pages of at least a tile, with
    pieces of 192 tokens: pieces start at 64 mod 128, so their tiles straddle
    page boundaries and must take the per-block page lookups."""
    spec = workloads.random_tree(2500 + P, max_nodes=6, max_len=1500, min_len=300, max_queries=12,
                                 num_q_heads=8, num_kv_heads=2, head_dim=64, dtype="bf16")
    q, k, v = workloads.make_tensors(spec, "cuda")
    paged, kp, vp = workloads.page_pools(spec, k, v, P, spare_pages=1)
    tree = pst.Tree.from_paged(spec, paged, out_dtype="f32")
    plan = pst.Plan(tree, num_bins=5, fixed_chunk=192, dot_small=dot_small)
    assert any(int(t[2]) % 128 == 64 for t in plan.view()["tasks"])
    out, lse = pst.decode_attn(plan, q, kp, vp)
    torch.cuda.synchronize()
    check(spec, (q, k, v), out, lse)


@pytest.mark.parametrize("name,P", [("2", 16), ("4", 8)])
def test_paged_config_sampled(name, P):
    """A full workload over a paged pool (document QA; masked speculative drafts), sampled queries."""
    spec = workloads.config(name)
    q, k, v = workloads.make_tensors(spec, "cuda")
    paged, kp, vp = workloads.page_pools(spec, k, v, P)
    say(f"config {name} paged by {P}: {paged['page_ptr'][-1]} pages")
    tree = pst.Tree.from_paged(spec, paged, out_dtype="f32")
    plan = pst.Plan(tree)
    out, lse = pst.decode_attn(plan, q, kp, vp)
    torch.cuda.synchronize()
    del kp, vp
    check(spec, (q, k, v), out, lse, queries=sample(spec.num_queries, 16, 11))


def test_paged_config5_mha():
    """The largest workload over 16-token pages: the paged pools hold ~43 GB,
    so per-head bases lie beyond 2^32 bytes while page rows and tile offsets
    stay 32-bit; bf16 output (fp16 partials) as the bench runs it.  One query
    for every fourth node with queries, so every level of the tree is
    checked."""
    spec = workloads.config("5-mha")
    q, k, v = workloads.make_tensors(spec, "cuda")
    paged, kp, vp = workloads.page_pools(spec, k, v, 16)
    say(f"config 5-mha paged by 16: {paged['page_ptr'][-1]} pages, pool {kp.shape[1]} rows per head")
    tree = pst.Tree.from_paged(spec, paged)
    plan = pst.Plan(tree)
    out, lse = pst.decode_attn(plan, q, kp, vp)
    torch.cuda.synchronize()
    del kp, vp, tree, plan
    queries = per_leaf_queries(spec)[::4]
    say(f"  checking {len(queries)} queries")
    check(spec, (q, k, v), out, lse, queries=queries, by_node=True)


FLAT_CASES = [
    # seed, dtype, H_kv, g, d, chunk, page (0 = contiguous), masked fraction, max queries, dot_small
    (0, "bf16", 2, 4, 128, 128, 0, 0.0, 40, False),
    (1, "bf16", 1, 32, 128, 256, 0, 0.0, 12, False),   # many rows: the one-slab-per-wave layout
    (2, "bf16", 2, 4, 64, 256, 0, 0.4, 40, False),     # head dim 64 (128-token tiles, two mask words), masked nodes
    (3, "f32", 2, 4, 64, 128, 0, 0.0, 12, False),      # float32 dot path
    (4, "f32", 1, 4, 128, 384, 0, 0.4, 12, False),     # float32, 32-token tiles
    (5, "bf16", 4, 1, 128, 512, 0, 0.4, 40, True),     # bf16 dot path below 16 rows
    (6, "bf16", 2, 8, 128, 1024, 0, 0.0, 40, False),   # 16 mask words: few entries per row group
    (7, "bf16", 2, 4, 128, 256, 16, 0.4, 40, False),   # paged pool (NaN in page tails and holes)
    (8, "f32", 2, 4, 128, 128, 8, 0.0, 12, False),     # paged, float32
]


@pytest.mark.parametrize("case", FLAT_CASES, ids=[f"flat{c[0]}" for c in FLAT_CASES])
def test_flatten_parity(case):
    """DEFT-Flatten partition: chunks span nodes, every tile takes the bit
    causal mask test, K/V rows come from the row table."""
    seed, dtype, hkv, g, d, chunk, P, masked, maxq, dot_small = case
    spec = workloads.random_tree(3000 + seed, max_nodes=10, max_len=700, max_queries=maxq, num_q_heads=hkv * g,
                                 num_kv_heads=hkv, head_dim=d, dtype=dtype, masked_prob=masked)
    say(f"flat case {seed}: chunk {chunk} page {P} dtype {dtype} H {hkv * g}/{hkv} d {d} "
        f"N {spec.num_nodes} B {spec.num_queries}")
    q, k, v = workloads.make_tensors(spec, "cuda")
    if P:
        paged, kp, vp = workloads.page_pools(spec, k, v, P, spare_pages=1)
        tree = pst.Tree.from_paged(spec, paged, out_dtype="f32")
    else:
        kp, vp = k, v
        tree = pst.Tree.from_spec(spec, out_dtype="f32")
    plan = pst.Plan(tree, num_bins=6, flatten=chunk, dot_small=dot_small,
                    max_rows=16 if dtype == "f32" else 0)
    out, lse = pst.decode_attn(plan, q, kp, vp)
    torch.cuda.synchronize()
    check(spec, (q, k, v), out, lse)


@pytest.mark.parametrize("name,chunk", [("1", 256), ("3", 512), ("4", 256), ("2", 1024), ("5-mqa", 256)])
def test_flatten_config(name, chunk):
    """Whole workloads under the flattened partition, checked against the
    oracle (sampled queries on the large ones) and against the cost-model
    plan's output."""
    spec = workloads.config(name)
    q, k, v = workloads.make_tensors(spec, "cuda")
    tree = pst.Tree.from_spec(spec, out_dtype="f32")
    flat = pst.Plan(tree, flatten=chunk)
    say(f"config {name} flattened by {chunk}: {flat.view()['num_chunks']} chunks, {len(flat.view()['tasks'])} tasks")
    out, lse = pst.decode_attn(flat, q, k, v)
    ref, rlse = pst.decode_attn(pst.Plan(tree), q, k, v)
    torch.cuda.synchronize()
    queries = list(range(spec.num_queries)) if spec.num_queries <= 16 else sample(spec.num_queries, 16, 5)
    check(spec, (q, k, v), out, lse, queries=queries)
    tol = TOL[spec.dtype]
    assert (out - ref).abs().max().item() <= 2 * tol
    assert (lse - rlse).abs().max().item() <= 8 * max(tol, 1e-5)


def test_graph_capture_replays():
    """PAC + POR captured in a graph (several layers' worth, as a decode step
    would be): the calls allocate nothing and set no memory, so every replay,
    with eager work and synchronisation between them, equals the eager
    result bit for bit."""
    spec = workloads.config("3")
    q, k, v = workloads.make_tensors(spec, "cuda")
    tree = pst.Tree.from_spec(spec, out_dtype="f32")
    plan = pst.Plan(tree)
    ws = pst.workspace(plan)
    out = torch.empty((spec.num_queries, spec.num_q_heads, spec.head_dim), device="cuda")
    lse = torch.empty((spec.num_queries, spec.num_q_heads), device="cuda")
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        pst.decode_attn(plan, q, k, v, out=out, lse=lse, ws=ws)
    s.synchronize()
    ref, rlse = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for _ in range(4):
            pst.pac(plan, q, k, v, ws, stream=s)
            pst.por(plan, out, lse, ws, stream=s)
    for rep in range(5):
        out.fill_(float("nan"))
        lse.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        say(f"  replay {rep}: max|dO| {(out - ref).abs().max().item():.1e}")
        assert torch.equal(out, ref) and torch.equal(lse, rlse)
    check(spec, (q, k, v), out, lse, queries=sample(spec.num_queries, 8, 3))


def test_injected_allocation_failure():
    """A device allocation forced to fail from the host (PST_FAULT_INJECT,
    read once per process, so in a child): the tree builds, the plan's
    upload fails with PST_E_OOM and a message, and the process then plans
    and decodes normally."""
    import os
    import subprocess

    code = """
import sys
sys.path.insert(0, {root!r})
import torch, numpy as np
import prefix_shared_tree_amd as pst, workloads
spec = workloads.config("1")
q, k, v = workloads.make_tensors(spec, "cuda")
tree = pst.Tree.from_spec(spec, out_dtype="f32")          # allocation 1
try:
    pst.Plan(tree)                                         # allocation 2: injected failure
    print("NO-ERROR")
except pst.PstError as e:
    print("ERR", e.code, str(e))
plan = pst.Plan(tree)                                      # allocation 3
out, lse = pst.decode_attn(plan, q, k, v)
torch.cuda.synchronize()
print("OK", float(out.abs().sum()) > 0)
""".format(root=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    env = dict(os.environ, PST_FAULT_INJECT="alloc:2")
    r = subprocess.run([sys.executable, "-c", code], env=env, capture_output=True, text=True, timeout=100)
    say(r.stdout.strip())
    assert r.returncode == 0, r.stderr[-2000:]
    assert "ERR PST_E_OOM" in r.stdout and "injected device allocation failure" in r.stdout
    assert "OK True" in r.stdout


@pytest.mark.parametrize("seed", range(64))
def test_random_configurations(seed):
    """Random combinations of dtype, GQA group, head dim, tree shape, masked
    nodes, paged pools, bin count, row cap, dot path and partition (cost
    model, fixed or odd chunks, one piece per node, flattened), all queries
    against the oracle."""
    rng = np.random.default_rng(10000 + seed)
    dtype = "f32" if rng.random() < 0.25 else "bf16"
    hkv = int(rng.choice([1, 2, 4]))
    g = int(rng.choice([1, 2, 4, 8, 16, 32] if dtype == "bf16" else [1, 2, 4]))
    d = int(rng.choice([64, 128]))
    spec = workloads.random_tree(70000 + seed, max_nodes=int(rng.choice([3, 8, 16])),
                                 max_len=int(rng.choice([20, 200, 1500])), max_queries=int(rng.choice([2, 8, 24])),
                                 num_q_heads=hkv * g, num_kv_heads=hkv, head_dim=d, dtype=dtype,
                                 masked_prob=float(rng.choice([0.0, 0.3])))
    q, k, v = workloads.make_tensors(spec, "cuda")
    P = int(rng.choice([0, 0, 8, 16, 64, 128, 256, 512]))
    # The output dtype from a generator of its own (the other draws stay as they were).
    odt = "bf16" if dtype == "bf16" and np.random.default_rng(20000 + seed).random() < 0.5 else "f32"
    if P:
        paged, kk, vv = workloads.page_pools(spec, k, v, P, spare_pages=int(rng.integers(0, 2)))
        tree = pst.Tree.from_paged(spec, paged, out_dtype=odt)
    else:
        kk, vv = k, v
        tree = pst.Tree.from_spec(spec, out_dtype=odt)
    kw = dict(num_bins=int(rng.choice([0, 1, 3, 7, 32])), dot_small=bool(rng.random() < 0.3))
    if dtype == "bf16" and g <= 32 and rng.random() < 0.25:
        kw["max_rows"] = int(rng.choice([32, 64, 128]))
    u = rng.random()
    if u < 0.2:
        kw["fixed_chunk"] = int(rng.choice([64, 128, 192, 320, 512]))
    elif u < 0.45:
        kw["flatten"] = int(rng.choice([128, 256, 384, 640]))
    elif u < 0.55:
        kw["no_split"] = True
    say(f"seed {seed}: {dtype} (out {odt}) H {hkv * g}/{hkv} d {d} N {spec.num_nodes} B {spec.num_queries} page {P} {kw}")
    plan = pst.Plan(tree, **kw)
    out, lse = pst.decode_attn(plan, q, kk, vv)
    torch.cuda.synchronize()
    check(spec, (q, k, v), out, lse)


def test_max_rows_split():
    """More rows than one workgroup holds: the planner cuts row groups (> 256 rows)."""
    lens = [700] + [3] * 20
    spec = workloads.TreeSpec("rowgroups", np.array([-1] + [0] * 20), np.array(lens),
                              np.concatenate([[0], np.cumsum(lens)[:-1]]), np.arange(1, 21), 32, 1, 128, "bf16", 8)
    t, plan, out, lse = run(spec, num_bins=9)
    assert plan.view()["rows_per_group"][0] < 20 * 32
    check(spec, t, out, lse)


def test_bf16_output_rounding():
    """bf16 output: every query against the oracle (one bf16 ulp beyond the
    tolerance), and within one ulp plus the fp16 partials' rounding (2^-11
    of the largest partial, bounded by max|V|) of the float32-output run."""
    spec = workloads.config("3")
    t, plan, out_bf, lse_bf = run(spec, out_dtype="bf16")
    _, _, out32, lse32 = run(spec, tensors=t)
    assert out_bf.dtype == torch.bfloat16
    check(spec, t, out_bf, lse_bf)
    vmax = float(t[2].float().abs().max())
    ulp = torch.exp2(torch.floor(torch.log2(out32.abs().clamp_min(1e-38))) - 7)
    assert ((out_bf.float() - out32).abs() - ulp).max().item() <= 2.0 ** -10 * vmax
    assert torch.equal(lse_bf, lse32) or (lse_bf - lse32).abs().max().item() <= 1e-5


# Two nodes per query whose V differ in scale by 2^(2 s): the partials of one
# query carry different fp16 scales into the merge.
@pytest.mark.parametrize("s", [6, 20])
def test_bf16_output_mixed_scales(s):
    """bf16 output, partials in fp16 with their own power-of-two scale: a
    root whose V is scaled by 2^s and leaves scaled by 2^-s, peaked queries
    (q x 8), so every query merges partials of very different magnitude.
    Each (query, head) is held to a tolerance weighted by how much each node
    contributes (its merge weight from the float64 partials), so a wrong
    scale on either partial shows."""
    lens = [1500] + [300] * 6
    spec = workloads.TreeSpec(f"mixed{s}", np.array([-1] + [0] * 6), np.array(lens),
                              np.concatenate([[0], np.cumsum(lens)[:-1]]), np.repeat(np.arange(1, 7), 3),
                              16, 2, 128, "bf16", 91)
    q, k, v = workloads.make_tensors(spec, "cuda", q_scale=8.0)
    f = torch.full((spec.total_tokens,), 2.0 ** -s, device="cuda")
    f[:1500] = 2.0 ** s
    v = (v.float() * f[None, :, None]).to(torch.bfloat16).contiguous()
    t, plan, out, lse = run(spec, out_dtype="bf16", tensors=(q, k, v), num_bins=5)
    _, _, out32, _ = run(spec, tensors=(q, k, v), num_bins=5)
    assert plan.view()["num_slots"] > spec.num_queries  # merges happen
    O, _ = oracle.attend(spec, q, k, v)
    qh, kh, vh = (x.double().cpu().numpy() for x in (q, k, v))
    g = spec.num_q_heads // spec.num_kv_heads
    scale = 1.0 / math.sqrt(spec.head_dim)
    vmax = np.abs(vh).max(axis=2)  # [H_kv, T]
    bound = np.zeros((spec.num_queries, spec.num_q_heads))
    for r, n in enumerate(spec.query_node):
        lo, hi = int(spec.kv_offset[n]), int(spec.kv_offset[n] + spec.kv_len[n])
        for h in range(spec.num_q_heads):
            kv = h // g
            parts = [(0, 1500), (lo, hi)]
            lses = [oracle.partial_attend(qh[r, h][None], kh[kv, a:b], vh[kv, a:b], scale)[3][0] for a, b in parts]
            top = max(lses)
            w = np.exp(np.array(lses) - top)
            w /= w.sum()
            bound[r, h] = sum(wi * vmax[kv, a:b].max() for wi, (a, b) in zip(w, parts))
    got = out.double().cpu().numpy()
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(O), 1e-38))) - 7)
    excess = (np.abs(got - O) - ulp - TOL["bf16"] * bound[:, :, None]).max()
    say(f"  mixed scales 2^+-{s}: largest excess over the weighted bound {excess:.3e}")
    assert excess <= 0.0
    o32 = out32.double().cpu().numpy()
    ulp32 = np.exp2(np.floor(np.log2(np.maximum(np.abs(o32), 1e-38))) - 7)
    assert (np.abs(got - o32) - ulp32 - 2.0 ** -10 * bound[:, :, None]).max() <= 0.0


def test_query_guided_baseline():
    spec = workloads.config("3")
    t, plan, out, lse = run(spec, query_guided=True)
    v = plan.view()
    assert (v["tasks"][:, 5] == spec.group).all()
    check(spec, t, out, lse, queries=sample(128, 32, 3))


@pytest.mark.parametrize("name", ["2", "3", "4"])
def test_baseline_entry_point(name):
    """pst_decode_attn_baseline (shared nodes read once per query) on the
    document-QA, few-shot and speculative trees: against the oracle, and equal
    to a query-guided plan run through pst_decode_attn."""
    spec = workloads.config(name)
    say(f"baseline entry point, config {name}: {spec.name}")
    q, k, v = workloads.make_tensors(spec, "cuda")
    tree = pst.Tree.from_spec(spec, out_dtype="f32")
    out, lse = pst.decode_attn_baseline(tree, q, k, v)
    out2, lse2 = pst.decode_attn_baseline(tree, q, k, v)  # the tree's plan, reused
    plan = pst.Plan(tree, query_guided=True)
    out3, lse3 = pst.decode_attn(plan, q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    assert torch.equal(out, out3) and torch.equal(lse, lse3)
    if name == "4":
        queries = config4_queries(spec, extra=16)
    elif name == "2":
        queries = list(range(spec.num_queries))
    else:
        queries = sample(spec.num_queries, 32, 3)
    check(spec, (q, k, v), out, lse, queries=queries, by_node=name == "2")


@pytest.mark.parametrize("kw", [dict(no_split=True), dict(fixed_chunk=256), dict(num_bins=1)])
def test_plan_variants(kw):
    spec = workloads.config("3")
    t, plan, out, lse = run(spec, **kw)
    check(spec, t, out, lse, queries=sample(128, 16, 4))


def test_deterministic():
    spec = workloads.config("3")
    t, plan, out1, lse1 = run(spec)
    out2, lse2 = pst.decode_attn(plan, *t)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_plan_reuse_after_growth():
    spec = workloads.config("3")
    q, k, v = workloads.make_tensors(spec, "cuda", kv_tokens=spec.total_tokens + 64)
    tree = pst.Tree.from_spec(spec, out_dtype="f32", pool_tokens=spec.total_tokens + 64)
    plan = pst.Plan(tree)
    lens = spec.kv_len.copy()
    lens[-1] += 50  # the last leaf is the last run of the pool: it can grow in place
    tree.set_lengths(lens)
    out, lse = pst.decode_attn(plan, q, k, v)
    torch.cuda.synchronize()
    grown = workloads.TreeSpec("grown", spec.parent, lens, spec.kv_offset, spec.query_node, 32, 8, 128, "bf16", 3)
    check(grown, (q, k, v), out, lse, queries=[0, 126, 127])


def test_peaked_attention():
    """Queries scaled by 8 make attention peaked (a few tokens carry most of
    the weight): the bf16 tolerance still holds."""
    spec = workloads.config("3")
    t, plan, out, lse = run(spec, q_scale=8.0)
    check(spec, t, out, lse, queries=sample(128, 16, 5))


# (rows, V scale, V ramp along the piece (first, last factor))
VSCALE_CASES = [
    (4, 2.0 ** -12, None), (4, 2.0 ** 12, None),
    (100, 2.0 ** -12, None), (100, 2.0 ** 12, None),
    (256, 2.0 ** -12, None), (256, 2.0 ** 12, None),
    (4, 1.0, (2.0 ** -20, 2.0 ** 10)),    # |V| grows along the piece: the fp16 scale is raised tile after tile
    (100, 1.0, (2.0 ** -20, 2.0 ** 10)),
    (256, 1.0, (2.0 ** -20, 2.0 ** 10)),
    (256, 1.0, (2.0 ** 10, 2.0 ** -20)),  # |V| shrinks: later tiles convert below the first tile's scale
    (16, 2.0 ** -60, None),
    (16, 2.0 ** 60, None),
]


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
@pytest.mark.parametrize("rows,vscale,ramp", VSCALE_CASES)
def test_v_magnitudes(rows, vscale, ramp, out_dtype):
    """V far from unit scale, under peaked attention (q x 8), on one
    1000-token node of `rows` MQA rows (every matrix-core layout): the
    max-abs error stays within the bf16 tolerance relative to max|V|; with a
    bf16 output the fp16 partial carries the piece's scale to the merge."""
    spec = workloads.TreeSpec(f"vscale{rows}", np.array([-1]), np.array([1000]), np.array([0]), np.array([0]),
                              rows, 1, 128, "bf16", 83)
    q, k, v = workloads.make_tensors(spec, "cuda", q_scale=8.0)
    f = torch.full((1000,), vscale, device="cuda", dtype=torch.float32)
    if ramp is not None:
        f = torch.logspace(math.log2(ramp[0]), math.log2(ramp[1]), 1000, base=2.0, device="cuda")
    v = (v.float() * f[None, :, None]).to(torch.bfloat16).contiguous()
    vmax = float(v.float().abs().max())
    say(f"rows {rows}, V x {vscale:g}, ramp {ramp}, max|V| {vmax:.3e}")
    t, plan, out, lse = run(spec, tensors=(q, k, v), num_bins=1, out_dtype=out_dtype)
    assert plan.view()["b_eff"][0] == 1  # one piece: every raise of the scale happens inside it
    check(spec, t, out, lse, tol=TOL["bf16"] * vmax, lse_tol=4 * TOL["bf16"])


def test_empty_batch_and_single_token():
    spec = workloads.TreeSpec("empty", np.array([-1]), np.array([5]), np.array([0]), np.zeros(0, dtype=np.int32),
                              4, 4, 64, "f32", 1)
    q = torch.zeros((0, 4, 64), device="cuda")
    k = torch.randn((4, 5, 64), device="cuda")
    tree = pst.Tree.from_spec(spec, out_dtype="f32")
    plan = pst.Plan(tree)
    out, lse = pst.decode_attn(plan, q, k, k)
    torch.cuda.synchronize()
    assert out.shape == (0, 4, 64)
    spec1 = workloads.TreeSpec("one", np.array([-1]), np.array([1]), np.array([0]), np.array([0, 0]), 8, 2, 128,
                               "bf16", 2)
    t, plan, out, lse = run(spec1)
    check(spec1, t, out, lse)


def test_token_major_strides():
    """K/V pools in [T, H_kv, d] layout through the stride arguments."""
    spec = workloads.config("3")
    q, k, v = workloads.make_tensors(spec, "cuda")
    kt = k.permute(1, 0, 2).contiguous()
    vt = v.permute(1, 0, 2).contiguous()
    tree = pst.Tree.from_spec(spec, out_dtype="f32", kv_stride_head=128, kv_stride_token=8 * 128)
    plan = pst.Plan(tree)
    out, lse = pst.decode_attn(plan, q, kt, vt)
    torch.cuda.synchronize()
    check(spec, (q, k, v), out, lse, queries=sample(128, 16, 6))


def test_workspace_errors():
    spec = workloads.config("1")
    q, k, v = workloads.make_tensors(spec, "cuda")
    tree = pst.Tree.from_spec(spec, out_dtype="f32")
    plan = pst.Plan(tree)
    small = torch.empty(64, dtype=torch.uint8, device="cuda")
    with pytest.raises(pst.PstError) as e:
        pst.decode_attn(plan, q, k, v, ws=small)
    assert e.value.code == "PST_E_WORKSPACE"


@pytest.mark.parametrize("replan_every", [0, 2])
def test_decode_session_steps(replan_every):
    """Multi-step decoding: each step appends one token to every query's leaf
    (paged pool, plan reused through pst_tree_set_lengths, or re-planned every
    second step) and is checked against the oracle on a contiguous mirror."""
    from prefix_shared_tree_amd.decode_loop import DecodeSession

    parent = np.array([-1, 0, 0, 0, 1, 1, 2, 2, 3, 3])
    lens = np.array([700, 100, 37, 64, 40, 1, 63, 16, 9, 70])
    qnode = np.array([4, 5, 6, 7, 8, 9])
    steps = 6
    cap = lens.copy()
    cap[qnode] += steps
    off = np.concatenate([[0], np.cumsum(cap)[:-1]])
    spec0 = workloads.TreeSpec("decode", parent, lens, off, qnode, 16, 4, 128, "bf16", 91)
    q, k, v = workloads.make_tensors(spec0, "cuda", kv_tokens=int(cap.sum()))
    sess = DecodeSession(spec0, k, v, page_size=16, max_new_tokens=steps, replan_every=replan_every,
                         plan_kw=dict(num_bins=3))
    g = torch.Generator(device="cuda")
    g.manual_seed(4242 + replan_every)
    cur = lens.copy()
    for s in range(steps):
        kn = torch.randn((len(qnode), 4, 128), generator=g, device="cuda").to(torch.bfloat16)
        vn = torch.randn((len(qnode), 4, 128), generator=g, device="cuda").to(torch.bfloat16)
        sess.append(kn, vn)
        rows = torch.from_numpy(off[qnode] + cur[qnode]).cuda()
        k[:, rows] = kn.transpose(0, 1)
        v[:, rows] = vn.transpose(0, 1)
        cur[qnode] += 1
        spec = workloads.TreeSpec("decode", parent, cur, off, qnode, 16, 4, 128, "bf16", 91)
        qs = torch.randn((len(qnode), 16, 128), generator=g, device="cuda").to(torch.bfloat16)
        out, lse = sess.decode(qs)
        torch.cuda.synchronize()
        say(f"step {s + 1}: lengths {cur[qnode].tolist()}, replans {sess.replans}")
        check(spec, (qs, k, v), out, lse)
    assert sess.replans == (steps // replan_every if replan_every else 0)


@pytest.mark.gpu
def test_decode_session_flatten():
    """A decode session under the DEFT-Flatten partition: appends re-plan
    every step, forks and finishes rebuild; each step against the oracle."""
    from prefix_shared_tree_amd.decode_loop import DecodeSession

    parent = np.array([-1, 0, 0, 1])
    lens = np.array([300, 90, 7, 64])
    off = np.concatenate([[0], np.cumsum(lens)[:-1]])
    spec0 = workloads.TreeSpec("flatdecode", parent, lens, off, np.array([2, 3]), 16, 4, 128, "bf16", 23)
    q, k, v = workloads.make_tensors(spec0, "cuda")
    sess = DecodeSession(spec0, k, v, page_size=16, max_new_tokens=6, extra_pages=40,
                         plan_kw=dict(num_bins=4, flatten=128))
    g = torch.Generator(device="cuda")
    g.manual_seed(7)

    def rows(n):
        return torch.randn((n, 4, 128), generator=g, device="cuda").to(torch.bfloat16)

    for op in ["a", "b2", "a", "a", "p0", "a"]:
        if op == "a":
            sess.append(rows(sess.num_queries), rows(sess.num_queries))
        elif op[0] == "b":
            sess.branch(0, rows(int(op[1])), rows(int(op[1])))
        else:
            sess.prune(int(op[1]))
        parent, kv_len, koff, qn, kc, vc = sess.contiguous()
        spec = workloads.TreeSpec("flatdecode", parent, kv_len, koff, qn, 16, 4, 128, "bf16", 23)
        qs = torch.randn((sess.num_queries, 16, 128), generator=g, device="cuda").to(torch.bfloat16)
        out, lse = sess.decode(qs)
        torch.cuda.synchronize()
        assert sess.plan.view()["flat_chunk"] == 128
        say(f"{op}: {sess.num_queries} queries, {len(kv_len)} nodes, replans {sess.replans}")
        check(spec, (qs, kc, vc), out, lse)


@pytest.mark.gpu
def test_decode_session_branch_prune():
    """Tree search over a paged pool: queries grow, fork and finish; after every
    change each query's attention is checked against the oracle on the tree the
    session holds, gathered back to the contiguous layout."""
    from prefix_shared_tree_amd.decode_loop import DecodeSession

    parent = np.array([-1, 0, 0, 1])
    lens = np.array([900, 130, 7, 64])
    off = np.concatenate([[0], np.cumsum(lens)[:-1]])
    spec0 = workloads.TreeSpec("search", parent, lens, off, np.array([2, 3]), 16, 4, 128, "bf16", 17)
    q, k, v = workloads.make_tensors(spec0, "cuda")
    sess = DecodeSession(spec0, k, v, page_size=16, max_new_tokens=8, extra_pages=80, plan_kw=dict(num_bins=5))
    g = torch.Generator(device="cuda")
    g.manual_seed(99)

    def rows(n):
        return torch.randn((n, 4, 128), generator=g, device="cuda").to(torch.bfloat16)

    for op in ["a", "b3", "a", "b2", "a", "p1", "a", "b1", "p0", "a", "p2"]:
        if op == "a":
            B = sess.num_queries
            sess.append(rows(B), rows(B))
        elif op[0] == "b":
            n = int(op[1])
            sess.branch(sess.num_queries - 1, rows(n), rows(n))
        else:
            sess.prune(int(op[1]))
        parent, kv_len, koff, qn, kc, vc = sess.contiguous()
        spec = workloads.TreeSpec("search", parent, kv_len, koff, qn, 16, 4, 128, "bf16", 17)
        qs = torch.randn((sess.num_queries, 16, 128), generator=g, device="cuda").to(torch.bfloat16)
        out, lse = sess.decode(qs)
        torch.cuda.synchronize()
        say(f"{op}: {sess.num_queries} queries, {len(kv_len)} nodes, {len(sess.free)} free pages")
        check(spec, (qs, kc, vc), out, lse)


@pytest.mark.parametrize("rows", [4, 256])
def test_v_zero_tiles_then_values(rows):
    """The first 300 tokens of V are zero (the fp16 scale stays at its start
    value over several tiles), then V ~ N(0, 1) x 2^20: the scale is raised
    with O already accumulated."""
    spec = workloads.TreeSpec(f"vzero{rows}", np.array([-1]), np.array([1000]), np.array([0]), np.array([0]),
                              rows, 1, 128, "bf16", 85)
    q, k, v = workloads.make_tensors(spec, "cuda", q_scale=4.0)
    v = (v.float() * 2.0 ** 20).to(torch.bfloat16)
    v[:, :300] = 0
    v = v.contiguous()
    vmax = float(v.float().abs().max())
    t, plan, out, lse = run(spec, tensors=(q, k, v), num_bins=1)
    check(spec, t, out, lse, tol=TOL["bf16"] * vmax, lse_tol=4 * TOL["bf16"])


@pytest.mark.parametrize("dtype,hkv,d", [("bf16", 8, 128), ("f32", 2, 64), ("bf16", 1, 64)])
def test_write_kv_rows(dtype, hkv, d):
    """pst_write_kv_rows puts row i of k_new/v_new at pool token rows[i] of
    every kv head (as an index_put would) and leaves rows outside the pools alone."""
    T = 300
    spec = workloads.TreeSpec("rows", np.array([-1]), np.array([T]), np.array([0]), np.array([0]), hkv * 2, hkv, d,
                              dtype, 91)
    _, k, v = workloads.make_tensors(spec, "cuda")
    tree = pst.Tree.from_spec(spec)
    n = 7
    g = torch.Generator(device="cuda")
    g.manual_seed(3)
    kn = torch.randn((n, hkv, d), generator=g, device="cuda").to(k.dtype)
    vn = torch.randn((n, hkv, d), generator=g, device="cuda").to(k.dtype)
    rows = torch.tensor([5, 0, 299, 17, -1, 300, 123], dtype=torch.int64, device="cuda")
    want_k, want_v = k.clone(), v.clone()
    keep = (rows >= 0) & (rows < T)
    want_k[:, rows[keep]] = kn[keep].transpose(0, 1)
    want_v[:, rows[keep]] = vn[keep].transpose(0, 1)
    pst.write_kv_rows(tree, kn, vn, rows, k, v)
    torch.cuda.synchronize()
    assert torch.equal(k, want_k) and torch.equal(v, want_v)


@pytest.mark.parametrize("page_size", [0, 16])
def test_tree_append_steps(page_size):
    """pst_tree_append: five decode steps grow two leaves (contiguous pools
    with room, or pages with a spare page each); after every step the plan,
    made once, still gives the oracle's attention over the grown tree."""
    lens = np.array([100, 30, 50])
    off = np.array([0, 100, 200])
    spec = workloads.TreeSpec("append", np.array([-1, 0, 0]), lens, off, np.array([1, 2, 1]), 8, 2, 128, "bf16", 93)
    q, k, v = workloads.make_tensors(spec, "cuda", kv_tokens=300)
    if page_size:
        paged, kk, vv = workloads.page_pools(spec, k, v, page_size, spare_pages=1)
        tree = pst.Tree.from_paged(spec, paged, out_dtype="f32")
    else:
        kk, vv = k, v
        tree = pst.Tree.from_spec(spec, out_dtype="f32", pool_tokens=300)
    plan = pst.Plan(tree, num_bins=3)
    g = torch.Generator(device="cuda")
    g.manual_seed(11)
    cur = lens.copy()
    for step in range(5):
        kn = torch.randn((2, 2, 128), generator=g, device="cuda").to(torch.bfloat16)
        vn = torch.randn((2, 2, 128), generator=g, device="cuda").to(torch.bfloat16)
        tree.append([1, 2], kn, vn, kk, vv)
        for j, node in enumerate((1, 2)):  # the contiguous mirror the oracle reads
            k[:, off[node] + cur[node]] = kn[j]
            v[:, off[node] + cur[node]] = vn[j]
        cur[1:] += 1
        out, lse = pst.decode_attn(plan, q, kk, vv)
        torch.cuda.synchronize()
        grown = workloads.TreeSpec("grown", spec.parent, cur.copy(), off, spec.query_node, 8, 2, 128, "bf16", 93)
        check(grown, (q, k, v), out, lse)
    assert tree.index()["visible"].tolist() == [int(cur[0] + cur[1]), int(cur[0] + cur[2]), int(cur[0] + cur[1])]
    with pytest.raises(pst.PstError) as e:
        tree.append([1, 1], kn, vn, kk, vv)
    assert e.value.code == "PST_E_INVALID_ARG"
    if page_size:
        # Each leaf had one spare page of 16 tokens: 30 + 5 fits in 3 pages; 11 more tokens would not.
        one = kn[:1].contiguous()
        for _ in range(48 - 35):
            tree.append([1], one, one, kk, vv)
        with pytest.raises(pst.PstError) as e:
            tree.append([1], one, one, kk, vv)
        assert e.value.code == "PST_E_INVALID_TREE"
