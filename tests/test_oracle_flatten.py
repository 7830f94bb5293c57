"""Pins of the oracle's flattened tree KV splitting (CPU only).

DEFT: Decoding with Flash Tree-Attention, section 3.3 (remark 3.1, Fig.
3(c)) and appendix A.9.  The pages print no worked example of the split, so
the flattening is pinned by what the method fixes:
* every token some query sees is in exactly one chunk, nodes in depth-first
  pre-order (each node's tokens in order, each subtree one interval, parents
  first);
* the bit causal mask of (chunk, query) is exactly the query's visibility,
  taken from the attention oracle's own definition (root-to-node path and
  the own node's mask bits), and a chunk's group is exactly the queries
  that see one of its tokens;
* partial attention of every group under its mask, merged per query by LSE,
  is the full attention (the decomposition drops and repeats nothing);
* row groups, slots and bin loads tile what they claim to; LPT keeps
  Graham's list-scheduling bound;
* the paged row table addresses the same K/V as the contiguous one.
"""
import numpy as np
import pytest

import oracle
import workloads
from oracle.flatten import dfs_order, flatten_plan

ROWS = [1, 2, 4, 8, 16, 32, 64, 128, 256]
LENS = [16 << i for i in range(13)]
TABLE = oracle.CostTable(ROWS, LENS, [[900 + 3 * r + 2 * L for L in LENS] for r in ROWS])


def _plan(spec, chunk, m=5, r_max=256, **kw):
    ix = oracle.build_index(spec)
    return ix, flatten_plan(ix, spec.parent, spec.kv_len, spec.node_masked, spec.group, TABLE, m, chunk=chunk,
                            r_max=r_max, kv_offset=spec.kv_offset, **kw)


def _specs():
    out = [workloads.random_tree(s, max_nodes=9, max_len=300, max_queries=10, num_q_heads=8, num_kv_heads=2,
                                 masked_prob=0.5 if s % 2 else 0.0) for s in range(16)]
    out += [workloads.config("1"), workloads.config("3"), workloads.config("4")]
    return out


def _mask_cases():
    small = [(s, c) for s in _specs()[:-3] for c in (128, 256, 640)]
    return small + [(s, 640) for s in _specs()[-3:]]


@pytest.mark.parametrize("spec,chunk", _mask_cases(), ids=lambda x: getattr(x, "name", str(x)))
def test_masks_are_visibility(spec, chunk):
    ix, p = _plan(spec, chunk)
    W = chunk // 64
    rows = p["flat_rows"]
    vis = [oracle.visible_tokens(spec, r) for r in range(spec.num_queries)]
    fp, fq, fm = p["flat_ptr"], p["flat_query"], p["flat_mask"]
    shifts = np.arange(64, dtype=np.uint64)
    for c in range(len(fp) - 1):
        crow = rows[c * chunk:(c + 1) * chunk]
        seen = [np.isin(crow, vis[r]) & (crow >= 0) for r in range(spec.num_queries)]
        assert fq[fp[c]:fp[c + 1]].tolist() == [r for r in range(spec.num_queries) if seen[r].any()]
        for e in range(fp[c], fp[c + 1]):
            words = fm[e * W:(e + 1) * W]
            bits = ((words[:, None] >> shifts) & np.uint64(1)).ravel().astype(bool)  # token order
            assert np.array_equal(bits, seen[int(fq[e])]), (c, int(fq[e]))


@pytest.mark.parametrize("spec", _specs(), ids=lambda s: s.name)
def test_flattening_is_a_preorder_cover(spec):
    ix, p = _plan(spec, 128)
    rows = p["flat_rows"]
    live = rows[rows >= 0]
    n_q = ix["n_q"]
    expect = [int(spec.kv_offset[i]) + j for i in range(spec.num_nodes) if n_q[i] for j in range(int(spec.kv_len[i]))]
    assert sorted(live.tolist()) == sorted(expect)  # every seen token once
    # Padding only at the end of the last chunk.
    assert (rows[:len(live)] >= 0).all() and (rows[len(live):] == -1).all()
    pos = {int(x): t for t, x in enumerate(live)}
    first = {}
    for i in range(spec.num_nodes):
        if not n_q[i]:
            continue
        ts = [pos[int(spec.kv_offset[i]) + j] for j in range(int(spec.kv_len[i]))]
        assert ts == list(range(ts[0], ts[0] + len(ts)))  # a node's tokens in order, together
        first[i] = ts[0]
    for i in first:
        par = int(spec.parent[i])
        if par >= 0:
            assert first[par] < first[i]
        # The subtree of i is one interval starting at i.
        sub = [j for j in first if _is_ancestor(spec.parent, i, j)]
        span = sorted(t for j in sub for t in range(first[j], first[j] + int(spec.kv_len[j])))
        assert span == list(range(first[i], first[i] + len(span)))
    # Siblings by increasing id.
    order = dfs_order(spec.parent, n_q)
    assert [i for i in sorted(first, key=first.get)] == order


def _is_ancestor(parent, a, b):
    while b >= 0:
        if b == a:
            return True
        b = int(parent[b])
    return False


@pytest.mark.parametrize("chunk", [128, 384])
@pytest.mark.parametrize("seed", range(8))
def test_group_partials_merge_to_attention(seed, chunk):
    spec = workloads.random_tree(seed + 100, max_nodes=7, max_len=250, max_queries=6, num_q_heads=4, num_kv_heads=2,
                                 head_dim=16, masked_prob=0.5 if seed % 2 else 0.0)
    q, k, v = workloads.make_tensors(spec, "cpu")
    ix, p = _plan(spec, chunk)
    W = chunk // 64
    O, L = oracle.attend(spec, q, k, v)
    qd, kd, vd = (x.double().numpy() for x in (q, k, v))
    scale = 1.0 / np.sqrt(spec.head_dim)
    parts = [[] for _ in range(spec.num_queries)]
    fp, fq, fm, rows = p["flat_ptr"], p["flat_query"], p["flat_mask"], p["flat_rows"]
    for c in range(len(fp) - 1):
        for e in range(fp[c], fp[c + 1]):
            r = int(fq[e])
            sel = [int(rows[c * chunk + t]) for t in range(chunk) if (int(fm[e * W + t // 64]) >> (t % 64)) & 1]
            o = np.zeros((spec.num_q_heads, spec.head_dim))
            lse = np.zeros(spec.num_q_heads)
            for h in range(spec.num_q_heads):
                kvh = h // spec.group
                ob, _, _, lb = oracle.partial_attend(qd[r, h][None], kd[kvh, sel], vd[kvh, sel], scale)
                o[h], lse[h] = ob[0], lb[0]
            parts[r].append((o, lse))
    for r in range(spec.num_queries):
        outs = np.stack([x[0] for x in parts[r]])
        lses = np.stack([x[1] for x in parts[r]])
        Om, Lm = oracle.lse_merge(outs, lses)
        np.testing.assert_allclose(Om, O[r], rtol=0, atol=1e-12)
        np.testing.assert_allclose(Lm, L[r], rtol=0, atol=1e-12)


@pytest.mark.parametrize("m,r_max", [(1, 256), (4, 8), (7, 16), (32, 256)])
@pytest.mark.parametrize("spec", _specs()[::2], ids=lambda s: s.name)
def test_row_groups_slots_and_loads(spec, m, r_max):
    if spec.group > r_max:
        pytest.skip("GQA group larger than a row group")
    chunk = 512
    ix, p = _plan(spec, chunk, m=m, r_max=r_max)
    g, W = spec.group, chunk // 64
    e_max = min(r_max // g, 1024 // W)
    fp = p["flat_ptr"]
    covered = np.zeros(int(fp[-1]), dtype=np.int32)
    items = []
    for c, piece, kb, kn, rb, rc, flags in p["tasks"]:
        assert flags == 2 and piece == 0 and kb == c * chunk and rb % g == 0 and rc % g == 0
        assert kn == min(chunk, int((p["flat_rows"][c * chunk:(c + 1) * chunk] >= 0).sum()))
        assert 1 <= rc // g <= e_max
        covered[fp[c] + rb // g:fp[c] + (rb + rc) // g] += 1
        items.append(TABLE.lookup(int(rc), int(kn)))
    assert (covered == 1).all()
    bp = p["bin_ptr"]
    for b in range(m):
        assert p["bin_load"][b] == sum(TABLE.lookup(int(t[5]), int(t[3])) for t in p["tasks"][bp[b]:bp[b + 1]])
    if items:
        assert p["makespan"] <= sum(items) / m + max(items)  # Graham: list scheduling
    # Slots: a query's entries, in chunk order, own its consecutive slots.
    sp, fq = p["slot_ptr"], p["flat_query"]
    for r in range(spec.num_queries):
        ents = [e for e in range(len(fq)) if fq[e] == r]
        assert [int(p["flat_slot"][e]) for e in ents] == list(range(int(sp[r]), int(sp[r + 1])))
        assert len(ents) >= 1


def test_single_path_closed_form():
    # One query on a chain: every chunk has that one query, all its bits set.
    parent = np.array([-1, 0, 1])
    lens = np.array([300, 5, 200])
    spec = workloads.TreeSpec("chain", parent, lens, np.array([0, 300, 305]), np.array([2]), 4, 4, 64, "f32", 0)
    ix, p = _plan(spec, 128)
    assert p["flat_ptr"].tolist() == [0, 1, 2, 3, 4] and p["flat_query"].tolist() == [0, 0, 0, 0]
    assert p["flat_rows"][:505].tolist() == list(range(505))
    words = p["flat_mask"].reshape(4, 2)
    full = (1 << 64) - 1
    assert [int(x) for x in words[:3].ravel()] == [full] * 6
    assert [int(x) for x in words[3]] == [full, (1 << 57) - 1]  # 505 - 384 = 121 = 64 + 57 tokens
    assert p["slot_ptr"].tolist() == [0, 4]


@pytest.mark.parametrize("page", [8, 16, 64])
@pytest.mark.parametrize("name", ["1", "3"])
def test_paged_rows_address_the_same_kv(name, page):
    spec = workloads.config(name)
    q, k, v = workloads.make_tensors(spec, "cpu")
    paged, kk, vv = workloads.page_pools(spec, k, v, page, fill=0.0)
    _, pc = _plan(spec, 256)
    _, pp = _plan(spec, 256, page_size=page, page_ptr=paged["page_ptr"], page_idx=paged["page_idx"])
    rc, rp = pc["flat_rows"], pp["flat_rows"]
    assert ((rc >= 0) == (rp >= 0)).all()
    import torch

    ok = rc >= 0
    ip, ic = (torch.from_numpy(x[ok].astype(np.int64)) for x in (rp, rc))
    assert torch.equal(kk[:, ip], k[:, ic]) and torch.equal(vv[:, ip], v[:, ic])
    for key in ("flat_ptr", "flat_query", "flat_mask", "tasks", "slot_ptr"):
        assert np.array_equal(pc[key], pp[key]), key
