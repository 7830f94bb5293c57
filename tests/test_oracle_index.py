"""Pins of the oracle's tree index (CPU only): the pages' worked structures,
closed forms, the IO-complexity identity and every validation error."""
import json
import os

import numpy as np
import pytest

import oracle
import workloads
from workloads import TreeSpec

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _spec_from(tree, **kw):
    lens = np.array(tree["kv_len"])
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    return TreeSpec("golden", np.array(tree["parent"]), lens, offs, np.array(tree["query_node"]),
                    kw.get("hq", 2), kw.get("hkv", 1), 8, "f32", 0)


def _csr(ptr, idx):
    return [list(map(int, idx[ptr[i]:ptr[i + 1]])) for i in range(len(ptr) - 1)]


def test_deft_two_query_cascade():
    g = _load("deft_two_query_cascade.json")
    spec = _spec_from(g["tree"])
    ix = oracle.build_index(spec)
    assert _csr(ix["qn_ptr"], ix["qn_idx"]) == g["expect"]["query_to_nodes"]
    assert _csr(ix["nq_ptr"], ix["nq_idx"]) == g["expect"]["node_to_queries"]
    assert list(ix["visible"]) == g["expect"]["visible_tokens"]


def test_flashinfer_decode_cascade_indptr():
    g = _load("flashinfer_decode_cascade_7req.json")
    spec = _spec_from(g["tree"])
    ix = oracle.build_index(spec)
    n_q = ix["n_q"]
    assert [0, int(n_q[0])] == g["expect"]["qo_indptr_shared"]
    assert [0] + list(np.cumsum(n_q[1:])) == g["expect"]["qo_indptr_unique"]


def test_specinfer_segment_mask():
    g = _load("specinfer_qbcm_110.json")
    spec = _spec_from(g["tree"])
    ix = oracle.build_index(spec)
    paths = _csr(ix["qn_ptr"], ix["qn_idx"])
    got = ["".join("1" if s in paths[r] else "0" for s in range(spec.num_nodes)) for r in range(spec.num_queries)]
    assert got == g["expect"]["segment_mask"]


def test_config2_closed_forms():
    spec = workloads.config("2")
    ix = oracle.build_index(spec)
    assert _csr(ix["qn_ptr"], ix["qn_idx"]) == [[0, 1 + r] for r in range(64)]
    assert ix["n_q"][0] == 64 and (ix["n_q"][1:] == 1).all()
    assert len(ix["qn_idx"]) == int(ix["depth"][spec.query_node].sum()) == 128
    assert (ix["visible"] == 32768 + 512).all()


def test_config3_closed_forms():
    spec = workloads.config("3")
    ix = oracle.build_index(spec)
    assert ix["n_q"][0] == 128 and (ix["n_q"][1:9] == 16).all() and (ix["n_q"][9:] == 1).all()
    assert (ix["depth"][9:] == 3).all()
    assert (ix["visible"] == 4000 + 1024 + 128).all()


@pytest.mark.parametrize("seed", range(10))
def test_io_identity(seed):
    """CoDec's IO comparison (section 块间启动与树归约, complexity analysis):
    per-query reading costs sum_i n[i] n_q[i] tokens, shared reading sum_i n[i].
    With no masks, sum_i n[i] n_q[i] must equal the tokens every query sees."""
    spec = workloads.random_tree(seed, max_nodes=8, max_len=50, max_queries=8)
    ix = oracle.build_index(spec)
    assert int((ix["n_q"].astype(np.int64) * spec.kv_len).sum()) == int(ix["visible"].sum())
    assert sum(len(oracle.visible_tokens(spec, r)) for r in range(spec.num_queries)) == int(ix["visible"].sum())


def test_masks_sit_only_on_the_own_masked_node():
    spec = workloads.config("4")
    ix = oracle.build_index(spec)
    ones = np.uint64(0xFFFFFFFFFFFFFFFF)
    for i in range(spec.num_nodes):
        ent = slice(ix["nq_ptr"][i], ix["nq_ptr"][i + 1])
        if spec.node_masked[i]:
            qs = ix["nq_idx"][ent]
            assert (ix["nq_mask"][ent] == spec.query_mask[qs]).all()
        else:
            assert (ix["nq_mask"][ent] == ones).all()
    assert int(ix["visible"].sum()) == int(sum(spec.kv_len[spec.parent[spec.query_node]])) + \
        sum(bin(int(m)).count("1") for m in spec.query_mask)


BAD = {
    "parent_not_before_child": dict(parent=[-1, 2, 0]),
    "zero_length": dict(kv_len=[4, 0, 3]),
    "negative_offset": dict(kv_offset=[0, -1, 9]),
    "query_on_missing_node": dict(query_node=[1, 5]),
    "masked_node_too_long": dict(kv_len=[4, 65, 3], node_masked=[0, 1, 0], query_mask=[1, 0]),
    "mask_bit_past_length": dict(node_masked=[0, 1, 0], query_mask=[1 << 2, 0]),
    "query_sees_nothing": dict(parent=[-1, -1, 0], node_masked=[0, 1, 0], query_mask=[0, 0]),
}


@pytest.mark.parametrize("case", sorted(BAD))
def test_invalid_trees(case):
    base = dict(parent=[-1, 0, 0], kv_len=[4, 2, 3], kv_offset=[0, 4, 6], query_node=[1, 2],
                node_masked=None, query_mask=None)
    base.update(BAD[case])
    spec = TreeSpec(case, np.array(base["parent"]), np.array(base["kv_len"]), np.array(base["kv_offset"]),
                    np.array(base["query_node"]), 2, 1, 8, "f32", 0,
                    query_mask=None if base["query_mask"] is None else np.array(base["query_mask"], dtype=np.uint64),
                    node_masked=None if base["node_masked"] is None else np.array(base["node_masked"]))
    with pytest.raises(oracle.TreeError) as e:
        oracle.build_index(spec)
    assert e.value.code == "PST_E_INVALID_TREE"
