"""Pins of the oracle's attention against things other than itself (CPU only).

* brute force in 50-digit arithmetic (mpmath) from a different formulation
  of visibility (ancestor-or-self test per token instead of a path walk);
* the single-node tree against torch's scaled_dot_product_attention;
* closed forms: constant V, q = 0, one visible token;
* invariants: token permutation within a node, tree == per-query flattened
  sequences, masked node == explicit chain of one-token nodes,
  shared-root tree == two-level cascade merged by LSE.
"""
import math

import mpmath
import numpy as np
import pytest
import torch

import oracle
import workloads
from workloads import TreeSpec

mpmath.mp.dps = 50


def _is_ancestor_or_self(parent, a, b):
    while b != -1:
        if b == a:
            return True
        b = int(parent[b])
    return False


def _brute(spec, q, k, v):
    """Textbook softmax attention in 50-digit arithmetic, visibility decided token by token."""
    hq, hkv, d = spec.num_q_heads, spec.num_kv_heads, spec.head_dim
    g = hq // hkv
    scale = 1 / mpmath.sqrt(d)
    q = q.to(torch.float64).numpy()
    k = k.to(torch.float64).numpy()
    v = v.to(torch.float64).numpy()
    O = np.zeros((spec.num_queries, hq, d))
    L = np.zeros((spec.num_queries, hq))
    for r in range(spec.num_queries):
        own = int(spec.query_node[r])
        toks = []
        for node in range(spec.num_nodes):
            if not _is_ancestor_or_self(spec.parent, node, own):
                continue
            for j in range(int(spec.kv_len[node])):
                if (node == own and spec.node_masked is not None and spec.node_masked[node]
                        and not (int(spec.query_mask[r]) >> j) & 1):
                    continue
                toks.append(int(spec.kv_offset[node]) + j)
        for h in range(hq):
            kh = h // g
            s = [scale * mpmath.fsum(mpmath.mpf(q[r, h, c]) * mpmath.mpf(k[kh, t, c]) for c in range(d))
                 for t in toks]
            mx = max(s)
            w = [mpmath.exp(x - mx) for x in s]
            z = mpmath.fsum(w)
            for c in range(d):
                O[r, h, c] = float(mpmath.fsum(w[i] * mpmath.mpf(v[kh, t, c]) for i, t in enumerate(toks)) / z)
            L[r, h] = float(mx + mpmath.log(z))
    return O, L


@pytest.mark.parametrize("seed", range(6))
def test_brute_force_tiny_trees(seed):
    spec = workloads.random_tree(seed, max_nodes=4, max_len=8, max_queries=3, num_q_heads=4,
                                 num_kv_heads=2, head_dim=8, masked_prob=0.5 if seed % 2 else 0.0)
    q, k, v = workloads.make_tensors(spec)
    O, L = oracle.attend(spec, q, k, v)
    Ob, Lb = _brute(spec, q, k, v)
    assert np.abs(O - Ob).max() <= 1e-13
    assert np.abs(L - Lb).max() <= 1e-13


@pytest.mark.parametrize("hq,hkv,d,n", [(4, 4, 64, 37), (8, 2, 128, 300), (6, 1, 16, 5)])
def test_single_node_is_sdpa(hq, hkv, d, n):
    spec = TreeSpec("single", np.array([-1]), np.array([n]), np.array([0]), np.array([0, 0, 0]),
                    hq, hkv, d, "f32", 7)
    q, k, v = workloads.make_tensors(spec)
    O, L = oracle.attend(spec, q, k, v)
    g = hq // hkv
    K = k.to(torch.float64).repeat_interleave(g, dim=0)  # [H_q, n, d]
    V = v.to(torch.float64).repeat_interleave(g, dim=0)
    Q = q.to(torch.float64).unsqueeze(2)  # [B, H_q, 1, d]
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K.unsqueeze(0).expand(3, -1, -1, -1),
                                                           V.unsqueeze(0).expand(3, -1, -1, -1))
    assert np.abs(O - ref[:, :, 0].numpy()).max() <= 1e-13
    # LSE: log of the sum of exp of the scaled scores, computed directly.
    s = (Q @ K.unsqueeze(0).transpose(-1, -2))[:, :, 0] / math.sqrt(d)
    assert np.abs(L - torch.logsumexp(s, dim=-1).numpy()).max() <= 1e-12


def test_constant_v_returns_v():
    spec = workloads.random_tree(11, max_nodes=6, max_len=50, max_queries=5)
    q, k, v = workloads.make_tensors(spec)
    c = torch.linspace(-3, 3, spec.head_dim, dtype=torch.float32)
    v = c.expand_as(v).clone()
    O, _ = oracle.attend(spec, q, k, v)
    assert np.abs(O - c.numpy()[None, None, :]).max() <= 1e-14


def test_zero_query_gives_mean_of_visible_values():
    spec = workloads.random_tree(12, max_nodes=6, max_len=30, max_queries=5, masked_prob=0.5)
    q, k, v = workloads.make_tensors(spec)
    q = torch.zeros_like(q)
    O, L = oracle.attend(spec, q, k, v)
    g = spec.group
    for r in range(spec.num_queries):
        toks = oracle.visible_tokens(spec, r)
        for h in range(spec.num_q_heads):
            mean = v[h // g, toks].to(torch.float64).mean(0).numpy()
            assert np.abs(O[r, h] - mean).max() <= 1e-14
            assert abs(L[r, h] - math.log(len(toks))) <= 1e-13


def test_one_visible_token():
    # A masked leaf whose only visible token is token 2, on a root with no ancestors.
    spec = TreeSpec("one", np.array([-1]), np.array([5]), np.array([0]), np.array([0]), 2, 1, 8, "f32", 3,
                    query_mask=np.array([1 << 2], dtype=np.uint64), node_masked=np.array([1]))
    q, k, v = workloads.make_tensors(spec)
    O, L = oracle.attend(spec, q, k, v)
    for h in range(2):
        assert np.abs(O[0, h] - v[0, 2].double().numpy()).max() == 0
        score = float(q[0, h].double() @ k[0, 2].double()) / math.sqrt(8)
        assert abs(L[0, h] - score) <= 1e-14


def test_permuting_tokens_within_a_node():
    spec = workloads.random_tree(21, max_nodes=5, max_len=40, max_queries=5)
    q, k, v = workloads.make_tensors(spec)
    O, L = oracle.attend(spec, q, k, v)
    rng = np.random.default_rng(0)
    k2, v2 = k.clone(), v.clone()
    for i in range(spec.num_nodes):
        a, n = int(spec.kv_offset[i]), int(spec.kv_len[i])
        p = torch.as_tensor(rng.permutation(n)) + a
        k2[:, a:a + n] = k[:, p]
        v2[:, a:a + n] = v[:, p]
    O2, L2 = oracle.attend(spec, q, k2, v2)
    assert np.abs(O - O2).max() <= 1e-13 and np.abs(L - L2).max() <= 1e-13


def test_tree_equals_flattened_sequences():
    """Each query on a private single node holding a copy of its path's tokens."""
    spec = workloads.random_tree(31, max_nodes=6, max_len=30, max_queries=6)
    q, k, v = workloads.make_tensors(spec)
    O, L = oracle.attend(spec, q, k, v)
    lens, offs, ks, vs = [], [], [], []
    pos = 0
    for r in range(spec.num_queries):
        # Path by ancestry test, independent of the oracle's path walk.
        own = int(spec.query_node[r])
        toks = []
        for node in range(spec.num_nodes):
            if _is_ancestor_or_self(spec.parent, node, own):
                a = int(spec.kv_offset[node])
                toks += list(range(a, a + int(spec.kv_len[node])))
        ks.append(k[:, toks])
        vs.append(v[:, toks])
        lens.append(len(toks))
        offs.append(pos)
        pos += len(toks)
    B = spec.num_queries
    flat = TreeSpec("flat", np.full(B, -1), np.array(lens), np.array(offs), np.arange(B),
                    spec.num_q_heads, spec.num_kv_heads, spec.head_dim, "f32", 0)
    O2, L2 = oracle.attend(flat, q, torch.cat(ks, 1), torch.cat(vs, 1))
    assert np.abs(O - O2).max() <= 1e-13 and np.abs(L - L2).max() <= 1e-13


def test_masked_node_equals_chain_of_one_token_nodes():
    """The 64-bit mask of a draft node == the draft tree written as explicit 1-token nodes."""
    rng = np.random.default_rng(5)
    n = 40
    par = np.full(n, -1)
    depth = np.ones(n, dtype=int)
    for i in range(1, n):
        cand = np.nonzero(depth[:i] < 8)[0]
        par[i] = cand[rng.integers(len(cand))]
        depth[i] = depth[par[i]] + 1
    masks = workloads.draft_tree_masks(par)
    prefix = 23
    spec = TreeSpec("masked", np.array([-1, 0]), np.array([prefix, n]), np.array([0, prefix]),
                    np.full(n, 1), 4, 2, 16, "f32", 9, query_mask=masks, node_masked=np.array([0, 1]))
    q, k, v = workloads.make_tensors(spec)
    O, L = oracle.attend(spec, q, k, v)
    # Explicit tree: node 0 = prefix, node 1 + j = draft token j (parent = its draft parent).
    parent = [-1] + [0 if par[j] == -1 else 1 + int(par[j]) for j in range(n)]
    chain = TreeSpec("chain", np.array(parent), np.array([prefix] + [1] * n),
                     np.array([0] + [prefix + j for j in range(n)]), 1 + np.arange(n), 4, 2, 16, "f32", 9)
    O2, L2 = oracle.attend(chain, q, k, v)
    assert np.abs(O - O2).max() <= 1e-13 and np.abs(L - L2).max() <= 1e-13


def test_shared_root_equals_two_level_cascade():
    """A root shared by all queries plus private leaves == cascade: shared level, unique level, LSE merge."""
    nleaf = 7
    lens = [300] + [17 + 3 * i for i in range(nleaf)]
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]])
    spec = TreeSpec("cascade", np.array([-1] + [0] * nleaf), np.array(lens), offs,
                    1 + np.arange(nleaf), 8, 2, 32, "f32", 13)
    q, k, v = workloads.make_tensors(spec)
    O, L = oracle.attend(spec, q, k, v)
    g, scale = 4, 1 / math.sqrt(32)
    for r in range(nleaf):
        for h in range(8):
            kh = h // g
            qq = q[r, h:h + 1].double().numpy()
            K = k[kh].double().numpy()
            V = v[kh].double().numpy()
            O0, _, _, l0 = oracle.partial_attend(qq, K[:300], V[:300], scale)
            a = offs[1 + r]
            O1, _, _, l1 = oracle.partial_attend(qq, K[a:a + lens[1 + r]], V[a:a + lens[1 + r]], scale)
            Om, Lm = oracle.lse_merge(np.stack([O0, O1]), np.stack([l0, l1]))
            assert np.abs(Om[0] - O[r, h]).max() <= 1e-13
            assert abs(Lm[0] - L[r, h]) <= 1e-13


def test_config1_runs_and_is_finite():
    spec = workloads.config("1")
    q, k, v = workloads.make_tensors(spec)
    O, L = oracle.attend(spec, q, k, v)
    assert O.shape == (4, 4, 64) and np.isfinite(O).all() and np.isfinite(L).all()
