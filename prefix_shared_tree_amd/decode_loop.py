"""Multi-step decoding over a prefix tree: growth in place and plan reuse.

CoDec: Prefix-Shared Decoding Kernel for LLMs, implementation section: the
partition is computed once and reused across decoding steps, at a small
fraction of the attention time; DEFT: Decoding with Flash Tree-Attention,
section A.1: the tree's KV grows as each request appends its decoded token.

A session owns a paged K/V pool (page table as in ``pst_tree_desc``) in which
every query's own node is a leaf that only that query extends, with spare
pages reserved for growth.  Each step appends one token per query (the
caller's new K/V rows) into the leaf's next slot, updates the tree's
lengths in place (``pst_tree_set_lengths``: the last piece of every grown
node absorbs the growth, so the plan stays valid) and re-plans on a fixed
period (``replan_every`` steps; 0 = never).  Topology changes (branching,
pruning) need a new tree and plan; they are out of this session's scope.
"""
from __future__ import annotations

import time

import numpy as np

from . import Plan, Tree, decode_attn, workspace


class DecodeSession:
    """Decode loop over ``spec``'s tree (``workloads.TreeSpec``-like) with K/V
    ``k``, ``v`` ([H_kv, T, d], contiguous per ``spec.kv_offset``).

    Every query's own node must be a leaf no other query ends on.  Leaves get
    ``max_new_tokens`` tokens of spare capacity.
    """

    def __init__(self, spec, k, v, *, page_size=16, max_new_tokens=64, replan_every=0, out_dtype="f32",
                 plan_kw=None):
        import torch

        parent = np.asarray(spec.parent, dtype=np.int64)
        qn = np.asarray(spec.query_node, dtype=np.int64)
        if len(np.unique(qn)) != len(qn):
            raise ValueError("every query needs a leaf of its own")
        has_child = np.zeros(spec.num_nodes, dtype=bool)
        has_child[parent[parent >= 0]] = True
        if has_child[qn].any():
            raise ValueError("a query's own node has children")
        if spec.node_masked is not None and np.asarray(spec.node_masked)[qn].any():
            raise ValueError("masked nodes do not grow")
        P = int(page_size)
        self.page_size = P
        self.kv_len = np.asarray(spec.kv_len, dtype=np.int32).copy()
        spare = np.zeros(spec.num_nodes, dtype=np.int64)
        spare[qn] = int(max_new_tokens)
        npg = (self.kv_len.astype(np.int64) + spare + P - 1) // P
        self.page_ptr = np.concatenate([[0], np.cumsum(npg)]).astype(np.int32)
        total = int(self.page_ptr[-1])
        self.page_idx = np.arange(total, dtype=np.int32)
        rows = np.full(total * P, -1, dtype=np.int64)
        for i in range(spec.num_nodes):
            j = np.arange(int(self.kv_len[i]), dtype=np.int64)
            pages = self.page_idx[self.page_ptr[i]:self.page_ptr[i + 1]].astype(np.int64)
            rows[pages[j // P] * P + j % P] = int(spec.kv_offset[i]) + j
        src = torch.from_numpy(rows).to(k.device)
        ok = src >= 0
        self.k = torch.zeros((k.shape[0], total * P, k.shape[2]), dtype=k.dtype, device=k.device)
        self.v = torch.zeros_like(self.k)
        self.k[:, ok] = k[:, src[ok]]
        self.v[:, ok] = v[:, src[ok]]
        self.query_node = qn
        self.capacity = (npg * P).astype(np.int64)
        self.tree = Tree(spec.parent, None, self.kv_len, spec.query_node, num_q_heads=spec.num_q_heads,
                         num_kv_heads=spec.num_kv_heads, head_dim=spec.head_dim, dtype=spec.dtype,
                         out_dtype=out_dtype, query_mask=spec.query_mask, node_masked=spec.node_masked,
                         page_size=P, page_ptr=self.page_ptr, page_idx=self.page_idx)
        self.plan_kw = dict(plan_kw or {})
        self.replan_every = int(replan_every)
        self.plan = Plan(self.tree, **self.plan_kw)
        self.ws = workspace(self.plan, k.device)
        self.steps = 0
        self.steps_since_plan = 0
        self.replans = 0
        self.replan_s = 0.0

    def pool_rows(self, nodes, positions):
        """Pool rows of token ``positions`` of ``nodes`` (arrays of the same length)."""
        P = self.page_size
        nodes = np.asarray(nodes, dtype=np.int64)
        positions = np.asarray(positions, dtype=np.int64)
        pages = self.page_idx[self.page_ptr[nodes] + positions // P].astype(np.int64)
        return pages * P + positions % P

    def append(self, k_new, v_new):
        """Append one token per query: ``k_new``, ``v_new`` are [B, H_kv, d]."""
        import torch

        pos = self.kv_len[self.query_node].astype(np.int64)
        if (pos + 1 > self.capacity[self.query_node]).any():
            raise ValueError("a leaf has used its spare capacity (max_new_tokens)")
        rows = torch.from_numpy(self.pool_rows(self.query_node, pos)).to(self.k.device)
        self.k[:, rows] = k_new.transpose(0, 1).to(self.k.dtype)
        self.v[:, rows] = v_new.transpose(0, 1).to(self.v.dtype)
        self.kv_len[self.query_node] += 1
        self.tree.set_lengths(self.kv_len)
        self.steps += 1
        self.steps_since_plan += 1
        if self.replan_every and self.steps_since_plan >= self.replan_every:
            t0 = time.perf_counter()
            self.plan.free()
            self.plan = Plan(self.tree, **self.plan_kw)
            self.ws = workspace(self.plan, self.k.device)
            self.replan_s += time.perf_counter() - t0
            self.replans += 1
            self.steps_since_plan = 0

    def decode(self, q, *, out=None, lse=None):
        """Attention of this step's queries ``q`` [B, H_q, d] over the current tree."""
        return decode_attn(self.plan, q, self.k, self.v, out=out, lse=lse, ws=self.ws)
