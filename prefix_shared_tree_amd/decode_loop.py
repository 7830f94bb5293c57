"""Multi-step decoding over a prefix tree: growth in place, branching,
pruning and plan reuse.

CoDec: Prefix-Shared Decoding Kernel for LLMs, implementation section: the
partition is computed once and reused across decoding steps, at a small
fraction of the attention time; DEFT: Decoding with Flash Tree-Attention,
section A.1: the tree's KV grows as each request appends its decoded token,
and requests fork (tree search, speculative drafts) or finish.

A session owns a paged K/V pool (page table as in ``pst_tree_desc``) with a
free list of pages.  Every query's own node is a leaf that only that query
extends, with spare pages reserved for growth.
* ``append``: one token per query into its leaf's next slot; the lengths
  change in place (``pst_tree_append``: the last piece of every grown node
  absorbs the growth, so the plan stays valid); re-plan on a fixed
  period (``replan_every`` steps; 0 = never).  With a flattened partition
  (``plan_kw={"flatten": S_t}``) every step plans again: growth moves the
  chunks.
* ``branch``: a query's leaf becomes an inner node and gets new one-token
  leaves, one for the query and one for each new query that forks from it.
* ``prune``: a query finishes; the nodes only it used go back to the free
  list.
Branching and pruning change the topology: the tree is rebuilt over the same
pool and the plan made again.
"""
from __future__ import annotations

import time

import numpy as np

from . import Plan, Tree, decode_attn, workspace


class DecodeSession:
    """Decode loop over ``spec``'s tree (``workloads.TreeSpec``-like) with K/V
    ``k``, ``v`` ([H_kv, T, d], contiguous per ``spec.kv_offset``).

    Every query's own node must be a leaf no other query ends on.  Leaves get
    ``max_new_tokens`` tokens of spare capacity; the pool holds
    ``extra_pages`` pages beyond the initial tree for leaves made by
    ``branch``.  ``host_only``: tree and plan on the host only (bookkeeping
    without a GPU; ``decode`` is then unavailable).
    """

    def __init__(self, spec, k, v, *, page_size=16, max_new_tokens=64, extra_pages=0, replan_every=0,
                 out_dtype="f32", plan_kw=None, host_only=False):
        import torch

        parent = np.asarray(spec.parent, dtype=np.int64)
        qn = np.asarray(spec.query_node, dtype=np.int64)
        if len(np.unique(qn)) != len(qn):
            raise ValueError("every query needs a leaf of its own")
        has_child = np.zeros(spec.num_nodes, dtype=bool)
        has_child[parent[parent >= 0]] = True
        if has_child[qn].any():
            raise ValueError("a query's own node has children")
        if spec.query_mask is not None or (spec.node_masked is not None and np.asarray(spec.node_masked).any()):
            raise ValueError("the session takes trees without masks")
        P = int(page_size)
        self.page_size = P
        self.max_new = int(max_new_tokens)
        self.heads = (spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.dtype, out_dtype)
        self.parent = parent.astype(np.int32)
        self.kv_len = np.asarray(spec.kv_len, dtype=np.int32).copy()
        self.query_node = qn.astype(np.int32)
        spare = np.zeros(spec.num_nodes, dtype=np.int64)
        spare[qn] = self.max_new
        npg = (self.kv_len.astype(np.int64) + spare + P - 1) // P
        total = int(npg.sum())
        self.pool_pages = total + int(extra_pages)
        # Node i's pages: self.pages[i] (list of page numbers).
        self.pages = []
        nxt = 0
        for i in range(spec.num_nodes):
            self.pages.append(list(range(nxt, nxt + int(npg[i]))))
            nxt += int(npg[i])
        self.free = list(range(total, self.pool_pages))
        rows = np.full(self.pool_pages * P, -1, dtype=np.int64)
        for i in range(spec.num_nodes):
            j = np.arange(int(self.kv_len[i]), dtype=np.int64)
            pg = np.asarray(self.pages[i], dtype=np.int64)
            rows[pg[j // P] * P + j % P] = int(spec.kv_offset[i]) + j
        src = torch.from_numpy(rows).to(k.device)
        ok = src >= 0
        self.k = torch.zeros((k.shape[0], self.pool_pages * P, k.shape[2]), dtype=k.dtype, device=k.device)
        self.v = torch.zeros_like(self.k)
        self.k[:, ok] = k[:, src[ok]]
        self.v[:, ok] = v[:, src[ok]]
        self.plan_kw = dict(plan_kw or {})
        self.host_only = bool(host_only)
        self.replan_every = int(replan_every)
        self.steps = 0
        self.steps_since_plan = 0
        self.replans = 0
        self.replan_s = 0.0
        self.plan = None
        self._rebuild()

    # -- tree and plan -------------------------------------------------------
    def _table(self):
        page_ptr = np.zeros(len(self.pages) + 1, dtype=np.int32)
        page_ptr[1:] = np.cumsum([len(p) for p in self.pages])
        page_idx = np.asarray([x for p in self.pages for x in p], dtype=np.int32)
        return page_ptr, page_idx

    def _leaf_capacity(self):
        """Tokens each query's leaf can hold (its pages)."""
        qn = self.query_node.astype(np.int64)
        return (self.page_ptr[qn + 1] - self.page_ptr[qn]).astype(np.int64) * self.page_size

    def _rebuild(self):
        """A new tree and plan after a topology change."""
        hq, hkv, d, dtype, odt = self.heads
        self.page_ptr, self.page_idx = self._table()
        if self.plan is not None:
            self.plan.free()
            self.tree.free()
        self.tree = Tree(self.parent, None, self.kv_len, self.query_node, num_q_heads=hq, num_kv_heads=hkv,
                         head_dim=d, dtype=dtype, out_dtype=odt, page_size=self.page_size, page_ptr=self.page_ptr,
                         page_idx=self.page_idx, pool_tokens=self.pool_pages * self.page_size,
                         host_only=self.host_only)
        self.leaf_cap = self._leaf_capacity()
        self._make_plan()
        self.steps_since_plan = 0

    def _make_plan(self):
        self.plan = Plan(self.tree, **self.plan_kw)
        self.ws = None if self.host_only else workspace(self.plan, self.k.device)

    def _replan(self):
        t0 = time.perf_counter()
        if self.plan is not None:
            self.plan.free()
        self._make_plan()
        self.replan_s += time.perf_counter() - t0
        self.replans += 1
        self.steps_since_plan = 0

    def _pages_for(self, node):
        return (int(self.kv_len[node]) + self.page_size - 1) // self.page_size

    def _alloc(self, n):
        if n > len(self.free):
            raise ValueError("the pool has no free pages left (extra_pages)")
        got, self.free = self.free[:n], self.free[n:]
        return got

    @property
    def num_queries(self) -> int:
        return len(self.query_node)

    def pool_rows(self, nodes, positions):
        """Pool rows of token ``positions`` of ``nodes`` (arrays of the same length)."""
        P = self.page_size
        nodes = np.asarray(nodes, dtype=np.int64)
        positions = np.asarray(positions, dtype=np.int64)
        pages = self.page_idx[self.page_ptr[nodes] + positions // P].astype(np.int64)
        return pages * P + positions % P

    # -- steps ---------------------------------------------------------------
    def append(self, k_new, v_new):
        """Append one token per query: ``k_new``, ``v_new`` are [B, H_kv, d].
        On the GPU one library call (``pst_tree_append``) writes the rows at
        each leaf's next position and grows the lengths and the plan's last
        pieces, in one kernel launch and without waiting for the device."""
        qn = self.query_node.astype(np.int64)
        pos = self.kv_len[qn].astype(np.int64)
        if (pos + 1 > self.leaf_cap).any():
            raise ValueError("a leaf has used its spare capacity (max_new_tokens)")
        flat = bool(self.plan_kw.get("flatten"))
        if flat:
            # A flattened partition's chunks move when a node grows: plan again
            # every step (the tree refuses growth while such a plan is live).
            self.plan.free()
            self.plan = None
        if self.k.device.type == "cuda":
            self.tree.append(qn.astype(np.int32), k_new.to(self.k.dtype).contiguous(),
                             v_new.to(self.v.dtype).contiguous(), self.k, self.v)
            self.kv_len[qn] += 1
        else:
            import torch

            rows = torch.from_numpy(self.pool_rows(qn, pos))
            self.k[:, rows] = k_new.transpose(0, 1).to(self.k.dtype)
            self.v[:, rows] = v_new.transpose(0, 1).to(self.v.dtype)
            self.kv_len[qn] += 1
            self.tree.set_lengths(self.kv_len)
        self.steps += 1
        self.steps_since_plan += 1
        if flat:
            self._replan()
            return
        if self.replan_every and self.steps_since_plan >= self.replan_every:
            self._replan()

    def branch(self, query, k_first, v_first):
        """Fork ``query``: its leaf stops growing and gets ``n`` new one-token
        leaves (``k_first``, ``v_first``: [n, H_kv, d]).  The query continues
        on the first; queries num_queries .. num_queries + n - 2 (new, at the
        end) on the others.  Returns the new queries' ids."""
        import torch

        n = int(k_first.shape[0])
        if n < 1:
            raise ValueError("branch needs at least one new leaf")
        old = int(self.query_node[query])
        per = (1 + self.max_new + self.page_size - 1) // self.page_size
        if n * per > len(self.free) + len(self.pages[old]) - self._pages_for(old):
            raise ValueError("the pool has no free pages left (extra_pages)")
        # The old leaf stops growing: its spare pages go back.
        keep = self._pages_for(old)
        self.free.extend(self.pages[old][keep:])
        self.pages[old] = self.pages[old][:keep]
        new_nodes = []
        for _ in range(n):
            self.parent = np.append(self.parent, np.int32(old))
            self.kv_len = np.append(self.kv_len, np.int32(1))
            self.pages.append(self._alloc(per))
            new_nodes.append(len(self.pages) - 1)
        rows = torch.tensor([self.pages[i][0] * self.page_size for i in new_nodes], device=self.k.device)
        self.k[:, rows] = k_first.transpose(0, 1).to(self.k.dtype)
        self.v[:, rows] = v_first.transpose(0, 1).to(self.v.dtype)
        self.query_node[query] = new_nodes[0]
        first_new = self.num_queries
        self.query_node = np.append(self.query_node, np.asarray(new_nodes[1:], dtype=np.int32))
        self._rebuild()
        return list(range(first_new, self.num_queries))

    def prune(self, query):
        """``query`` finishes: it is removed (later queries' ids drop by one)
        and the nodes no remaining query uses return their pages."""
        if self.num_queries <= 1:
            raise ValueError("the last query cannot be pruned")
        self.query_node = np.delete(self.query_node, query)
        N = len(self.pages)
        used = np.zeros(N, dtype=bool)
        for q in self.query_node:
            n = int(q)
            while n >= 0 and not used[n]:
                used[n] = True
                n = int(self.parent[n])
        keep = np.flatnonzero(used)
        for i in np.flatnonzero(~used):
            self.free.extend(self.pages[i])
        remap = -np.ones(N, dtype=np.int64)
        remap[keep] = np.arange(len(keep))
        self.parent = np.asarray([remap[p] if p >= 0 else -1 for p in self.parent[keep]], dtype=np.int32)
        self.kv_len = self.kv_len[keep]
        self.pages = [self.pages[i] for i in keep]
        self.query_node = remap[self.query_node].astype(np.int32)
        self._rebuild()

    def decode(self, q, *, out=None, lse=None):
        """Attention of this step's queries ``q`` [B, H_q, d] over the current tree."""
        if self.host_only:
            raise RuntimeError("a host-only session has no device plan")
        return decode_attn(self.plan, q, self.k, self.v, out=out, lse=lse, ws=self.ws)

    def contiguous(self):
        """The session's tree in the contiguous layout: (parent, kv_len,
        kv_offset, query_node, k, v), nodes back to back, gathered from the
        pool (for checking against a reference)."""
        import torch

        off = np.zeros(len(self.kv_len), dtype=np.int64)
        off[1:] = np.cumsum(self.kv_len.astype(np.int64))[:-1]
        rows = np.concatenate([self.pool_rows(np.full(int(n), i), np.arange(int(n)))
                               for i, n in enumerate(self.kv_len)])
        idx = torch.from_numpy(rows).to(self.k.device)
        return (self.parent.copy(), self.kv_len.copy(), off, self.query_node.copy(),
                self.k[:, idx].contiguous(), self.v[:, idx].contiguous())
