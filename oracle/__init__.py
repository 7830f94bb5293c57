"""CPU oracle for prefix-shared tree decode attention.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call,
link or execute anything in this package: only ``tests/``, the smoke check
in ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py``
use it.  It shares no code with the HIP library (``prefix_shared_tree_amd``)
and imports nothing from it; both sides only consume the seeded inputs from
``workloads``.

Contents (each function cites the passage it follows):

* :mod:`oracle.attention` -- plain per-query full-softmax attention over the
  concatenated root-to-node KV in float64, returning O and the natural-log
  LSE.  This is what the method computes exactly (up to rounding order).
* :mod:`oracle.merge` -- the three printed forms of the partial-result merge
  (CoDec's POR, CoDec's streaming (M, D, U) accumulators, FlashDecoding's
  G-way reduction) and the LSE form used by DEFT.
* :mod:`oracle.tree_index` -- the tree index (node table, query->node and
  node->query CSR) in canonical order.
* :mod:`oracle.cost` and :mod:`oracle.planner` -- integer cost-table lookup
  and the task partitioner, as read from CoDec's workload-balance section;
  the pages leave the exact procedure open, so these follow the library's
  stated reading step by step.
* :mod:`oracle.flatten` -- DEFT's flattened tree KV splitting (depth-first
  flattening, equal chunks, per-chunk query groups with 64-bit bit causal
  masks), pinned against the attention oracle's visibility.

Parity status: attention, merge and index are pinned by tests against
brute force, closed forms, library routines and invariants.  The planner's
*quality* (how close to the optimal makespan) is parity unpinned; its
structure is pinned by invariants, Graham's LPT bound against brute force on
tiny instances, and a brute-force scan for the binary search.
"""
from .attention import attend, visible_tokens, partial_attend
from .merge import por_pair, por_chain, flashdecoding_merge, lse_merge, streaming_merge
from .tree_index import build_index, TreeError
from .cost import CostTable
from .planner import plan
from .flatten import flatten_plan

__all__ = [
    "attend", "visible_tokens", "partial_attend",
    "por_pair", "por_chain", "flashdecoding_merge", "lse_merge", "streaming_merge",
    "build_index", "TreeError", "CostTable", "plan", "flatten_plan",
]
