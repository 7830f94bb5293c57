// Tree validation and index construction (host).
//
// CoDec: Prefix-Shared Decoding Kernel for LLMs, section KV缓存管理 (KV-cache
// management): the cache is a forest of KV nodes under a virtual root, and
// the memory manager keeps the bijective index between queries and the KV
// nodes of their prefixes, so that the queries sharing a node can be
// gathered into one partial computation and each query's partial results
// found again for the reduction.  DEFT: Decoding with Flash Tree-Attention,
// section A.8 (Algorithm 1) builds the same two maps (QMapKV, KVMapQ).
//
// Canonical order: a query's nodes root first; a node's queries by ascending
// id.  The node->query entries carry the 64-bit visibility mask of the
// query (the bit causal mask of DEFT section 3.3 / Table 2) where the node is
// the query's own masked node, all ones otherwise.
#include <string>

#include "pst_internal.h"

namespace pst {

static pst_status bad(const std::string& m) {
  set_error(m);
  return PST_E_INVALID_TREE;
}

pst_status build_tree_index(const pst_tree_desc& d, TreeIndex* out) {
  TreeIndex& t = *out;
  const int32_t N = d.num_nodes, B = d.num_queries;
  if (N < 0 || B < 0) {
    set_error("negative node or query count");
    return PST_E_INVALID_ARG;
  }
  const bool paged = d.page_size != 0;
  if ((N > 0 && (!d.parent || (!paged && !d.kv_offset) || !d.kv_len)) || (B > 0 && !d.query_node) ||
      (paged && (!d.page_ptr || (N > 0 && d.page_ptr[N] > 0 && !d.page_idx)))) {
    set_error("null tree array");
    return PST_E_INVALID_ARG;
  }
  if (paged && (d.page_size < 8 || d.page_size > 65536 || (d.page_size & (d.page_size - 1)) != 0)) {
    set_error("page_size must be 0 or a power of two in [8, 65536]");
    return PST_E_INVALID_ARG;
  }
  t.N = N;
  t.B = B;
  t.parent.assign(d.parent, d.parent + N);
  t.kv_len.assign(d.kv_len, d.kv_len + N);
  if (paged) {
    // Paged K/V: validate the page table; kv_offset is unused (zeros).
    t.page_size = d.page_size;
    t.kv_offset.assign(N, 0);
    t.page_ptr.assign(d.page_ptr, d.page_ptr + N + 1);
    if (t.page_ptr[0] != 0) return bad("page_ptr[0] != 0");
    for (int32_t i = 0; i < N; ++i) {
      if (t.page_ptr[i + 1] < t.page_ptr[i]) return bad("page_ptr decreases at node " + std::to_string(i));
      if (static_cast<int64_t>(t.page_ptr[i + 1] - t.page_ptr[i]) * d.page_size < d.kv_len[i])
        return bad("node " + std::to_string(i) + " has fewer pages than its tokens need");
    }
    t.page_idx.assign(d.page_idx, d.page_idx + t.page_ptr[N]);
    for (size_t k = 0; k < t.page_idx.size(); ++k)
      if (t.page_idx[k] < 0) return bad("page_idx[" + std::to_string(k) + "] < 0");
  } else {
    t.kv_offset.assign(d.kv_offset, d.kv_offset + N);
  }
  t.query_node.assign(d.query_node, d.query_node + B);
  t.masked.assign(N, 0);
  if (d.node_masked)
    for (int32_t i = 0; i < N; ++i) t.masked[i] = d.node_masked[i] ? 1 : 0;
  t.qmask.assign(B, ~0ull);
  const bool have_mask = d.query_mask != nullptr;
  t.have_mask = have_mask;
  if (have_mask) t.qmask.assign(d.query_mask, d.query_mask + B);

  for (int32_t i = 0; i < N; ++i) {
    if (t.parent[i] < -1 || t.parent[i] >= i)
      return bad("parent[" + std::to_string(i) + "] not in [-1, " + std::to_string(i) + ")");
    if (t.kv_len[i] < 1) return bad("kv_len[" + std::to_string(i) + "] < 1");
    if (t.kv_offset[i] < 0) return bad("kv_offset[" + std::to_string(i) + "] < 0");
    if (t.masked[i] && t.kv_len[i] > 64) return bad("masked node " + std::to_string(i) + " longer than 64");
  }
  t.depth.assign(N, 0);
  for (int32_t i = 0; i < N; ++i) t.depth[i] = t.parent[i] < 0 ? 1 : t.depth[t.parent[i]] + 1;

  // query -> node CSR: each path root first.
  t.qn_ptr.assign(B + 1, 0);
  t.visible.assign(B, 0);
  for (int32_t r = 0; r < B; ++r) {
    const int32_t n = t.query_node[r];
    if (n < 0 || n >= N) return bad("query_node[" + std::to_string(r) + "] out of range");
    t.qn_ptr[r + 1] = t.qn_ptr[r] + t.depth[n];
  }
  t.qn_idx.assign(t.qn_ptr[B], 0);
  for (int32_t r = 0; r < B; ++r) {
    const int32_t own = t.query_node[r];
    int64_t vis = 0;
    int32_t pos = t.qn_ptr[r + 1];
    for (int32_t n = own; n != -1; n = t.parent[n]) {
      t.qn_idx[--pos] = n;
      if (n != own) vis += t.kv_len[n];
    }
    if (t.masked[own] && have_mask) {
      const uint64_t bits = t.qmask[r];
      if (t.kv_len[own] < 64 && (bits >> t.kv_len[own]) != 0)
        return bad("mask of query " + std::to_string(r) + " has bits past the node length");
      vis += __builtin_popcountll(bits);
    } else {
      vis += t.kv_len[own];
    }
    if (vis == 0) return bad("query " + std::to_string(r) + " sees no token");
    t.visible[r] = vis;
  }

  // node -> query CSR: counting sort by node; queries visited in ascending order.
  t.nq_ptr.assign(N + 1, 0);
  for (int32_t e = 0; e < t.qn_ptr[B]; ++e) t.nq_ptr[t.qn_idx[e] + 1]++;
  for (int32_t i = 0; i < N; ++i) t.nq_ptr[i + 1] += t.nq_ptr[i];
  t.n_q.assign(N, 0);
  for (int32_t i = 0; i < N; ++i) t.n_q[i] = t.nq_ptr[i + 1] - t.nq_ptr[i];
  t.nq_idx.assign(t.qn_ptr[B], 0);
  t.nq_mask.assign(t.qn_ptr[B], ~0ull);
  std::vector<int32_t> cur(t.nq_ptr.begin(), t.nq_ptr.end() - (N > 0 ? 1 : 0));
  if (N == 0) cur.clear();
  for (int32_t r = 0; r < B; ++r) {
    for (int32_t e = t.qn_ptr[r]; e < t.qn_ptr[r + 1]; ++e) {
      const int32_t n = t.qn_idx[e];
      const int32_t slot = cur[n]++;
      t.nq_idx[slot] = r;
      if (t.masked[n] && have_mask && n == t.query_node[r]) t.nq_mask[slot] = t.qmask[r];
    }
  }
  return PST_OK;
}

}  // namespace pst
