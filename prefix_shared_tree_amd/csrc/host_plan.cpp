// Cost model and task partitioner (host).
//
// CoDec: Prefix-Shared Decoding Kernel for LLMs, section 工作负载平衡
// (workload balance).  A node is a task (n_q, n); it can be cut along the
// KV axis into b_k vertical slices; the slices are assigned to m blocks so
// that the slowest block is as fast as possible (the min-max objective of
// section 速读).  CoDec keeps the query axis whole (b_q = 1, so shared KV is
// read once), finds a lower bound cost_l of the per-block cost by binary
// search from "slices cost at least the whole" and "the maximum is at least
// the average", caps b_k[i] at ceil(C_est(n_q[i], n[i]) / cost_l), and grid
// searches the splits.  The cost of a slice comes from a profiled table
// C_est(n_q, n) with interpolation (profile-based cost estimation).
//
// The pages give no constants, tie-breaks or piece geometry; the reading
// implemented here (identically to the CPU oracle, in integers):
//  * rows r = n_q * g (queries x GQA group) are cut into ceil(r / R_max) row
//    groups only when a node has more rows than a workgroup holds;
//  * b pieces have Lp = roundup(ceil(n / b), G) tokens (the last shorter);
//  * b(T) = smallest b whose longest piece of the largest row group costs
//    <= T; W(T) = the least total cost of splits into b(T) or more pieces
//    per node (every such split has all pieces <= T); cost_l = smallest T
//    with m T >= W(T) (W is non-increasing, so a binary search finds it);
//  * candidates T_k = cost_l + cost_l * k / K (k = 0..K), b = min(ub, b(T_k));
//  * pieces placed by longest-processing-time list scheduling (Graham 1966,
//    cited by CoDec) onto the bin with the smallest (load, id); the
//    candidate with the smallest makespan wins (ties: fewer pieces, smaller k).
#include <algorithm>
#include <functional>
#include <queue>
#include <string>
#include <utility>

#include "pst_internal.h"

namespace pst {

static inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

int64_t CostModel::lookup(int64_t rows, int64_t len) const {
  const int nr = static_cast<int>(rows_grid.size());
  const int nl = static_cast<int>(len_grid.size());
  int ri = static_cast<int>(std::lower_bound(rows_grid.begin(), rows_grid.end(), rows) - rows_grid.begin());
  if (ri == nr) ri = nr - 1;
  const int64_t* row = table.data() + static_cast<size_t>(ri) * nl;
  if (len <= len_grid[0]) return row[0];
  if (len >= len_grid[nl - 1]) {
    const int64_t c0 = row[nl - 2], c1 = row[nl - 1];
    return c1 + (c1 - c0) * (len - len_grid[nl - 1]) / (len_grid[nl - 1] - len_grid[nl - 2]);
  }
  const int j = static_cast<int>(std::upper_bound(len_grid.begin(), len_grid.end(), len) - len_grid.begin()) - 1;
  const int64_t c0 = row[j], c1 = row[j + 1];
  return c0 + (c1 - c0) * (len - len_grid[j]) / (len_grid[j + 1] - len_grid[j]);
}

// A fallback when no profiled table is given: per-piece launch/setup time
// plus the larger of the KV streaming time at one compute unit's share of
// HBM bandwidth and the matrix-core time at one compute unit's share of the
// peak, per kv head.  Only a placeholder for the profiled gfx950 table.
CostModel analytic_cost_model(int32_t g, int32_t head_dim, int32_t elem_bytes) {
  (void)g;
  CostModel c;
  for (int r = 1; r <= kMaxRows; r *= 2) c.rows_grid.push_back(r);
  for (int l = 16; l <= 65536; l *= 2) c.len_grid.push_back(l);
  const double bytes_per_token = 2.0 * head_dim * elem_bytes;
  const double cu_bw = 8.0e12 / 256 / 1e9;   // bytes per ns per compute unit
  const double cu_flops = 2.5e15 / 256 / 1e9;  // flop per ns per compute unit
  for (int r : c.rows_grid) {
    for (int l : c.len_grid) {
      const double mem = l * bytes_per_token / cu_bw;
      const double flop = 4.0 * head_dim * static_cast<double>(r) * l / cu_flops;
      c.table.push_back(static_cast<int64_t>(3000.0 + std::max(mem, flop)));
    }
  }
  return c;
}

namespace {

struct PNode {
  int32_t i;
  int64_t n, rows, gq, rpg, last_rows, bmax;
};

inline int64_t lp_of(int64_t n, int64_t b, int64_t G) { return cdiv(cdiv(n, b), G) * G; }

int64_t cost_with_lp(const CostModel& c, const PNode& nd, int64_t Lp) {
  const int64_t beff = cdiv(nd.n, Lp);
  const int64_t last_len = nd.n - (beff - 1) * Lp;
  int64_t total = 0;
  if (nd.gq - 1 > 0) total += (nd.gq - 1) * ((beff - 1) * c.lookup(nd.rpg, Lp) + c.lookup(nd.rpg, last_len));
  total += (beff - 1) * c.lookup(nd.last_rows, Lp) + c.lookup(nd.last_rows, last_len);
  return total;
}

int64_t b_of_T(const CostModel& c, const PNode& nd, int64_t T, int64_t G) {
  auto f = [&](int64_t b) { return c.lookup(nd.rpg, std::min(lp_of(nd.n, b, G), nd.n)); };
  if (f(nd.bmax) > T) return nd.bmax;
  int64_t lo = 1, hi = nd.bmax;
  while (lo < hi) {
    const int64_t mid = (lo + hi) / 2;
    if (f(mid) <= T)
      hi = mid;
    else
      lo = mid + 1;
  }
  return lo;
}

struct Item {
  int64_t cost;
  int32_t node, group, piece;
};

void lpt(std::vector<Item>& items, int32_t m, std::vector<std::vector<Item>>* bins, std::vector<int64_t>* loads) {
  std::sort(items.begin(), items.end(), [](const Item& a, const Item& b) {
    if (a.cost != b.cost) return a.cost > b.cost;
    if (a.node != b.node) return a.node < b.node;
    if (a.group != b.group) return a.group < b.group;
    return a.piece < b.piece;
  });
  using E = std::pair<int64_t, int32_t>;
  std::priority_queue<E, std::vector<E>, std::greater<E>> heap;
  for (int32_t b = 0; b < m; ++b) heap.push({0, b});
  bins->assign(m, {});
  loads->assign(m, 0);
  for (const Item& it : items) {
    E top = heap.top();
    heap.pop();
    (*bins)[top.second].push_back(it);
    top.first += it.cost;
    (*loads)[top.second] = top.first;
    heap.push(top);
  }
}

}  // namespace

// Uniform piece lengths G x {1, 2, 3, 4, 6, 8, 12, 16, ...} in increasing
// order, up to and including the first one that holds the longest node.
static std::vector<int64_t> uniform_lengths(const std::vector<PNode>& nodes, int64_t G) {
  int64_t nmax = 0;
  for (const PNode& nd : nodes) nmax = std::max(nmax, nd.n);
  std::vector<int64_t> us;
  for (int64_t p = 1;; p *= 2) {
    us.push_back(G * p);
    if (G * p >= nmax) break;
    if (p >= 2) {
      us.push_back(G * p * 3 / 2);
      if (G * p * 3 / 2 >= nmax) break;
    }
  }
  return us;
}

pst_status build_plan(const TreeIndex& ix, int32_t g, const CostModel& cost, const PlanOptions& o,
                      PlanResult* out) {
  const int64_t G = o.tile;
  const int32_t m = o.m;
  const int64_t r_max = o.query_guided ? g : o.r_max;
  const int32_t N = ix.N, B = ix.B;
  std::vector<PNode> nodes;
  for (int32_t i = 0; i < N; ++i) {
    if (ix.n_q[i] == 0) continue;
    PNode nd;
    nd.i = i;
    nd.n = ix.kv_len[i];
    nd.rows = static_cast<int64_t>(ix.n_q[i]) * g;
    nd.gq = cdiv(nd.rows, r_max);
    nd.rpg = cdiv(nd.rows, nd.gq);
    nd.last_rows = nd.rows - (nd.gq - 1) * nd.rpg;
    nd.bmax = cdiv(nd.n, G);
    nodes.push_back(nd);
  }

  std::vector<std::vector<int64_t>> candidates;  // piece length per entry of `nodes`
  if (nodes.empty()) {
  } else if (o.no_split || o.fixed_chunk > 0) {
    std::vector<int64_t> lps;
    for (const PNode& nd : nodes) lps.push_back(o.fixed_chunk > 0 ? o.fixed_chunk : lp_of(nd.n, 1, G));
    candidates.push_back(lps);
  } else {
    // least[a][b] = min over b' in [b, bmax] of cost(node a, b'): a makespan
    // of T allows any split into b(T) or more pieces, so W(T), the least
    // total work at T, takes the cheapest of them (cost is not monotone in b
    // under every table).
    std::vector<std::vector<int64_t>> least(nodes.size());
    for (size_t a = 0; a < nodes.size(); ++a) {
      const PNode& nd = nodes[a];
      least[a].assign(nd.bmax + 2, 0);
      for (int64_t b = nd.bmax; b >= 1; --b) {
        const int64_t c = cost_with_lp(cost, nd, lp_of(nd.n, b, G));
        least[a][b] = b == nd.bmax ? c : std::min(c, least[a][b + 1]);
      }
    }
    auto W = [&](int64_t T) {
      int64_t w = 0;
      for (size_t a = 0; a < nodes.size(); ++a) w += least[a][b_of_T(cost, nodes[a], T, G)];
      return w;
    };
    int64_t lo = 0, hi = 0;
    for (const PNode& nd : nodes) {
      lo = std::max(lo, cost.lookup(nd.rpg, std::min<int64_t>(nd.n, G)));
      hi += cost_with_lp(cost, nd, lp_of(nd.n, 1, G));
    }
    while (lo < hi) {
      const int64_t mid = lo + (hi - lo) / 2;
      if (static_cast<int64_t>(m) * mid >= W(mid))
        hi = mid;
      else
        lo = mid + 1;
    }
    const int64_t cost_l = lo;
    out->cost_l = cost_l;
    std::vector<int64_t> ub;
    for (const PNode& nd : nodes)
      ub.push_back(std::min(nd.bmax, std::max<int64_t>(1, cdiv(cost.lookup(nd.rpg, nd.n), cost_l))));
    for (int32_t k = 0; k <= o.grid_steps; ++k) {
      const int64_t T = cost_l + (cost_l * k) / o.grid_steps;
      std::vector<int64_t> lps;
      for (size_t a = 0; a < nodes.size(); ++a)
        lps.push_back(lp_of(nodes[a].n, std::min(ub[a], b_of_T(cost, nodes[a], T, G)), G));
      candidates.push_back(lps);
    }
    // Candidates with one piece length for every node: U = G x {1, 2, 3, 4,
    // 6, 8, 12, ...}, up to the first U that holds the longest node.
    for (const int64_t u : uniform_lengths(nodes, G)) candidates.push_back(std::vector<int64_t>(nodes.size(), u));
  }

  std::vector<std::vector<Item>> best_bins(m);
  std::vector<int64_t> best_loads(m, 0), best_lps;
  int64_t best_span = -1, best_count = 0;
  int32_t best_k = 0;
  for (size_t k = 0; k < candidates.size(); ++k) {
    const std::vector<int64_t>& lps = candidates[k];
    std::vector<Item> items;
    for (size_t a = 0; a < nodes.size(); ++a) {
      const PNode& nd = nodes[a];
      const int64_t Lp = lps[a];
      const int64_t beff = cdiv(nd.n, Lp);
      for (int64_t gi = 0; gi < nd.gq; ++gi) {
        const int64_t rows = gi < nd.gq - 1 ? nd.rpg : nd.last_rows;
        for (int64_t p = 0; p < beff; ++p) {
          const int64_t plen = std::min(Lp, nd.n - p * Lp);
          items.push_back({cost.lookup(rows, plen), nd.i, static_cast<int32_t>(gi), static_cast<int32_t>(p)});
        }
      }
    }
    std::vector<std::vector<Item>> bins;
    std::vector<int64_t> loads;
    const int64_t count = static_cast<int64_t>(items.size());
    lpt(items, m, &bins, &loads);
    const int64_t span = *std::max_element(loads.begin(), loads.end());
    const bool better = best_span < 0 || span < best_span || (span == best_span && count < best_count);
    if (better) {
      best_span = span;
      best_count = count;
      best_k = static_cast<int32_t>(k);
      best_bins = std::move(bins);
      best_loads = std::move(loads);
      best_lps = lps;
    }
  }

  out->chosen_k = best_k;
  out->bin_load = best_loads;
  out->makespan = nodes.empty() ? 0 : best_span;
  out->piece_len.assign(N, 0);
  out->b_eff.assign(N, 0);
  out->rows_per_group.assign(N, 0);
  std::vector<const PNode*> by_id(N, nullptr);
  for (size_t a = 0; a < nodes.size(); ++a) {
    const PNode& nd = nodes[a];
    by_id[nd.i] = &nd;
    out->piece_len[nd.i] = static_cast<int32_t>(best_lps[a]);
    out->b_eff[nd.i] = static_cast<int32_t>(cdiv(nd.n, best_lps[a]));
    out->rows_per_group[nd.i] = static_cast<int32_t>(nd.rpg);
  }
  out->tasks.clear();
  out->bin_ptr.assign(m + 1, 0);
  for (int32_t b = 0; b < m; ++b) {
    for (const Item& it : best_bins[b]) {
      const PNode& nd = *by_id[it.node];
      const int64_t Lp = out->piece_len[it.node];
      Task t;
      t.node = it.node;
      t.piece = it.piece;
      t.kv_begin = static_cast<int32_t>(it.piece * Lp);
      t.kv_len = static_cast<int32_t>(std::min<int64_t>(Lp, nd.n - it.piece * Lp));
      t.row_begin = static_cast<int32_t>(it.group * nd.rpg);
      t.row_count = static_cast<int32_t>(std::min<int64_t>(nd.rpg, nd.rows - t.row_begin));
      t.flags = it.piece == out->b_eff[it.node] - 1 ? PST_TASK_LAST_PIECE : 0;
      t.reserved = 0;
      out->tasks.push_back(t);
    }
    out->bin_ptr[b + 1] = static_cast<int32_t>(out->tasks.size());
  }

  out->slot_ptr.assign(B + 1, 0);
  out->entry_slot.assign(ix.qn_idx.size(), 0);
  std::vector<int64_t> cursor(ix.nq_ptr.begin(), ix.nq_ptr.end());
  for (int32_t r = 0; r < B; ++r) {
    int64_t off = out->slot_ptr[r];
    for (int32_t e = ix.qn_ptr[r]; e < ix.qn_ptr[r + 1]; ++e) {
      const int32_t i = ix.qn_idx[e];
      out->entry_slot[cursor[i]++] = off;
      off += out->b_eff[i];
    }
    out->slot_ptr[r + 1] = off;
  }
  return PST_OK;
}


// DEFT: Decoding with Flash Tree-Attention, section 3.3 (remark 3.1, Fig.
// 3(c)) and appendix A.9: depth-first flattening of the tree KV, chunks of
// S_t tokens, one group per chunk with every query that sees any of its
// tokens and a 64-bit bit causal mask per (query, 64 tokens).  The reading
// (traversal order, entry order, mask words, row groups, assignment, slots)
// is the one stated with PST_PLAN_FLATTEN in pst.h, identical to the CPU
// oracle's.
pst_status build_flat_plan(const TreeIndex& ix, int32_t g, const CostModel& cost, const PlanOptions& o,
                           PlanResult* out) {
  const int32_t N = ix.N, B = ix.B, m = o.m;
  const int64_t S = o.flat_chunk;
  if (m < 1 || S <= 0 || S % 128 != 0) {
    set_error("flattened plans need num_bins >= 1 and a chunk length that is a positive multiple of 128");
    return PST_E_INVALID_ARG;
  }
  const int64_t W = S / 64;
  const int64_t e_max = std::min<int64_t>(o.r_max / g, kMaskWordsMax / W);
  if (e_max < 1) {
    set_error("the chunk's masks or the GQA group do not fit one workgroup (lower the chunk length)");
    return PST_E_UNSUPPORTED;
  }
  // 1. Depth-first pre-order over the nodes some query sees.
  std::vector<std::vector<int32_t>> children(N);
  std::vector<int32_t> stack, order;
  for (int32_t i = N - 1; i >= 0; --i) {
    if (ix.parent[i] < 0)
      stack.push_back(i);
    else
      children[ix.parent[i]].push_back(i);
  }
  // Roots and children were collected from high id to low: pushed in that
  // order, the lowest id is popped first.
  while (!stack.empty()) {
    const int32_t i = stack.back();
    stack.pop_back();
    if (ix.n_q[i] == 0) continue;
    order.push_back(i);
    for (int32_t c : children[i]) stack.push_back(c);
  }
  int64_t total = 0;
  for (int32_t i : order) total += ix.kv_len[i];
  const int64_t nchunks = cdiv(total, S);
  if (nchunks * S > INT32_MAX) {
    set_error("the flattened tree is too long");
    return PST_E_UNSUPPORTED;
  }
  // 8. Pool row of every flattened token.
  out->flat_chunk = static_cast<int32_t>(S);
  out->flat_rows.assign(static_cast<size_t>(nchunks * S), -1);
  {
    int64_t t = 0;
    for (int32_t i : order) {
      for (int32_t j = 0; j < ix.kv_len[i]; ++j, ++t) {
        int64_t row;
        if (ix.page_size > 0)
          row = static_cast<int64_t>(ix.page_idx[ix.page_ptr[i] + j / ix.page_size]) * ix.page_size + j % ix.page_size;
        else
          row = ix.kv_offset[i] + j;
        if (row > INT32_MAX) {
          set_error("a pool row beyond 2^31 - 1");
          return PST_E_UNSUPPORTED;
        }
        out->flat_rows[t] = static_cast<int32_t>(row);
      }
    }
  }
  // 2-4. Chunks, their entries and masks, by node segments.
  out->flat_ptr.assign(nchunks + 1, 0);
  out->flat_query.clear();
  out->flat_mask.clear();
  std::vector<int64_t> chunk_len(nchunks, 0);
  std::vector<uint64_t> words(static_cast<size_t>(B) * W, 0);
  std::vector<uint8_t> seen(B, 0);
  std::vector<int32_t> touched;
  size_t seg = 0;      // index into order
  int64_t seg_pos = 0;  // tokens of order[seg] already in earlier chunks
  for (int64_t c = 0; c < nchunks; ++c) {
    int64_t t0 = 0;  // chunk-relative position
    const int64_t len = std::min<int64_t>(S, total - c * S);
    chunk_len[c] = len;
    while (t0 < len) {
      const int32_t i = order[seg];
      const int64_t take = std::min<int64_t>(ix.kv_len[i] - seg_pos, len - t0);
      for (int32_t e = ix.nq_ptr[i]; e < ix.nq_ptr[i + 1]; ++e) {
        const int32_t r = ix.nq_idx[e];
        uint64_t* w = words.data() + static_cast<size_t>(r) * W;
        bool any = false;
        for (int64_t k = 0; k < take; ++k) {
          const int64_t j = seg_pos + k;
          if (ix.masked[i] && !((ix.nq_mask[e] >> j) & 1ull)) continue;
          const int64_t tt = t0 + k;
          w[tt >> 6] |= 1ull << (tt & 63);
          any = true;
        }
        if (any && !seen[r]) {
          seen[r] = 1;
          touched.push_back(r);
        }
      }
      t0 += take;
      seg_pos += take;
      if (seg_pos == ix.kv_len[i]) {
        ++seg;
        seg_pos = 0;
      }
    }
    std::sort(touched.begin(), touched.end());
    for (int32_t r : touched) {
      out->flat_query.push_back(r);
      uint64_t* w = words.data() + static_cast<size_t>(r) * W;
      out->flat_mask.insert(out->flat_mask.end(), w, w + W);
      std::fill(w, w + W, 0ull);
      seen[r] = 0;
    }
    touched.clear();
    out->flat_ptr[c + 1] = static_cast<int32_t>(out->flat_query.size());
  }
  // 5-6. Row groups of whole entries, placed by LPT.
  std::vector<int64_t> epg(nchunks, 0);
  std::vector<Item> items;
  for (int64_t c = 0; c < nchunks; ++c) {
    const int64_t ne = out->flat_ptr[c + 1] - out->flat_ptr[c];
    if (ne == 0) continue;
    const int64_t gq = cdiv(ne, e_max);
    epg[c] = cdiv(ne, gq);
    for (int64_t k = 0; k < gq; ++k) {
      const int64_t n_ent = std::min<int64_t>(epg[c], ne - k * epg[c]);
      items.push_back({cost.lookup(n_ent * g, chunk_len[c]), static_cast<int32_t>(c), static_cast<int32_t>(k), 0});
    }
  }
  std::vector<std::vector<Item>> bins;
  std::vector<int64_t> loads;
  lpt(items, m, &bins, &loads);
  out->bin_load = loads;
  out->makespan = loads.empty() ? 0 : *std::max_element(loads.begin(), loads.end());
  out->cost_l = 0;
  out->chosen_k = 0;
  out->piece_len.assign(N, 0);
  out->b_eff.assign(N, 0);
  out->rows_per_group.assign(N, 0);
  out->tasks.clear();
  out->bin_ptr.assign(m + 1, 0);
  for (int32_t b = 0; b < m; ++b) {
    for (const Item& it : bins[b]) {
      const int64_t c = it.node;
      const int64_t ne = out->flat_ptr[c + 1] - out->flat_ptr[c];
      const int64_t n_ent = std::min<int64_t>(epg[c], ne - it.group * epg[c]);
      Task t;
      t.node = static_cast<int32_t>(c);
      t.piece = 0;
      t.kv_begin = static_cast<int32_t>(c * S);
      t.kv_len = static_cast<int32_t>(chunk_len[c]);
      t.row_begin = static_cast<int32_t>(it.group * epg[c] * g);
      t.row_count = static_cast<int32_t>(n_ent * g);
      t.flags = PST_TASK_FLAT;
      t.reserved = 0;
      out->tasks.push_back(t);
    }
    out->bin_ptr[b + 1] = static_cast<int32_t>(out->tasks.size());
  }
  // 7. One slot per (query, chunk), a query's in chunk order.
  out->slot_ptr.assign(B + 1, 0);
  for (int32_t r : out->flat_query) out->slot_ptr[r + 1]++;
  for (int32_t r = 0; r < B; ++r) out->slot_ptr[r + 1] += out->slot_ptr[r];
  std::vector<int64_t> cursor(out->slot_ptr.begin(), out->slot_ptr.end() - 1);
  out->entry_slot.resize(out->flat_query.size());
  for (size_t e = 0; e < out->flat_query.size(); ++e) out->entry_slot[e] = cursor[out->flat_query[e]]++;
  return PST_OK;
}

}  // namespace pst
