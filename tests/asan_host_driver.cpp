// Host-only exercise of the C ABI for an AddressSanitizer / UBSan build.
//
// Compiled by tests/test_asan_host.py with g++ together with the library's
// host sources (api.cpp, host_tree.cpp, host_plan.cpp, cost_json.cpp); the
// kernel launchers live in the .hip sources, so this file supplies stand-ins
// that fail if called (nothing here asks for a device).  It walks trees,
// plans, views, growth and every error path that the host can force, so
// that a use-after-free, an out-of-bounds access or undefined behaviour in
// those paths stops the run with the sanitizer's report.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "pst.h"
#include "pst_internal.h"

namespace pst {
int launch_pac(const PacParams&, int, int, void*) { return 1; }
int launch_por(const PorParams&, int, int, void*) { return 1; }
int launch_flush(void*, size_t, void*) { return 1; }
int launch_read(const void*, size_t, float*, void*) { return 1; }
int launch_write_rows(const KvRowsParams&, void*) { return 1; }
int launch_append(const AppendParams&, void*) { return 1; }
int pac_blocks_per_cu(int, int, int*) { return 1; }
size_t pac_lds_bytes() { return 0; }
}  // namespace pst

static int g_fail = 0;
#define EXPECT(cond)                                                        \
  do {                                                                      \
    if (!(cond)) {                                                          \
      std::fprintf(stderr, "%s:%d: expectation failed: %s (last error: %s)\n", __FILE__, __LINE__, #cond, \
                   pst_last_error());                                       \
      ++g_fail;                                                             \
    }                                                                       \
  } while (0)

struct Lcg {
  uint64_t s;
  uint32_t next() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return static_cast<uint32_t>(s >> 33);
  }
  int range(int lo, int hi) { return lo + static_cast<int>(next() % static_cast<uint32_t>(hi - lo + 1)); }
};

struct HostTree {
  std::vector<int32_t> parent, len, qnode, page_ptr, page_idx;
  std::vector<int64_t> off;
  std::vector<uint64_t> qmask;
  std::vector<uint8_t> masked;
  int32_t page = 0;
  pst_tree_desc desc() const {
    pst_tree_desc d{};
    d.num_nodes = static_cast<int32_t>(parent.size());
    d.parent = parent.data();
    d.kv_offset = page ? nullptr : off.data();
    d.kv_len = len.data();
    d.num_queries = static_cast<int32_t>(qnode.size());
    d.query_node = qnode.data();
    d.query_mask = qmask.empty() ? nullptr : qmask.data();
    d.node_masked = masked.empty() ? nullptr : masked.data();
    d.page_size = page;
    d.page_ptr = page ? page_ptr.data() : nullptr;
    d.page_idx = page ? page_idx.data() : nullptr;
    return d;
  }
};

static HostTree random_tree(Lcg& r, bool paged, bool with_masks) {
  HostTree t;
  const int N = r.range(1, 12);
  int64_t pos = 0;
  for (int i = 0; i < N; ++i) {
    t.parent.push_back(i == 0 ? -1 : r.range(-1, i - 1));
    const bool m = with_masks && i > 0 && r.range(0, 2) == 0;
    t.masked.push_back(m ? 1 : 0);
    t.len.push_back(m ? r.range(1, 64) : r.range(1, 700));
    t.off.push_back(pos);
    pos += t.len.back() + r.range(0, 9);
  }
  const int B = r.range(1, 20);
  for (int q = 0; q < B; ++q) {
    const int n = r.range(0, N - 1);
    t.qnode.push_back(n);
    const int L = t.len[n];
    uint64_t bits = L >= 64 ? ~0ull : ((1ull << L) - 1);
    bits &= (static_cast<uint64_t>(r.next()) << 32) | r.next();
    if (bits == 0) bits = 1;
    t.qmask.push_back(bits);
  }
  if (!with_masks) {
    t.masked.clear();
    t.qmask.clear();
  }
  if (paged) {
    t.page = 1 << r.range(3, 7);
    t.page_ptr.push_back(0);
    int next_page = 0;
    for (int i = 0; i < N; ++i) {
      const int pages = (t.len[i] + t.page - 1) / t.page + r.range(0, 2);
      for (int k = 0; k < pages; ++k) t.page_idx.push_back(next_page++ * 3 % 1000 + r.range(0, 1) * 1000);
      t.page_ptr.push_back(static_cast<int32_t>(t.page_idx.size()));
    }
  }
  return t;
}

static pst_shape shape(int hq, int hkv, int d, int dt) {
  pst_shape s{};
  s.num_q_heads = hq;
  s.num_kv_heads = hkv;
  s.head_dim = d;
  s.in_dtype = dt;
  s.out_dtype = dt;
  return s;
}

static pst_cost_model_t affine_cost() {
  std::vector<int32_t> rows, lens;
  for (int r = 1; r <= 256; r *= 2) rows.push_back(r);
  for (int l = 16; l <= 65536; l *= 2) lens.push_back(l);
  std::vector<int64_t> tab;
  for (int r : rows)
    for (int l : lens) tab.push_back(900 + 3 * r + 2 * static_cast<int64_t>(l));
  pst_cost_model_t c = nullptr;
  EXPECT(pst_cost_model_create(static_cast<int32_t>(rows.size()), rows.data(), static_cast<int32_t>(lens.size()),
                               lens.data(), tab.data(), &c) == PST_OK);
  return c;
}

static void walk_plans(pst_tree_t t, pst_cost_model_t cost, int g, Lcg& r, bool bf16) {
  const uint32_t flag_sets[] = {0u, PST_PLAN_QUERY_GUIDED, PST_PLAN_NO_SPLIT, PST_PLAN_DOT_SMALL, PST_PLAN_FLATTEN};
  for (uint32_t extra : flag_sets) {
    pst_plan_opts o{};
    o.num_bins = r.range(1, 40);
    o.flags = PST_PLAN_HOST_ONLY | extra;
    o.max_rows = bf16 ? (r.range(0, 1) ? 0 : 64) : 16;
    if (extra == PST_PLAN_FLATTEN) o.fixed_chunk = 128 * r.range(1, 4);
    if (extra == 0 && r.range(0, 2) == 0) o.fixed_chunk = 64 * r.range(1, 5);
    if (extra == PST_PLAN_QUERY_GUIDED && (!bf16 && g > 16)) continue;
    pst_plan_t p = nullptr;
    const pst_status st = pst_plan(t, r.range(0, 1) ? cost : nullptr, &o, nullptr, &p);
    if (st != PST_OK) {
      EXPECT(p == nullptr);
      continue;
    }
    pst_plan_view v{};
    EXPECT(pst_plan_get(p, &v) == PST_OK);
    int64_t pieces = 0;
    for (int32_t b = 0; b < v.num_bins; ++b) pieces += v.bin_ptr[b + 1] - v.bin_ptr[b];
    EXPECT(pieces == v.num_tasks);
    size_t ws = 0;
    EXPECT(pst_plan_workspace_size(p, &ws) == PST_OK);
    EXPECT(pst_decode_attn(p, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) == PST_E_NO_DEVICE);
    EXPECT(pst_free(p) == PST_OK);
  }
}

static void valid_trees() {
  Lcg r{12345};
  pst_cost_model_t cost = affine_cost();
  for (int it = 0; it < 300; ++it) {
    const bool paged = it % 3 == 1, masks = it % 4 == 0, bf16 = it % 2 == 0;
    HostTree h = random_tree(r, paged, masks);
    const pst_tree_desc d = h.desc();
    const int hkv = bf16 ? 2 : 1;
    const int g = bf16 ? (1 << r.range(0, 4)) : r.range(1, 4);
    pst_shape s = shape(hkv * g, hkv, it % 5 == 0 ? 64 : 128, bf16 ? PST_BF16 : PST_F32);
    if (!paged) s.pool_tokens = h.off.back() + h.len.back() + 8;  // room for the last node to grow
    pst_tree_t t = nullptr;
    const pst_status st = pst_tree_build(&d, &s, PST_TREE_HOST_ONLY, nullptr, &t);
    if (st != PST_OK) {  // a random query on a masked node may see nothing
      EXPECT(t == nullptr);
      continue;
    }
    pst_index_view ix{};
    EXPECT(pst_tree_get_index(t, &ix) == PST_OK);
    EXPECT(ix.num_nodes == d.num_nodes && ix.num_queries == d.num_queries);
    walk_plans(t, cost, g, r, bf16);
    // A live plan, then growth of every unmasked node by one token where the layout has room.
    pst_plan_opts o{};
    o.num_bins = 8;
    o.flags = PST_PLAN_HOST_ONLY;
    if (!bf16) o.max_rows = 16;
    pst_plan_t p = nullptr;
    if (pst_plan(t, cost, &o, nullptr, &p) == PST_OK) {
      EXPECT(pst_free(t) == PST_E_INVALID_ARG);  // the plan borrows the tree
      std::vector<int32_t> grown(h.len);
      for (size_t i = 0; i < grown.size(); ++i) {
        const bool m = !h.masked.empty() && h.masked[i];
        const int64_t cap = paged ? static_cast<int64_t>(h.page_ptr[i + 1] - h.page_ptr[i]) * h.page : -1;
        if (!m && (!paged || grown[i] + 1 <= cap) && (paged || i + 1 == grown.size())) grown[i] += 1;
      }
      EXPECT(pst_tree_set_lengths(t, grown.data(), nullptr) == PST_OK);
      std::vector<int32_t> shrunk(grown);
      shrunk[0] -= 1;
      EXPECT(pst_tree_set_lengths(t, shrunk.data(), nullptr) == PST_E_INVALID_ARG);
      EXPECT(pst_free(p) == PST_OK);
    }
    EXPECT(pst_decode_attn_baseline(t, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr) ==
           PST_E_NO_DEVICE);
    EXPECT(pst_write_kv_rows(t, nullptr, nullptr, nullptr, 0, nullptr, nullptr, nullptr) == PST_E_NO_DEVICE);
    {
      // pst_tree_append's checks run before it asks for the device.
      int dummy = 0;
      std::vector<int32_t> all;
      for (int32_t i = 0; i < d.num_nodes; ++i) all.push_back(i);
      const pst_status a = pst_tree_append(t, static_cast<int32_t>(all.size()), all.data(), &dummy, &dummy, &dummy,
                                           &dummy, nullptr);
      EXPECT(a == PST_E_NO_DEVICE || a == PST_E_INVALID_TREE);  // full pages, masked nodes at 64, pool end
      const int32_t twice[2] = {0, 0};
      EXPECT(pst_tree_append(t, 2, twice, &dummy, &dummy, &dummy, &dummy, nullptr) == PST_E_INVALID_ARG);
      const int32_t outside[1] = {d.num_nodes};
      EXPECT(pst_tree_append(t, 1, outside, &dummy, &dummy, &dummy, &dummy, nullptr) == PST_E_INVALID_ARG);
    }
    EXPECT(pst_write_kv_rows(t, nullptr, nullptr, nullptr, -1, nullptr, nullptr, nullptr) == PST_E_INVALID_ARG);
    EXPECT(pst_free(t) == PST_OK);
  }
  EXPECT(pst_free(cost) == PST_OK);
}

static pst_status build_once(const HostTree& h, int64_t pool_tokens) {
  pst_tree_desc d = h.desc();
  pst_shape s = shape(2, 1, 64, PST_F32);
  s.pool_tokens = pool_tokens;
  pst_tree_t t = nullptr;
  const pst_status st = pst_tree_build(&d, &s, PST_TREE_HOST_ONLY, nullptr, &t);
  if (st == PST_OK) pst_free(t);
  else EXPECT(t == nullptr);
  return st;
}

static void error_paths() {
  HostTree base;
  base.parent = {-1, 0, 0};
  base.len = {4, 2, 3};
  base.off = {0, 4, 6};
  base.qnode = {1, 2};
  EXPECT(build_once(base, 0) == PST_OK);
  EXPECT(build_once(base, 8) == PST_E_INVALID_TREE);  // contiguous node outside the pool (message after free)
  {
    HostTree h = base;
    h.parent = {-1, 2, 0};
    EXPECT(build_once(h, 0) == PST_E_INVALID_TREE);
    h = base;
    h.len = {4, 0, 3};
    EXPECT(build_once(h, 0) == PST_E_INVALID_TREE);
    h = base;
    h.off = {0, -1, 9};
    EXPECT(build_once(h, 0) == PST_E_INVALID_TREE);
    h = base;
    h.qnode = {1, 5};
    EXPECT(build_once(h, 0) == PST_E_INVALID_TREE);
    h = base;
    h.len = {4, 65, 3};
    h.masked = {0, 1, 0};
    h.qmask = {1, 0};
    EXPECT(build_once(h, 0) == PST_E_INVALID_TREE);
    h = base;
    h.masked = {0, 1, 0};
    h.qmask = {4, 0};
    EXPECT(build_once(h, 0) == PST_E_INVALID_TREE);
    h = base;
    h.parent = {-1, -1, 0};
    h.masked = {0, 1, 0};
    h.qmask = {0, 0};
    EXPECT(build_once(h, 0) == PST_E_INVALID_TREE);
  }
  {
    HostTree h;
    h.parent = {-1, 0, 0};
    h.len = {20, 9, 3};
    h.qnode = {1, 2};
    h.page = 8;
    h.page_ptr = {0, 3, 5, 6};
    h.page_idx = {7, 2, 9, 0, 4, 11};
    EXPECT(build_once(h, 0) == PST_OK);
    EXPECT(build_once(h, 64) == PST_E_INVALID_TREE);  // paged: page outside the pool (message after free)
    HostTree b = h;
    b.page = 12;
    EXPECT(build_once(b, 0) == PST_E_INVALID_ARG);
    b = h;
    b.page_ptr = {0, 2, 4, 6};
    EXPECT(build_once(b, 0) == PST_E_INVALID_TREE);
    b = h;
    b.page_idx = {7, 2, -1, 0, 4, 11};
    EXPECT(build_once(b, 0) == PST_E_INVALID_TREE);
  }
  {
    pst_tree_desc d = base.desc();
    pst_shape s = shape(3, 2, 64, PST_F32);
    pst_tree_t t = nullptr;
    EXPECT(pst_tree_build(&d, &s, PST_TREE_HOST_ONLY, nullptr, &t) == PST_E_UNSUPPORTED && !t);
    s = shape(4, 4, 96, PST_F32);
    EXPECT(pst_tree_build(&d, &s, PST_TREE_HOST_ONLY, nullptr, &t) == PST_E_UNSUPPORTED && !t);
    EXPECT(pst_tree_build(nullptr, &s, PST_TREE_HOST_ONLY, nullptr, &t) == PST_E_INVALID_ARG);
    s = shape(2, 1, 64, PST_F32);
    s.kv_stride_token = 10;
    EXPECT(pst_tree_build(&d, &s, PST_TREE_HOST_ONLY, nullptr, &t) == PST_E_INVALID_ARG && !t);
    s = shape(2, 1, 64, PST_F32);
    EXPECT(pst_tree_build(&d, &s, PST_TREE_HOST_ONLY, nullptr, &t) == PST_OK);
    pst_plan_opts o{};
    o.flags = PST_PLAN_HOST_ONLY;
    o.tile = 100;
    pst_plan_t p = nullptr;
    EXPECT(pst_plan(t, nullptr, &o, nullptr, &p) == PST_E_INVALID_ARG && !p);
    o.tile = 0;
    o.max_rows = 64;
    EXPECT(pst_plan(t, nullptr, &o, nullptr, &p) == PST_E_UNSUPPORTED && !p);
    o.max_rows = 0;
    o.flags = PST_PLAN_HOST_ONLY | PST_PLAN_FLATTEN;
    o.fixed_chunk = 192;
    EXPECT(pst_plan(t, nullptr, &o, nullptr, &p) == PST_E_INVALID_ARG && !p);
    o.fixed_chunk = 256;
    o.num_bins = 3;
    EXPECT(pst_plan(t, nullptr, &o, nullptr, &p) == PST_OK);
    const int32_t same[3] = {4, 2, 3};
    EXPECT(pst_tree_set_lengths(t, same, nullptr) == PST_E_UNSUPPORTED);  // flattened plan live
    EXPECT(pst_free(p) == PST_OK);
    EXPECT(pst_tree_set_lengths(t, same, nullptr) == PST_OK);
    const int32_t beyond[3] = {4, 2, 30};
    EXPECT(pst_tree_set_lengths(t, beyond, nullptr) == PST_E_INVALID_TREE);
    EXPECT(pst_free(t) == PST_OK);
  }
  {
    const int32_t rows[2] = {1, 2}, lens[2] = {16, 32};
    const int64_t bad[4] = {5, 4, 6, 7};
    pst_cost_model_t c = nullptr;
    EXPECT(pst_cost_model_create(2, rows, 2, lens, bad, &c) == PST_E_INVALID_ARG && !c);
    const int32_t rows_desc[2] = {2, 1};
    const int64_t good[4] = {5, 6, 6, 7};
    EXPECT(pst_cost_model_create(2, rows_desc, 2, lens, good, &c) == PST_E_INVALID_ARG && !c);
    EXPECT(pst_cost_model_create(2, rows, 2, lens, good, &c) == PST_OK);
    int64_t ns = 0;
    EXPECT(pst_cost_model_lookup(c, 1, 24, &ns) == PST_OK && ns == 5);
    EXPECT(pst_free(c) == PST_OK);
  }
  {
    const char* dir = std::getenv("PST_ASAN_TMP");
    const std::string base_path = std::string(dir ? dir : "/tmp") + "/pst_asan_cost";
    const char* texts[] = {
        "{\"rows_grid\": [1, 2], \"len_grid\": [16, 32], \"table_ns\": [[5, 6], [6, 7]], \"note\": [1.5e3, null]}",
        "{\"rows_grid\": [1, 2], \"len_grid\": [16, 32], \"table_ns\": [[5, 6]]}",
        "{\"rows_grid\": [1], \"len_grid\": [16, 32], \"table_ns\": [[5, 6.5]]}",
        "{\"rows_grid\": [1], \"len_grid\": [16, 32], \"table_ns\": [[5, 6]] trailing",
        "{\"rows_grid\": [1], \"len_grid\": [16, 32], \"table_ns\": [[5, 6]], \"s\": \"\\u12\"}",
        "{\"rows_grid\": [1], \"len_grid\": [16, 32], \"table_ns\": [[5, 6]], \"deep\": [[[[[[[[[[[]]]]]]]]]]]}",
        "[", "", "{\"rows_grid\": [99999999999], \"len_grid\": [16, 32], \"table_ns\": [[5, 6]]}",
    };
    const pst_status want[] = {PST_OK, PST_E_INVALID_ARG, PST_E_INVALID_ARG, PST_E_INVALID_ARG, PST_E_INVALID_ARG,
                               PST_OK, PST_E_INVALID_ARG, PST_E_INVALID_ARG, PST_E_INVALID_ARG};
    for (size_t i = 0; i < sizeof(texts) / sizeof(texts[0]); ++i) {
      const std::string path = base_path + std::to_string(i) + ".json";
      std::FILE* f = std::fopen(path.c_str(), "wb");
      if (!f) {
        ++g_fail;
        continue;
      }
      std::fputs(texts[i], f);
      std::fclose(f);
      pst_cost_model_t c = nullptr;
      const pst_status st = pst_cost_model_load(path.c_str(), &c);
      EXPECT(st == want[i]);
      EXPECT((st == PST_OK) == (c != nullptr));
      pst_free(c);
      std::remove(path.c_str());
    }
    pst_cost_model_t c = nullptr;
    EXPECT(pst_cost_model_load("/nonexistent/dir/table.json", &c) == PST_E_INVALID_ARG && !c);
    EXPECT(pst_cost_model_load(nullptr, &c) == PST_E_INVALID_ARG);
  }
  {
    uint32_t not_an_object[4] = {0xdeadbeefu, 0, 0, 0};
    EXPECT(pst_free(not_an_object) == PST_E_INVALID_ARG);
    EXPECT(pst_free(nullptr) == PST_OK);
    EXPECT(std::strlen(pst_last_error()) > 0);
  }
}

int main() {
  valid_trees();
  error_paths();
  if (g_fail) {
    std::fprintf(stderr, "%d expectations failed\n", g_fail);
    return 1;
  }
  std::printf("asan host driver: all checks passed\n");
  return 0;
}
