// C ABI of libpst (see include/pst.h): object lifetimes, argument checks,
// device uploads of the tree index and the plan, and the two launches of the
// hot path (PAC, then POR).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstddef>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>

#include "pst_internal.h"

namespace pst {

static thread_local std::string g_last_error;
void set_error(const std::string& msg) { g_last_error = msg; }

// PST_FAULT_INJECT=alloc:N makes the N-th device allocation of the process
// fail (1-based), so error paths can be tested from the host.
static int g_alloc_count = 0;
static bool inject_alloc_failure() {
  static int target = [] {
    const char* s = std::getenv("PST_FAULT_INJECT");
    if (!s || std::strncmp(s, "alloc:", 6) != 0) return 0;
    return std::atoi(s + 6);
  }();
  ++g_alloc_count;
  return target > 0 && g_alloc_count == target;
}

static pst_status hip_fail(const char* what, hipError_t e) {
  set_error(std::string(what) + ": " + hipGetErrorString(e));
  return PST_E_HIP;
}

// One device allocation per object: every array sits at a 256-byte aligned
// offset and arrives with one host-to-device copy from a packed staging
// buffer (a tree or plan rebuilt per topology change then costs one
// allocation, one copy and one free instead of one of each per array).
class DevArena {
 public:
  template <typename T>
  void add(T** dst, const T* src, size_t count) {
    parts_.push_back({reinterpret_cast<void**>(dst), src, count * sizeof(T), size_});
    size_ += (std::max<size_t>(count * sizeof(T), 1) + 255) & ~static_cast<size_t>(255);
  }
  // Allocates, copies on stream s and waits for the copy (the staging buffer
  // is freed on return).  On failure *base stays null.
  pst_status commit(void** base, hipStream_t s) {
    *base = nullptr;
    if (inject_alloc_failure()) {
      set_error("injected device allocation failure");
      return PST_E_OOM;
    }
    hipError_t e = hipMalloc(base, size_);
    if (e != hipSuccess) {
      *base = nullptr;
      (void)hipGetLastError();
      set_error(std::string("hipMalloc failed: ") + hipGetErrorString(e));
      return PST_E_OOM;
    }
    std::vector<char> staging(size_, 0);
    for (const Part& a : parts_) {
      if (a.bytes) std::memcpy(staging.data() + a.offset, a.src, a.bytes);
      *a.dst = static_cast<char*>(*base) + a.offset;
    }
    e = hipMemcpyAsync(*base, staging.data(), size_, hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
      for (const Part& a : parts_) *a.dst = nullptr;
      (void)hipFree(*base);
      *base = nullptr;
      return hip_fail("upload", e);
    }
    return PST_OK;
  }

 private:
  struct Part {
    void** dst;
    const void* src;
    size_t bytes, offset;
  };
  std::vector<Part> parts_;
  size_t size_ = 0;
};

}  // namespace pst

using namespace pst;

struct pst_tree_s {
  uint32_t magic = kTreeMagic;
  TreeIndex ix;
  pst_shape shape{};
  int64_t pool_tokens = 0;
  bool on_device = false;
  int device = -1;
  uint64_t generation = 0;  // bumped when the device index is rebuilt
  int live_plans = 0;               // plans handed out by pst_plan and not yet freed
  std::vector<pst_plan_s*> plans;  // every plan of this tree: their device tasks follow length changes
  pst_plan_s* baseline = nullptr;  // query-guided plan of pst_decode_attn_baseline (owned by the tree)
  // Pinned staging buffers of pst_tree_set_lengths, used in turn: a copy from
  // pinned memory runs asynchronously, and a buffer is written again only
  // after the copy queued from it kLengthSlots calls earlier has finished.
  static constexpr int kLengthSlots = 4;
  struct Staging {
    char* host = nullptr;  // hipHostMalloc
    size_t bytes = 0;
    hipEvent_t copied = nullptr;  // recorded after the copies out of `host`
  };
  Staging staging[kLengthSlots];
  int staging_next = 0;
  uint64_t baseline_cost = 0;      // id of the cost model it was made with (0 = built-in model)
  void* d_arena = nullptr;  // holds every d_ array below
  int64_t* d_node_off = nullptr;
  int32_t* d_node_len = nullptr;
  int32_t* d_page_ptr = nullptr;
  int32_t* d_page_idx = nullptr;
  uint8_t* d_node_masked = nullptr;
  int32_t* d_nq_ptr = nullptr;
  int32_t* d_nq_idx = nullptr;
  uint64_t* d_nq_mask = nullptr;
};

struct pst_plan_s {
  uint32_t magic = kPlanMagic;
  pst_tree_s* tree = nullptr;
  uint64_t generation = 0;
  PlanOptions opts;
  PlanResult r;
  bool on_device = false;
  void* d_arena = nullptr;  // holds every d_ array below
  DevTask* d_tasks = nullptr;
  int32_t* d_bin_ptr = nullptr;
  int32_t* d_entry_slot = nullptr;
  int64_t* d_slot_ptr = nullptr;
  int32_t* d_flat_query = nullptr;  // flattened plans
  uint64_t* d_flat_mask = nullptr;
  int32_t* d_flat_rows = nullptr;
  int64_t flat_pool_bytes = 0;      // bytes from a kv head's first row past the last row the plan reads
  std::vector<DevTask> dev_tasks;  // host copy of d_tasks
};

struct pst_cost_s {
  uint32_t magic = kCostMagic;
  uint64_t id = 0;  // unique per model made in this process
  CostModel model;
};

static void free_tree_device(pst_tree_s* t) {
  for (auto& st : t->staging) {
    if (st.copied) {
      (void)hipEventSynchronize(st.copied);
      (void)hipEventDestroy(st.copied);
    }
    if (st.host) (void)hipHostFree(st.host);
    st = pst_tree_s::Staging{};
  }
  if (t->d_arena) (void)hipFree(t->d_arena);
  t->d_arena = nullptr;
  t->d_node_off = nullptr;
  t->d_node_len = nullptr;
  t->d_page_ptr = t->d_page_idx = nullptr;
  t->d_node_masked = nullptr;
  t->d_nq_ptr = t->d_nq_idx = nullptr;
  t->d_nq_mask = nullptr;
  t->on_device = false;
}

static void free_plan_device(pst_plan_s* p) {
  if (p->d_arena) (void)hipFree(p->d_arena);
  p->d_arena = nullptr;
  p->d_tasks = nullptr;
  p->d_bin_ptr = p->d_entry_slot = nullptr;
  p->d_slot_ptr = nullptr;
  p->d_flat_query = p->d_flat_rows = nullptr;
  p->d_flat_mask = nullptr;
  p->on_device = false;
}

// Unlinks a plan from its tree's list and frees it (the caller fixes the
// tree's count of handed-out plans).
static void release_plan(pst_plan_s* p) {
  if (p->tree) {
    auto& v = p->tree->plans;
    v.erase(std::remove(v.begin(), v.end(), p), v.end());
  }
  free_plan_device(p);
  p->magic = 0;
  delete p;
}

static int elem_bytes(int dt) { return dt == PST_F32 ? 4 : 2; }

static pst_status check_shape(const pst_shape& s) {
  if (s.num_q_heads < 1 || s.num_kv_heads < 1 || s.num_q_heads % s.num_kv_heads != 0) {
    set_error("num_q_heads must be a positive multiple of num_kv_heads");
    return PST_E_UNSUPPORTED;
  }
  if (s.num_q_heads / s.num_kv_heads > kMaxRows) {
    set_error("GQA group larger than 256");
    return PST_E_UNSUPPORTED;
  }
  if (s.head_dim != 64 && s.head_dim != 128) {
    set_error("head_dim must be 64 or 128");
    return PST_E_UNSUPPORTED;
  }
  if (s.in_dtype != PST_F32 && s.in_dtype != PST_BF16) {
    set_error("in_dtype must be PST_F32 or PST_BF16");
    return PST_E_UNSUPPORTED;
  }
  if (s.out_dtype != PST_F32 && s.out_dtype != s.in_dtype) {
    set_error("out_dtype must be PST_F32 or in_dtype");
    return PST_E_UNSUPPORTED;
  }
  if (s.kv_stride_head < 0 || s.kv_stride_token < 0 || s.pool_tokens < 0) {
    set_error("negative stride or pool size");
    return PST_E_INVALID_ARG;
  }
  return PST_OK;
}

namespace pst {
pst_status plan_ready_for_launch(pst_plan_t p) {
  if (!p || p->magic != kPlanMagic) {
    set_error("bad plan");
    return PST_E_INVALID_ARG;
  }
  if (!p->on_device || !p->tree->on_device) {
    set_error("plan or tree was built host-only");
    return PST_E_NO_DEVICE;
  }
  if (p->generation != p->tree->generation) {
    set_error("plan is stale: its tree changed");
    return PST_E_PLAN_STALE;
  }
  return PST_OK;
}
}  // namespace pst

extern "C" {

const char* pst_last_error(void) { return g_last_error.c_str(); }

pst_status pst_tree_build(const pst_tree_desc* desc, const pst_shape* shape, uint32_t flags, void* stream,
                          pst_tree_t* out) {
  if (!out) {
    set_error("out is NULL");
    return PST_E_INVALID_ARG;
  }
  *out = nullptr;
  if (!desc || !shape) {
    set_error("desc or shape is NULL");
    return PST_E_INVALID_ARG;
  }
  pst_status st = check_shape(*shape);
  if (st != PST_OK) return st;
  pst_tree_s* t = new (std::nothrow) pst_tree_s();
  if (!t) {
    set_error("host allocation failed");
    return PST_E_OOM;
  }
  st = build_tree_index(*desc, &t->ix);
  if (st != PST_OK) {
    delete t;
    return st;
  }
  t->shape = *shape;
  if (t->shape.scale <= 0.f) t->shape.scale = 1.0f / std::sqrt(static_cast<float>(shape->head_dim));
  int64_t need = 0;
  if (t->ix.page_size > 0) {
    for (const int32_t pg : t->ix.page_idx) need = std::max(need, (static_cast<int64_t>(pg) + 1) * t->ix.page_size);
  } else {
    for (int32_t i = 0; i < t->ix.N; ++i) need = std::max(need, t->ix.kv_offset[i] + t->ix.kv_len[i]);
  }
  t->pool_tokens = shape->pool_tokens > 0 ? shape->pool_tokens : need;
  if (need > t->pool_tokens) {
    const bool paged = t->ix.page_size > 0;
    delete t;
    set_error(paged ? "a page lies outside the K/V pools (pool_tokens too small)"
                    : "a node lies outside the K/V pools (pool_tokens too small)");
    return PST_E_INVALID_TREE;
  }
  if (t->shape.kv_stride_token == 0) t->shape.kv_stride_token = shape->head_dim;
  if (t->shape.kv_stride_head == 0) t->shape.kv_stride_head = t->pool_tokens * shape->head_dim;
  if (t->shape.kv_stride_token < shape->head_dim) {
    delete t;
    set_error("kv_stride_token smaller than head_dim");
    return PST_E_INVALID_ARG;
  }
  const int eb = elem_bytes(shape->in_dtype);
  if ((t->shape.kv_stride_token * eb) % 16 != 0 || (t->shape.kv_stride_head * eb) % 16 != 0) {
    delete t;
    set_error("K/V strides must be multiples of 16 bytes (128-bit loads)");
    return PST_E_INVALID_ARG;
  }
  // The kernels address a tile's tokens with 32-bit offsets (up to 128
  // tokens times the stride) and a paged pool's rows with 32-bit numbers.
  if (t->shape.kv_stride_token * eb >= (int64_t{1} << 24)) {
    delete t;
    set_error("kv_stride_token must be below 16 MiB");
    return PST_E_INVALID_ARG;
  }
  if (t->ix.page_size > 0 && t->pool_tokens > INT32_MAX) {
    delete t;
    set_error("a paged pool holds at most 2^31 - 1 tokens per head");
    return PST_E_INVALID_ARG;
  }
  if (!(flags & PST_TREE_HOST_ONLY)) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipGetDevice(&t->device);
    if (e != hipSuccess) {
      delete t;
      set_error(std::string("no HIP device: ") + hipGetErrorString(e));
      return PST_E_NO_DEVICE;
    }
    const TreeIndex& ix = t->ix;
    DevArena arena;
    arena.add(&t->d_node_off, ix.kv_offset.data(), ix.N);
    arena.add(&t->d_node_len, ix.kv_len.data(), ix.N);
    if (ix.page_size > 0) {
      arena.add(&t->d_page_ptr, ix.page_ptr.data(), ix.page_ptr.size());
      arena.add(&t->d_page_idx, ix.page_idx.data(), ix.page_idx.size());
    }
    arena.add(&t->d_node_masked, ix.masked.data(), ix.N);
    arena.add(&t->d_nq_ptr, ix.nq_ptr.data(), ix.nq_ptr.size());
    arena.add(&t->d_nq_idx, ix.nq_idx.data(), ix.nq_idx.size());
    arena.add(&t->d_nq_mask, ix.nq_mask.data(), ix.nq_mask.size());
    st = arena.commit(&t->d_arena, s);
    if (st != PST_OK) {
      free_tree_device(t);
      delete t;
      return st;
    }
    t->on_device = true;
  }
  static uint64_t counter = 0;
  t->generation = ++counter;
  *out = t;
  return PST_OK;
}

// Growth checks shared by pst_tree_set_lengths and pst_tree_append: every
// length >= the current one, masked nodes <= 64, every node inside its pages
// or the pools, and no flattened plan live.
static pst_status check_growth(const pst_tree_s* t, const int32_t* kv_len) {
  const TreeIndex& ix = t->ix;
  for (const pst_plan_s* p : t->plans) {
    if (p->r.flat_chunk > 0) {
      set_error("a flattened plan of this tree is live: its chunks would move (free it, grow, plan again)");
      return PST_E_UNSUPPORTED;
    }
  }
  for (int32_t i = 0; i < ix.N; ++i) {
    if (kv_len[i] < ix.kv_len[i]) {
      set_error("kv_len may only grow (node " + std::to_string(i) + ")");
      return PST_E_INVALID_ARG;
    }
    if (ix.masked[i] && kv_len[i] > 64) {
      set_error("masked node " + std::to_string(i) + " would exceed 64 tokens");
      return PST_E_INVALID_TREE;
    }
    if (ix.page_size > 0) {
      if (static_cast<int64_t>(ix.page_ptr[i + 1] - ix.page_ptr[i]) * ix.page_size < kv_len[i]) {
        set_error("node " + std::to_string(i) + " would outgrow its pages");
        return PST_E_INVALID_TREE;
      }
    } else if (ix.kv_offset[i] + kv_len[i] > t->pool_tokens) {
      set_error("node " + std::to_string(i) + " would leave the K/V pools");
      return PST_E_INVALID_TREE;
    }
  }
  return PST_OK;
}

// The host side of growth: visible counts, the index's lengths, and the host
// copies of the plans' device tasks (the last piece of every node absorbs
// its growth).
static void apply_growth(pst_tree_s* t, const int32_t* kv_len) {
  TreeIndex& ix = t->ix;
  // Visible counts: every node on a path grows, except that a query's own
  // masked node keeps its mask bits.
  for (int32_t r = 0; r < ix.B; ++r) {
    const int32_t own = ix.query_node[r];
    int64_t vis = 0;
    for (int32_t e = ix.qn_ptr[r]; e < ix.qn_ptr[r + 1]; ++e) {
      const int32_t n = ix.qn_idx[e];
      if (n == own && ix.masked[n] && ix.have_mask)
        vis += __builtin_popcountll(ix.qmask[r]);
      else
        vis += kv_len[n];
    }
    ix.visible[r] = vis;
  }
  std::copy(kv_len, kv_len + ix.N, ix.kv_len.begin());
  for (pst_plan_s* p : t->plans) {
    for (size_t i = 0; i < p->r.tasks.size(); ++i) {
      const Task& a = p->r.tasks[i];
      if (!(a.flags & PST_TASK_LAST_PIECE)) continue;
      const int32_t len = ix.kv_len[a.node] - a.kv_begin;
      if (i < p->dev_tasks.size()) p->dev_tasks[i].kv_len = len;
    }
  }
}

pst_status pst_tree_set_lengths(pst_tree_t t, const int32_t* kv_len, void* stream) {
  if (!t || t->magic != kTreeMagic || !kv_len) {
    set_error("bad tree or kv_len");
    return PST_E_INVALID_ARG;
  }
  TreeIndex& ix = t->ix;
  pst_status st = check_growth(t, kv_len);
  if (st != PST_OK) return st;
  // The device copies of the new lengths and of every plan's tasks leave from
  // a pinned staging buffer (so the copies are asynchronous: no host wait).
  hipStream_t s = static_cast<hipStream_t>(stream);
  auto align = [](size_t x) { return (x + 255) & ~static_cast<size_t>(255); };
  size_t need = 0;
  pst_tree_s::Staging* slot = nullptr;
  if (t->on_device && ix.N > 0) {
    need = align(ix.N * sizeof(int32_t));
    for (const pst_plan_s* p : t->plans)
      if (p->on_device) need += align(p->dev_tasks.size() * sizeof(DevTask));
    slot = &t->staging[t->staging_next];
    if (slot->copied) {
      hipError_t e = hipEventSynchronize(slot->copied);  // the copies queued from it kLengthSlots calls ago
      if (e != hipSuccess) return hip_fail("hipEventSynchronize", e);
    } else {
      hipError_t e = hipEventCreateWithFlags(&slot->copied, hipEventDisableTiming);
      if (e != hipSuccess) {
        slot->copied = nullptr;
        return hip_fail("hipEventCreateWithFlags", e);
      }
    }
    if (slot->bytes < need) {
      if (slot->host) (void)hipHostFree(slot->host);
      slot->host = nullptr;
      slot->bytes = 0;
      void* h = nullptr;
      hipError_t e = hipHostMalloc(&h, need, hipHostMallocDefault);
      if (e != hipSuccess) {
        (void)hipGetLastError();
        set_error(std::string("hipHostMalloc failed: ") + hipGetErrorString(e));
        return PST_E_OOM;
      }
      slot->host = static_cast<char*>(h);
      slot->bytes = need;
    }
  }
  apply_growth(t, kv_len);
  if (slot) {
    size_t off = 0;
    std::memcpy(slot->host, ix.kv_len.data(), ix.N * sizeof(int32_t));
    hipError_t e = hipMemcpyAsync(t->d_node_len, slot->host, ix.N * sizeof(int32_t), hipMemcpyHostToDevice, s);
    off += align(ix.N * sizeof(int32_t));
    for (pst_plan_s* p : t->plans) {
      if (e != hipSuccess) break;
      if (!p->on_device) continue;
      const size_t bytes = p->dev_tasks.size() * sizeof(DevTask);
      if (bytes) {
        std::memcpy(slot->host + off, p->dev_tasks.data(), bytes);
        e = hipMemcpyAsync(p->d_tasks, slot->host + off, bytes, hipMemcpyHostToDevice, s);
      }
      off += align(bytes);
    }
    if (e == hipSuccess) e = hipEventRecord(slot->copied, s);
    t->staging_next = (t->staging_next + 1) % pst_tree_s::kLengthSlots;
    if (e != hipSuccess) return hip_fail("length upload", e);
  }
  return PST_OK;
}

pst_status pst_tree_append(pst_tree_t t, int32_t n, const int32_t* nodes, const void* k_new, const void* v_new,
                           void* k_pool, void* v_pool, void* stream) {
  if (!t || t->magic != kTreeMagic || n < 0 || (n > 0 && (!nodes || !k_new || !v_new || !k_pool || !v_pool))) {
    set_error("bad tree, negative count or NULL argument");
    return PST_E_INVALID_ARG;
  }
  TreeIndex& ix = t->ix;
  std::vector<int32_t> lens(ix.kv_len);
  std::vector<uint8_t> grown(ix.N, 0);
  std::vector<int64_t> rows(n);
  for (int32_t i = 0; i < n; ++i) {
    const int32_t node = nodes[i];
    if (node < 0 || node >= ix.N) {
      set_error("nodes[" + std::to_string(i) + "] out of range");
      return PST_E_INVALID_ARG;
    }
    if (grown[node]) {
      set_error("node " + std::to_string(node) + " listed twice");
      return PST_E_INVALID_ARG;
    }
    grown[node] = 1;
    lens[node] += 1;
  }
  pst_status st = check_growth(t, lens.data());  // every new token inside its node's pages or the pools
  if (st != PST_OK) return st;
  if (!t->on_device) {
    set_error("tree was built host-only");
    return PST_E_NO_DEVICE;
  }
  for (int32_t i = 0; i < n; ++i) {
    const int32_t node = nodes[i];
    const int64_t pos = ix.kv_len[node];  // the new token's position in its node
    rows[i] = ix.page_size > 0 ? static_cast<int64_t>(ix.page_idx[ix.page_ptr[node] + pos / ix.page_size]) * ix.page_size +
                                     pos % ix.page_size
                               : ix.kv_offset[node] + pos;
  }
  apply_growth(t, lens.data());
  // The device words to set: the grown nodes' lengths, and the kv_len of
  // every live plan's last pieces of those nodes.
  std::vector<std::pair<int32_t*, int32_t>> sets;
  for (int32_t i = 0; i < n; ++i) sets.push_back({t->d_node_len + nodes[i], lens[nodes[i]]});
  for (pst_plan_s* p : t->plans) {
    if (!p->on_device) continue;
    for (size_t j = 0; j < p->r.tasks.size() && j < p->dev_tasks.size(); ++j) {
      const Task& a = p->r.tasks[j];
      if (!(a.flags & PST_TASK_LAST_PIECE) || !grown[a.node]) continue;
      int32_t* field = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(p->d_tasks + j) + offsetof(DevTask, kv_len));
      sets.push_back({field, p->dev_tasks[j].kv_len});
    }
  }
  const int eb = elem_bytes(t->shape.in_dtype);
  AppendParams ap{};
  ap.kv.hkv = t->shape.num_kv_heads;
  ap.kv.chunks = t->shape.head_dim * eb / 16;
  ap.kv.pool_tokens = t->pool_tokens;
  ap.kv.stride_head_bytes = t->shape.kv_stride_head * eb;
  ap.kv.stride_token_bytes = t->shape.kv_stride_token * eb;
  ap.kv.k_pool = k_pool;
  ap.kv.v_pool = v_pool;
  const int64_t row_bytes = static_cast<int64_t>(ap.kv.hkv) * ap.kv.chunks * 16;
  const int64_t nsets = static_cast<int64_t>(sets.size());
  const int64_t launches = std::max((static_cast<int64_t>(n) + kAppendRows - 1) / kAppendRows,
                                    (nsets + kAppendSets - 1) / kAppendSets);
  for (int64_t L = 0; L < launches; ++L) {
    const int64_t r0 = L * kAppendRows, s0 = L * kAppendSets;
    ap.kv.n = std::max<int64_t>(0, std::min<int64_t>(kAppendRows, n - r0));
    ap.kv.k_new = static_cast<const char*>(k_new) + r0 * row_bytes;
    ap.kv.v_new = static_cast<const char*>(v_new) + r0 * row_bytes;
    for (int64_t r = 0; r < ap.kv.n; ++r) ap.rows[r] = rows[r0 + r];
    ap.n_sets = static_cast<int32_t>(std::max<int64_t>(0, std::min<int64_t>(kAppendSets, nsets - s0)));
    for (int32_t k = 0; k < ap.n_sets; ++k) {
      ap.set_addr[k] = sets[s0 + k].first;
      ap.set_val[k] = sets[s0 + k].second;
    }
    int e = launch_append(ap, stream);
    if (e != 0) return hip_fail("append launch", static_cast<hipError_t>(e));
  }
  return PST_OK;
}

pst_status pst_tree_get_index(pst_tree_t t, pst_index_view* v) {
  if (!t || t->magic != kTreeMagic || !v) {
    set_error("bad tree or view");
    return PST_E_INVALID_ARG;
  }
  const TreeIndex& ix = t->ix;
  v->num_nodes = ix.N;
  v->num_queries = ix.B;
  v->num_entries = static_cast<int64_t>(ix.qn_idx.size());
  v->depth = ix.depth.data();
  v->n_q = ix.n_q.data();
  v->qn_ptr = ix.qn_ptr.data();
  v->qn_idx = ix.qn_idx.data();
  v->nq_ptr = ix.nq_ptr.data();
  v->nq_idx = ix.nq_idx.data();
  v->nq_mask = ix.nq_mask.data();
  v->visible = ix.visible.data();
  v->page_size = ix.page_size;
  v->page_ptr = ix.page_size > 0 ? ix.page_ptr.data() : nullptr;
  v->page_idx = ix.page_size > 0 ? ix.page_idx.data() : nullptr;
  return PST_OK;
}

static pst_status make_cost(int32_t n_rows, const int32_t* rows_grid, int32_t n_len, const int32_t* len_grid,
                            const int64_t* table, pst_cost_model_t* out) {
  if (n_rows < 1 || n_len < 2 || !rows_grid || !len_grid || !table) {
    set_error("cost table needs >= 1 rows point, >= 2 length points and non-NULL arrays");
    return PST_E_INVALID_ARG;
  }
  for (int i = 0; i < n_rows; ++i)
    if (rows_grid[i] < 1 || (i && rows_grid[i] <= rows_grid[i - 1])) {
      set_error("rows grid must be ascending and >= 1");
      return PST_E_INVALID_ARG;
    }
  for (int j = 0; j < n_len; ++j)
    if (len_grid[j] < 1 || (j && len_grid[j] <= len_grid[j - 1])) {
      set_error("length grid must be ascending and >= 1");
      return PST_E_INVALID_ARG;
    }
  for (int i = 0; i < n_rows; ++i)
    for (int j = 0; j < n_len; ++j) {
      const int64_t c = table[i * n_len + j];
      if (c < 1 || (j && c < table[i * n_len + j - 1]) || (i && c < table[(i - 1) * n_len + j])) {
        set_error("cost table must be >= 1 and non-decreasing along both axes");
        return PST_E_INVALID_ARG;
      }
    }
  pst_cost_s* c = new (std::nothrow) pst_cost_s();
  if (!c) {
    set_error("host allocation failed");
    return PST_E_OOM;
  }
  static uint64_t next_id = 0;
  c->id = ++next_id;
  c->model.rows_grid.assign(rows_grid, rows_grid + n_rows);
  c->model.len_grid.assign(len_grid, len_grid + n_len);
  c->model.table.assign(table, table + static_cast<size_t>(n_rows) * n_len);
  *out = c;
  return PST_OK;
}

pst_status pst_cost_model_create(int32_t n_rows, const int32_t* rows_grid, int32_t n_len, const int32_t* len_grid,
                                 const int64_t* table, pst_cost_model_t* out) {
  if (!out) {
    set_error("out is NULL");
    return PST_E_INVALID_ARG;
  }
  *out = nullptr;
  return make_cost(n_rows, rows_grid, n_len, len_grid, table, out);
}

pst_status pst_cost_model_load(const char* json_path, pst_cost_model_t* out) {
  if (!out) {
    set_error("out is NULL");
    return PST_E_INVALID_ARG;
  }
  *out = nullptr;
  if (!json_path) {
    set_error("json_path is NULL");
    return PST_E_INVALID_ARG;
  }
  std::vector<int32_t> rows, lens;
  std::vector<int64_t> table;
  pst_status st = load_cost_json(json_path, &rows, &lens, &table);
  if (st != PST_OK) return st;
  if (rows.size() > INT32_MAX || lens.size() > INT32_MAX) {
    set_error("cost table too large");
    return PST_E_INVALID_ARG;
  }
  st = make_cost(static_cast<int32_t>(rows.size()), rows.data(), static_cast<int32_t>(lens.size()), lens.data(),
                 table.data(), out);
  if (st != PST_OK) set_error(std::string("cost table ") + json_path + ": " + g_last_error);
  return st;
}

pst_status pst_cost_model_lookup(pst_cost_model_t c, int32_t rows, int64_t len, int64_t* ns) {
  if (!c || c->magic != kCostMagic || !ns) {
    set_error("bad cost model or output");
    return PST_E_INVALID_ARG;
  }
  *ns = c->model.lookup(rows, len);
  return PST_OK;
}

pst_status pst_device_info(int32_t* num_cu, int32_t* per_cu) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error(std::string("no HIP device: ") + hipGetErrorString(e));
    return PST_E_NO_DEVICE;
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return hip_fail("hipDeviceGetAttribute", e);
  int blocks = 0;
  int he = pac_blocks_per_cu(PST_BF16, 128, &blocks);
  if (he != 0) return hip_fail("occupancy query", static_cast<hipError_t>(he));
  if (num_cu) *num_cu = cus;
  if (per_cu) *per_cu = std::max(1, blocks);
  return PST_OK;
}

// Builds a plan object (host arrays, and the device copy unless host-only)
// without registering it with its tree.
static pst_status make_plan(pst_tree_t t, pst_cost_model_t cost, const pst_plan_opts* opts, void* stream,
                            pst_plan_t* out) {
  *out = nullptr;
  if (!t || t->magic != kTreeMagic) {
    set_error("bad tree");
    return PST_E_INVALID_ARG;
  }
  if (cost && cost->magic != kCostMagic) {
    set_error("bad cost model");
    return PST_E_INVALID_ARG;
  }
  pst_plan_opts o{};
  if (opts) o = *opts;
  const bool host_only = (o.flags & PST_PLAN_HOST_ONLY) || !t->on_device;
  const int32_t g = t->shape.num_q_heads / t->shape.num_kv_heads;
  PlanOptions po;
  po.tile = o.tile > 0 ? o.tile : kTile;
  po.grid_steps = o.grid_steps > 0 ? o.grid_steps : 8;
  po.fixed_chunk = o.fixed_chunk;
  po.no_split = (o.flags & PST_PLAN_NO_SPLIT) != 0;
  po.query_guided = (o.flags & PST_PLAN_QUERY_GUIDED) != 0;
  po.mfma_min_rows = (o.flags & PST_PLAN_DOT_SMALL) ? kMfmaMinRowsDot : 1;
  if (o.flags & PST_PLAN_FLATTEN) {
    if (po.no_split || po.query_guided || o.fixed_chunk < 0 || o.fixed_chunk % 128 != 0) {
      set_error("PST_PLAN_FLATTEN takes no other partition flag and a chunk length that is a multiple of 128");
      return PST_E_INVALID_ARG;
    }
    po.flat_chunk = o.fixed_chunk > 0 ? o.fixed_chunk : 256;
    po.fixed_chunk = 0;
  }
  const int32_t default_rows = t->shape.in_dtype == PST_F32 ? kMaxRowsDot : kMaxRows;
  po.r_max = o.max_rows > 0 ? o.max_rows : default_rows;
  if (po.tile % kTile != 0 || po.r_max > kMaxRows || po.fixed_chunk < 0 || po.fixed_chunk % kTile != 0 ||
      o.num_bins < 0) {
    set_error("tile and fixed_chunk must be multiples of 64, max_rows <= 256, num_bins >= 0");
    return PST_E_INVALID_ARG;
  }
  if (t->shape.in_dtype == PST_F32 && (po.query_guided ? g : po.r_max) > kMaxRowsDot) {
    set_error("float32 inputs run on the dot-product path: rows per workgroup must be <= 16");
    return PST_E_UNSUPPORTED;
  }
  if (po.query_guided && g > kMaxRows) {
    set_error("GQA group exceeds the rows of one workgroup");
    return PST_E_UNSUPPORTED;
  }
  if (o.num_bins > 0) {
    po.m = o.num_bins;
  } else if (!host_only) {
    int32_t cus = 0, per = 0;
    pst_status st = pst_device_info(&cus, &per);
    if (st != PST_OK) return st;
    po.m = std::max(1, cus * per / t->shape.num_kv_heads);
  } else {
    po.m = std::max(1, 256 / t->shape.num_kv_heads);
  }
  CostModel fallback;
  const CostModel* cm = nullptr;
  if (cost) {
    cm = &cost->model;
  } else {
    fallback = analytic_cost_model(g, t->shape.head_dim, elem_bytes(t->shape.in_dtype));
    cm = &fallback;
  }
  pst_plan_s* p = new (std::nothrow) pst_plan_s();
  if (!p) {
    set_error("host allocation failed");
    return PST_E_OOM;
  }
  p->tree = t;
  p->generation = t->generation;
  p->opts = po;
  pst_status st = po.flat_chunk > 0 ? build_flat_plan(t->ix, g, *cm, po, &p->r) : build_plan(t->ix, g, *cm, po, &p->r);
  if (st != PST_OK) {
    delete p;
    return st;
  }
  if (!p->r.slot_ptr.empty() && p->r.slot_ptr.back() > INT32_MAX / 2) {
    delete p;
    set_error("too many partial slots");
    return PST_E_UNSUPPORTED;
  }
  const bool flat = po.flat_chunk > 0;
  if (flat) {
    // Every row the plan reads must be addressable with 32-bit offsets from
    // its kv head's first row.
    int64_t max_row = -1;
    for (int32_t r : p->r.flat_rows) max_row = std::max<int64_t>(max_row, r);
    p->flat_pool_bytes = (max_row + 1) * t->shape.kv_stride_token * elem_bytes(t->shape.in_dtype);
    if (p->flat_pool_bytes > INT32_MAX) {
      delete p;
      set_error("flattened plans address K/V with 32-bit offsets: a kv head spans more than 2^31 - 1 bytes");
      return PST_E_UNSUPPORTED;
    }
  }
  if (!host_only) {
    hipStream_t s = static_cast<hipStream_t>(stream);
    std::vector<int32_t> es32(p->r.entry_slot.begin(), p->r.entry_slot.end());
    std::vector<DevTask>& dt = p->dev_tasks;
    dt.resize(p->r.tasks.size());
    for (size_t i = 0; i < dt.size(); ++i) {
      const Task& a = p->r.tasks[i];
      DevTask& b = dt[i];
      if (flat) {
        // A chunk: its first entry of the row table and of the entry arrays.
        // The mask test is needed unless every entry of the row group sees
        // every token; a chunk over consecutive pool rows (inside one
        // contiguous node, or nodes stored back to back) is addressed as a run.
        b.tok0 = a.kv_begin;
        b.node = a.node;
        b.kv_begin = 0;
        b.kv_len = a.kv_len;
        b.e0 = p->r.flat_ptr[a.node];
        b.row_begin = a.row_begin;
        b.row_count = a.row_count;
        b.piece = 0;
        const int64_t W = p->r.flat_chunk / 64;
        bool all_seen = true;
        for (int64_t e = b.e0 + a.row_begin / g; all_seen && e < b.e0 + (a.row_begin + a.row_count) / g; ++e) {
          for (int64_t w = 0; w < W && all_seen; ++w) {
            const int64_t valid = std::min<int64_t>(64, std::max<int64_t>(0, a.kv_len - 64 * w));
            const uint64_t need = valid == 64 ? ~0ull : ((1ull << valid) - 1);
            all_seen = (p->r.flat_mask[e * W + w] & need) == need;
          }
        }
        const int32_t* rows = p->r.flat_rows.data() + a.kv_begin;
        bool linear = true;
        for (int32_t k = 1; linear && k < a.kv_len; ++k) linear = rows[k] == rows[0] + k;
        const int64_t chunk_rows = static_cast<int64_t>(p->r.flat_ptr[a.node + 1] - p->r.flat_ptr[a.node]) * g;
        b.flags = (all_seen ? 0 : kDevMasked) | (linear ? kDevLinear : 0) | (a.row_count < chunk_rows ? kDevShared : 0);
        b.row0 = linear ? rows[0] : 0;
        continue;
      }
      // Contiguous: the piece's first pool token; paged: its position in the node.
      b.tok0 = t->ix.page_size > 0 ? a.kv_begin : t->ix.kv_offset[a.node] + a.kv_begin;
      b.node = a.node;
      b.kv_begin = a.kv_begin;
      b.kv_len = a.kv_len;
      b.e0 = t->ix.nq_ptr[a.node];
      b.row_begin = a.row_begin;
      b.row_count = a.row_count;
      b.piece = a.piece;
      const int64_t node_rows = static_cast<int64_t>(t->ix.nq_ptr[a.node + 1] - t->ix.nq_ptr[a.node]) * g;
      b.flags = ((a.flags & PST_TASK_LAST_PIECE) ? kDevLast : 0) | (t->ix.masked[a.node] ? kDevMasked : 0) |
                (a.row_count < node_rows ? kDevShared : 0);
      b.row0 = 0;
    }
    DevArena arena;
    arena.add(&p->d_tasks, dt.data(), dt.size());
    arena.add(&p->d_bin_ptr, p->r.bin_ptr.data(), p->r.bin_ptr.size());
    arena.add(&p->d_entry_slot, es32.data(), es32.size());
    arena.add(&p->d_slot_ptr, p->r.slot_ptr.data(), p->r.slot_ptr.size());
    if (flat) {
      arena.add(&p->d_flat_query, p->r.flat_query.data(), p->r.flat_query.size());
      arena.add(&p->d_flat_mask, p->r.flat_mask.data(), p->r.flat_mask.size());
      arena.add(&p->d_flat_rows, p->r.flat_rows.data(), p->r.flat_rows.size());
    }
    st = arena.commit(&p->d_arena, s);
    if (st != PST_OK) {
      free_plan_device(p);
      delete p;
      return st;
    }
    p->on_device = true;
  }
  *out = p;
  return PST_OK;
}

pst_status pst_plan(pst_tree_t t, pst_cost_model_t cost, const pst_plan_opts* opts, void* stream, pst_plan_t* out) {
  if (!out) {
    set_error("out is NULL");
    return PST_E_INVALID_ARG;
  }
  pst_status st = make_plan(t, cost, opts, stream, out);
  if (st != PST_OK) return st;
  t->live_plans++;
  t->plans.push_back(*out);
  return PST_OK;
}

static size_t align256(size_t x) { return (x + 255) & ~static_cast<size_t>(255); }

// Partial outputs in fp16 (with a power-of-two scale per slot and head)
// when the output is bf16 anyway and every piece runs on the matrix cores
// (bf16 input, no dot-product pieces): half the bytes PAC writes and POR
// reads, at a rounding (2^-11 relative) four times finer than the bf16
// output's own.  float32 otherwise.
static bool partials_f16(const pst_plan_s* p) {
  const pst_shape& s = p->tree->shape;
  return s.in_dtype == PST_BF16 && s.out_dtype == PST_BF16 && p->opts.mfma_min_rows <= 1;
}

// Workspace: partial outputs [slots][hq][d], then their LSE [slots][hq]
// (float32; for fp16 partials, (LSE, scale exponent) pairs of 8 bytes), each
// array 256-byte aligned.
static void workspace_layout(const pst_plan_s* p, size_t* o_bytes, size_t* total) {
  const pst_shape& s = p->tree->shape;
  const size_t slots = p->r.slot_ptr.empty() ? 0 : static_cast<size_t>(p->r.slot_ptr.back());
  const bool f16 = partials_f16(p);
  *o_bytes = align256(slots * s.num_q_heads * s.head_dim * (f16 ? 2 : sizeof(float)));
  *total = *o_bytes + align256(slots * s.num_q_heads * (f16 ? 2 : 1) * sizeof(float));
}

pst_status pst_plan_workspace_size(pst_plan_t p, size_t* bytes) {
  if (!p || p->magic != kPlanMagic || !bytes) {
    set_error("bad plan or output");
    return PST_E_INVALID_ARG;
  }
  size_t ob = 0;
  workspace_layout(p, &ob, bytes);
  return PST_OK;
}

pst_status pst_plan_get(pst_plan_t p, pst_plan_view* v) {
  if (!p || p->magic != kPlanMagic || !v) {
    set_error("bad plan or view");
    return PST_E_INVALID_ARG;
  }
  v->num_bins = p->opts.m;
  v->num_tasks = static_cast<int32_t>(p->r.tasks.size());
  v->num_queries = p->tree->ix.B;
  v->num_nodes = p->tree->ix.N;
  v->num_slots = p->r.slot_ptr.empty() ? 0 : p->r.slot_ptr.back();
  v->num_entries = static_cast<int64_t>(p->r.entry_slot.size());
  v->tasks = reinterpret_cast<const int32_t*>(p->r.tasks.data());
  v->bin_ptr = p->r.bin_ptr.data();
  v->slot_ptr = p->r.slot_ptr.data();
  v->entry_slot = p->r.entry_slot.data();
  v->piece_len = p->r.piece_len.data();
  v->b_eff = p->r.b_eff.data();
  v->rows_per_group = p->r.rows_per_group.data();
  v->bin_load = p->r.bin_load.data();
  v->makespan = p->r.makespan;
  v->cost_l = p->r.cost_l;
  v->chosen_k = p->r.chosen_k;
  v->max_rows = p->opts.query_guided ? p->tree->shape.num_q_heads / p->tree->shape.num_kv_heads : p->opts.r_max;
  v->mfma_min_rows = p->tree->shape.in_dtype == PST_BF16 ? p->opts.mfma_min_rows : INT32_MAX;
  const bool flat = p->r.flat_chunk > 0;
  v->flat_chunk = p->r.flat_chunk;
  v->num_chunks = flat ? static_cast<int32_t>(p->r.flat_ptr.size()) - 1 : 0;
  v->flat_ptr = flat ? p->r.flat_ptr.data() : nullptr;
  v->flat_query = flat ? p->r.flat_query.data() : nullptr;
  v->flat_mask = flat ? p->r.flat_mask.data() : nullptr;
  v->flat_rows = flat ? p->r.flat_rows.data() : nullptr;
  return PST_OK;
}

static pst_status check_run(pst_plan_t p, const void* ws, size_t ws_bytes) {
  pst_status st = plan_ready_for_launch(p);
  if (st != PST_OK) return st;
  size_t ob = 0, need = 0;
  workspace_layout(p, &ob, &need);
  if (need > 0 && (!ws || ws_bytes < need)) {
    set_error("workspace missing or smaller than pst_plan_workspace_size");
    return PST_E_WORKSPACE;
  }
  if (reinterpret_cast<uintptr_t>(ws) % 256 != 0) {
    set_error("workspace must be 256-byte aligned");
    return PST_E_WORKSPACE;
  }
  return PST_OK;
}

pst_status pst_pac(pst_plan_t p, const void* q, const void* k, const void* v, void* ws, size_t ws_bytes,
                   void* stream) {
  pst_status st = check_run(p, ws, ws_bytes);
  if (st != PST_OK) return st;
  if (p->r.tasks.empty()) return PST_OK;
  if (!q || !k || !v) {
    set_error("q, k_pool or v_pool is NULL");
    return PST_E_INVALID_ARG;
  }
  const pst_tree_s* t = p->tree;
  size_t ob = 0, total = 0;
  workspace_layout(p, &ob, &total);
  PacParams pp{};
  pp.q = q;
  pp.k = k;
  pp.v = v;
  pp.opart = static_cast<float*>(ws);
  pp.lsepart = reinterpret_cast<float*>(static_cast<char*>(ws) + ob);
  pp.part_f16 = partials_f16(p) ? 1 : 0;
  pp.tasks = p->d_tasks;
  pp.bin_ptr = p->d_bin_ptr;
  pp.nq_idx = t->d_nq_idx;
  pp.page_ptr = t->d_page_ptr;
  pp.page_idx = t->d_page_idx;
  pp.page_shift = t->ix.page_size > 0 ? __builtin_ctz(static_cast<unsigned>(t->ix.page_size)) : -1;
  pp.nq_mask = t->d_nq_mask;
  pp.entry_slot = p->d_entry_slot;
  if (p->r.flat_chunk > 0) {
    // Flattened chunks: entries, masks and rows of the plan; pages are in the row table.
    pp.nq_idx = p->d_flat_query;
    pp.nq_mask = p->d_flat_mask;
    pp.flat_rows = p->d_flat_rows;
    pp.mask_words = p->r.flat_chunk / 64;
    pp.pool_bytes = p->flat_pool_bytes;
    pp.page_shift = -1;
  }
  pp.stride_head = t->shape.kv_stride_head;
  pp.stride_token = t->shape.kv_stride_token;
  pp.q_bytes = static_cast<int64_t>(t->ix.B) * t->shape.num_q_heads * t->shape.head_dim *
               elem_bytes(t->shape.in_dtype);
  if (pp.q_bytes > INT32_MAX) {
    set_error("the query tensor exceeds 2 GiB (gathered with 32-bit offsets)");
    return PST_E_UNSUPPORTED;
  }
  pp.num_bins = p->opts.m;
  pp.hq = t->shape.num_q_heads;
  pp.hkv = t->shape.num_kv_heads;
  pp.g = pp.hq / pp.hkv;
  pp.mfma_min_rows = p->opts.mfma_min_rows;
  pp.scale_log2 = t->shape.scale * 1.4426950408889634f;
  int e = launch_pac(pp, t->shape.in_dtype, t->shape.head_dim, stream);
  if (e != 0) return hip_fail("PAC launch", static_cast<hipError_t>(e));
  return PST_OK;
}

pst_status pst_por(pst_plan_t p, void* out, float* lse_out, const void* ws, size_t ws_bytes, void* stream) {
  pst_status st = check_run(p, ws, ws_bytes);
  if (st != PST_OK) return st;
  const pst_tree_s* t = p->tree;
  if (t->ix.B == 0) return PST_OK;
  if (!out) {
    set_error("out is NULL");
    return PST_E_INVALID_ARG;
  }
  size_t ob = 0, total = 0;
  workspace_layout(p, &ob, &total);
  PorParams pp{};
  pp.opart = static_cast<const float*>(ws);
  pp.lsepart = reinterpret_cast<const float*>(static_cast<const char*>(ws) + ob);
  pp.part_f16 = partials_f16(p) ? 1 : 0;
  pp.slot_ptr = p->d_slot_ptr;
  pp.out = out;
  pp.lse_out = lse_out;
  pp.num_queries = t->ix.B;
  pp.hq = t->shape.num_q_heads;
  int e = launch_por(pp, t->shape.head_dim, t->shape.out_dtype, stream);
  if (e != 0) return hip_fail("POR launch", static_cast<hipError_t>(e));
  return PST_OK;
}

pst_status pst_decode_attn(pst_plan_t p, const void* q, const void* k, const void* v, void* out, float* lse_out,
                           void* ws, size_t ws_bytes, void* stream) {
  pst_status st = pst_pac(p, q, k, v, ws, ws_bytes, stream);
  if (st != PST_OK) return st;
  return pst_por(p, out, lse_out, ws, ws_bytes, stream);
}

// The tree's query-guided plan under `cost` (made on first use, and again
// when the cost model or the tree's generation changed).
static pst_status baseline_plan(pst_tree_t t, pst_cost_model_t cost, void* stream, pst_plan_s** out) {
  *out = nullptr;
  if (!t || t->magic != kTreeMagic) {
    set_error("bad tree");
    return PST_E_INVALID_ARG;
  }
  if (cost && cost->magic != kCostMagic) {
    set_error("bad cost model");
    return PST_E_INVALID_ARG;
  }
  if (!t->on_device) {
    set_error("tree was built host-only");
    return PST_E_NO_DEVICE;
  }
  const uint64_t cid = cost ? cost->id : 0;
  if (t->baseline && (t->baseline_cost != cid || t->baseline->generation != t->generation)) {
    release_plan(t->baseline);
    t->baseline = nullptr;
  }
  if (!t->baseline) {
    pst_plan_opts o{};
    o.flags = PST_PLAN_QUERY_GUIDED;
    pst_plan_s* p = nullptr;
    pst_status st = make_plan(t, cost, &o, stream, &p);
    if (st != PST_OK) return st;
    t->plans.push_back(p);  // follows length changes like any plan of the tree
    t->baseline = p;
    t->baseline_cost = cid;
  }
  *out = t->baseline;
  return PST_OK;
}

pst_status pst_baseline_workspace_size(pst_tree_t t, pst_cost_model_t cost, void* stream, size_t* bytes) {
  if (!bytes) {
    set_error("bytes is NULL");
    return PST_E_INVALID_ARG;
  }
  pst_plan_s* p = nullptr;
  pst_status st = baseline_plan(t, cost, stream, &p);
  if (st != PST_OK) return st;
  size_t ob = 0;
  workspace_layout(p, &ob, bytes);
  return PST_OK;
}

pst_status pst_decode_attn_baseline(pst_tree_t t, pst_cost_model_t cost, const void* q, const void* k,
                                    const void* v, void* out, float* lse_out, void* ws, size_t ws_bytes,
                                    void* stream) {
  pst_plan_s* p = nullptr;
  pst_status st = baseline_plan(t, cost, stream, &p);
  if (st != PST_OK) return st;
  return pst_decode_attn(p, q, k, v, out, lse_out, ws, ws_bytes, stream);
}

pst_status pst_free(void* obj) {
  if (!obj) return PST_OK;
  const uint32_t magic = *static_cast<uint32_t*>(obj);
  if (magic == kTreeMagic) {
    pst_tree_s* t = static_cast<pst_tree_s*>(obj);
    if (t->live_plans > 0) {
      set_error("tree still has live plans: free them first");
      return PST_E_INVALID_ARG;
    }
    if (t->baseline) release_plan(t->baseline);
    t->baseline = nullptr;
    free_tree_device(t);
    t->magic = 0;
    delete t;
    return PST_OK;
  }
  if (magic == kPlanMagic) {
    pst_plan_s* p = static_cast<pst_plan_s*>(obj);
    if (p->tree && p == p->tree->baseline) {
      set_error("this plan belongs to its tree (pst_decode_attn_baseline); it goes with the tree");
      return PST_E_INVALID_ARG;
    }
    if (p->tree) p->tree->live_plans--;
    release_plan(p);
    return PST_OK;
  }
  if (magic == kCostMagic) {
    pst_cost_s* c = static_cast<pst_cost_s*>(obj);
    c->magic = 0;
    delete c;
    return PST_OK;
  }
  set_error("pst_free: not a pst object");
  return PST_E_INVALID_ARG;
}

pst_status pst_write_kv_rows(pst_tree_t t, const void* k_new, const void* v_new, const int64_t* rows, int32_t n,
                             void* k_pool, void* v_pool, void* stream) {
  if (!t || t->magic != kTreeMagic) {
    set_error("bad tree");
    return PST_E_INVALID_ARG;
  }
  if (n < 0 || (n > 0 && (!k_new || !v_new || !rows || !k_pool || !v_pool))) {
    set_error("negative row count or NULL tensor");
    return PST_E_INVALID_ARG;
  }
  if (!t->on_device) {
    set_error("tree was built host-only");
    return PST_E_NO_DEVICE;
  }
  const int eb = elem_bytes(t->shape.in_dtype);
  KvRowsParams kp{};
  kp.k_new = k_new;
  kp.v_new = v_new;
  kp.rows = rows;
  kp.n = n;
  kp.hkv = t->shape.num_kv_heads;
  kp.chunks = t->shape.head_dim * eb / 16;
  kp.pool_tokens = t->pool_tokens;
  kp.stride_head_bytes = t->shape.kv_stride_head * eb;
  kp.stride_token_bytes = t->shape.kv_stride_token * eb;
  kp.k_pool = k_pool;
  kp.v_pool = v_pool;
  int e = launch_write_rows(kp, stream);
  if (e != 0) return hip_fail("row write launch", static_cast<hipError_t>(e));
  return PST_OK;
}

pst_status pst_bench_flush(void* buf, size_t bytes, void* stream) {
  if (!buf || bytes % 16 != 0) {
    set_error("flush buffer NULL or size not a multiple of 16");
    return PST_E_INVALID_ARG;
  }
  int e = launch_flush(buf, bytes, stream);
  if (e != 0) return hip_fail("flush launch", static_cast<hipError_t>(e));
  return PST_OK;
}

pst_status pst_bench_read(const void* buf, size_t bytes, float* sink, void* stream) {
  if (!buf || !sink || bytes % 16 != 0) {
    set_error("read buffer or sink NULL, or size not a multiple of 16");
    return PST_E_INVALID_ARG;
  }
  int e = launch_read(buf, bytes, sink, stream);
  if (e != 0) return hip_fail("read launch", static_cast<hipError_t>(e));
  return PST_OK;
}

}  // extern "C"
