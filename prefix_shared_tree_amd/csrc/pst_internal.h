// Internal declarations of libpst: host objects, the plan builder and the
// kernel parameter blocks shared between the host library and the kernels.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "pst.h"

namespace pst {

constexpr uint32_t kTreeMagic = 0x31545350u;  // "PST1"
constexpr uint32_t kPlanMagic = 0x32545350u;  // "PST2"
constexpr uint32_t kCostMagic = 0x33545350u;  // "PST3"

constexpr int kTile = 64;         // tokens per K/V tile of the partial-attention kernel
constexpr int kMaxRows = 256;     // rows one workgroup holds (matrix-core path: 8 waves x 32 rows)
constexpr int kMfmaMinRowsDot = 16;  // matrix-core threshold with PST_PLAN_DOT_SMALL (else 1)
constexpr int kMaxRowsDot = 16;   // the dot-product path keeps up to this many rows in registers

void set_error(const std::string& msg);

// Piece of partial attention: one node, one KV range, one row group.  Rows
// of node i are (node->query entry e, head j in the GQA group) = e * g + j.
struct Task {
  int32_t node;
  int32_t piece;
  int32_t kv_begin;
  int32_t kv_len;
  int32_t row_begin;
  int32_t row_count;
  int32_t flags;  // PST_TASK_LAST_PIECE
  int32_t reserved;
};
static_assert(sizeof(Task) == 32, "task layout");

// What the kernel reads per piece (built from a Task and the tree's node table).
struct DevTask {
  int64_t tok0;     // first token of the piece in the K/V pools
  int32_t node;
  int32_t kv_begin;
  int32_t kv_len;   // tokens (kept current for a growing last piece by pst_tree_set_lengths)
  int32_t e0;       // first node->query entry of the node
  int32_t row_begin;
  int32_t row_count;
  int32_t piece;
  int32_t flags;    // kDevLast | kDevMasked | kDevLinear | kDevShared
  int64_t row0;     // kDevLinear: pool row of the chunk's first token (its rows are consecutive)
};
static_assert(sizeof(DevTask) == 48, "device task layout");
constexpr int32_t kDevLast = 1;
constexpr int32_t kDevMasked = 2;  // the task needs the mask test (a masked node, a chunk whose masks are not all ones)
constexpr int32_t kDevLinear = 4;  // flattened chunk over consecutive pool rows (addressed as a contiguous run)
constexpr int32_t kDevShared = 8;  // another task (a row group of the same node or chunk) reads the same K/V tokens
constexpr int32_t kMaskWordsMax = 1024;  // mask words of one flattened task (8 KB of LDS)

struct CostModel {
  uint32_t magic = kCostMagic;
  std::vector<int32_t> rows_grid;
  std::vector<int32_t> len_grid;
  std::vector<int64_t> table;  // [rows][len]
  int64_t lookup(int64_t rows, int64_t len) const;
};

// Validates and indexes a tree on the host.  Returns PST_OK or an error with set_error().
struct TreeIndex {
  int32_t N = 0, B = 0;
  bool have_mask = false;
  std::vector<int32_t> parent, kv_len, query_node;
  std::vector<int64_t> kv_offset;  // contiguous layout (zeros when paged)
  int32_t page_size = 0;           // > 0: paged layout
  std::vector<int32_t> page_ptr, page_idx;
  std::vector<uint8_t> masked;
  std::vector<uint64_t> qmask;
  std::vector<int32_t> depth, n_q, qn_ptr, qn_idx, nq_ptr, nq_idx;
  std::vector<uint64_t> nq_mask;
  std::vector<int64_t> visible;
};
pst_status build_tree_index(const pst_tree_desc& d, TreeIndex* out);

struct PlanOptions {
  int32_t m = 1;
  int32_t r_max = kMaxRows;
  int32_t tile = kTile;
  int32_t grid_steps = 8;
  int32_t fixed_chunk = 0;
  bool no_split = false;
  bool query_guided = false;
  int32_t mfma_min_rows = 1;
  int32_t flat_chunk = 0;  // > 0: flattened partition with chunks of this many tokens
};

struct PlanResult {
  std::vector<Task> tasks;
  std::vector<int32_t> bin_ptr;
  std::vector<int64_t> slot_ptr, entry_slot;
  std::vector<int32_t> piece_len, b_eff, rows_per_group;
  std::vector<int64_t> bin_load;
  int64_t makespan = 0, cost_l = 0;
  int32_t chosen_k = 0;
  // Flattened partition (flat_chunk > 0): entries are (chunk, query) pairs;
  // entry_slot holds each entry's slot.
  int32_t flat_chunk = 0;
  std::vector<int32_t> flat_ptr, flat_query, flat_rows;
  std::vector<uint64_t> flat_mask;
};
pst_status build_plan(const TreeIndex& ix, int32_t g, const CostModel& cost, const PlanOptions& o,
                      PlanResult* out);
pst_status build_flat_plan(const TreeIndex& ix, int32_t g, const CostModel& cost, const PlanOptions& o,
                           PlanResult* out);
CostModel analytic_cost_model(int32_t g, int32_t head_dim, int32_t elem_bytes);
// Reads a profiled table (keys rows_grid, len_grid, table_ns) from a JSON
// file; the table comes back row-major.  Validation of its values is the
// caller's.
pst_status load_cost_json(const char* path, std::vector<int32_t>* rows_grid, std::vector<int32_t>* len_grid,
                          std::vector<int64_t>* table);

// ---------------------------------------------------------------------------
// Kernel parameter blocks (passed by value)
// ---------------------------------------------------------------------------
struct PacParams {
  const void* q;
  const void* k;
  const void* v;
  float* opart;    // [slots][hq][d] float32, or float16 when part_f16 (see below)
  float* lsepart;  // [slots][hq] LSE; part_f16: [slots][hq] pairs (LSE, exponent e as int32 bits),
                   // the fp16 partial being the output times 2^(15 - e)
  int32_t part_f16;  // partials in fp16 with a per-(slot, head) power-of-two scale (bf16 in and out, matrix cores)
  const DevTask* tasks;
  const int32_t* bin_ptr;
  const int32_t* nq_idx;
  const uint64_t* nq_mask;
  const int32_t* entry_slot;
  int64_t stride_head;   // elements
  int64_t stride_token;  // elements
  int64_t q_bytes;       // bytes of q ([B][hq][d]); below 2^31 (32-bit gather offsets)
  const int32_t* page_ptr;  // paged layout: [nodes + 1] (NULL when contiguous)
  const int32_t* page_idx;  // paged layout: page numbers
  int32_t page_shift;       // log2(page_size); -1 = contiguous (task tok0 = pool token), else tok0 = position in node
  int32_t num_bins;
  int32_t hq;
  int32_t hkv;
  int32_t g;
  int32_t mfma_min_rows;  // bf16 pieces with at least this many rows use the matrix cores
  float scale_log2;       // scale * log2(e)
  int32_t mask_words;       // flattened plans: 64-bit mask words per entry (S_t / 64); 0 otherwise
  const int32_t* flat_rows; // flattened plans: pool row of every chunk token (-1 past a chunk's end); tok0 indexes it
  int64_t pool_bytes;       // flattened plans: bytes from a kv head's first row past the last row read
};

struct PorParams {
  const float* opart;     // float32, or float16 when part_f16
  const float* lsepart;   // LSE, or (LSE, scale exponent) pairs when part_f16
  int32_t part_f16;
  const int64_t* slot_ptr;
  void* out;
  float* lse_out;
  int32_t num_queries;
  int32_t hq;
};

struct KvRowsParams {
  const void* k_new;  // [n][hkv][chunks] 16-byte chunks
  const void* v_new;
  const int64_t* rows;  // [n] pool token of each new row
  int64_t n;
  int32_t hkv;
  int32_t chunks;  // 16-byte chunks per row and head (head_dim * elem / 16)
  int64_t pool_tokens;
  int64_t stride_head_bytes;
  int64_t stride_token_bytes;
  void* k_pool;
  void* v_pool;
};
int launch_write_rows(const KvRowsParams& p, void* stream);

// One launch of pst_tree_append: the new rows' pool tokens and the device
// words to set (lengths of the grown nodes, kv_len of the plans' last pieces)
// travel in the kernel's arguments, so a decode step needs no copy.
constexpr int kAppendRows = 128;
constexpr int kAppendSets = 192;
struct AppendParams {
  KvRowsParams kv;  // kv.rows unused; kv.n rows of this launch
  int32_t n_sets;
  int64_t rows[kAppendRows];
  int32_t* set_addr[kAppendSets];
  int32_t set_val[kAppendSets];
};
static_assert(sizeof(AppendParams) <= 4096, "kernel arguments are limited to 4 KB");
int launch_append(const AppendParams& p, void* stream);

// The checks every launch makes first (a valid plan, built for the device,
// not stale); PST_OK or an error with set_error().
pst_status plan_ready_for_launch(pst_plan_t plan);

// Kernel launchers (defined in the .hip sources).  Return hipError_t as int.
int launch_pac(const PacParams& p, int in_dtype, int head_dim, void* stream);
int launch_por(const PorParams& p, int head_dim, int out_dtype, void* stream);
int launch_flush(void* buf, size_t bytes, void* stream);
int launch_read(const void* buf, size_t bytes, float* sink, void* stream);
int pac_blocks_per_cu(int in_dtype, int head_dim, int* blocks);
size_t pac_lds_bytes();

}  // namespace pst
