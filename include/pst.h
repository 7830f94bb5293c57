/*
 * pst.h -- prefix-shared tree decode attention on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libpst.so.  Plain pointers and sizes only; no C++ or framework
 * types cross it.  Streams are passed as `void*` and mean a hipStream_t
 * (NULL = the device's null stream).
 *
 * What the library computes.  A batch of decode queries sits on a forest of
 * KV-cache nodes joined under a virtual root; each edge p -> c says p's
 * tokens are the prefix of c's (CoDec: Prefix-Shared Decoding Kernel for
 * LLMs, section KV缓存管理 / KV-cache management).  Query r and q-head h
 * attend, with one softmax, to every token of every node on the path from
 * the root to the query's node (for a masked node, to the tokens whose bit
 * is set in the query's 64-bit mask: the bit causal mask of DEFT: Decoding
 * with Flash Tree-Attention, section 3.3 / Table 2):
 *     O[r,h] = softmax(scale * q[r,h] K_vis^T) V_vis,
 *     LSE[r,h] = ln sum exp(scale * q[r,h] K_vis^T).
 * It does so the way CoDec's kernel executor does (section 块内内核原语 and
 * 块间启动与树归约): one partial-attention (PAC) pass reads each node's K/V
 * once for all the queries whose path contains it and writes a normalised
 * partial output plus its LSE per (query, node piece); one partial-output
 * reduction (POR) pass merges each query's partials along an independent
 * chain.  Pieces and their assignment to workgroups come from a host plan
 * that balances a fitted per-piece cost C_est(rows, length) (section
 * 工作负载平衡 / workload balance).
 *
 * Conventions.
 *   g = num_q_heads / num_kv_heads; q-head h reads kv head h / g.
 *   Q   [num_queries][num_q_heads][head_dim], contiguous, in_dtype.
 *   K,V pools: element (kv head a, token t, channel c) at
 *       a * kv_stride_head + t * kv_stride_token + c      (elements, in_dtype)
 *       (default: head-major [num_kv_heads][pool_tokens][head_dim]).
 *   out [num_queries][num_q_heads][head_dim], contiguous, out_dtype.
 *   lse_out [num_queries][num_q_heads] float32, natural log (optional).
 *   Every pointer passed to pst_decode_attn / pst_pac / pst_por is device
 *   memory owned by the caller; the library never frees it.
 *
 * Errors.  Every entry point returns a pst_status; on failure
 * pst_last_error() returns a thread-local message.  Argument, tree and
 * staleness checks are synchronous.  Kernel launches are asynchronous on the
 * given stream; a launch failure returns PST_E_HIP, a fault in a kernel
 * surfaces at the caller's next synchronisation.
 *
 * Lifetime.  The library owns trees, plans and cost models (and the device
 * copies of their index arrays); pst_free releases them.  A plan borrows its
 * tree: free plans before their tree (freeing a tree with live plans returns
 * PST_E_INVALID_ARG).  Synchronise the stream before freeing anything a
 * launched kernel may still read.
 */
#ifndef PST_H
#define PST_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PST_OK = 0,
  PST_E_INVALID_ARG = 1,   /* null pointer, bad size, bad option */
  PST_E_INVALID_TREE = 2,  /* tree description violates the rules of pst_tree_build */
  PST_E_UNSUPPORTED = 3,   /* dtype / head_dim / head ratio not supported */
  PST_E_OOM = 4,           /* a host or device allocation failed */
  PST_E_PLAN_STALE = 5,    /* plan no longer matches its tree */
  PST_E_WORKSPACE = 6,     /* workspace missing or too small */
  PST_E_HIP = 7,           /* a HIP runtime call failed */
  PST_E_NO_DEVICE = 8      /* a device operation was asked of a host-only object */
} pst_status;

typedef enum { PST_F32 = 0, PST_BF16 = 1 } pst_dtype;

typedef struct pst_tree_s* pst_tree_t;
typedef struct pst_plan_s* pst_plan_t;
typedef struct pst_cost_s* pst_cost_model_t;

/* Tree description.  All arrays are host memory, read during the call and
 * copied; the caller keeps ownership.
 *   parent[i]      in [-1, i): the node whose tokens precede node i's; -1 =
 *                  child of the virtual root.  Parents come before children.
 *   kv_offset[i]   >= 0: first token of node i in the K/V pools (contiguous
 *                  layout; may be NULL when page_size > 0).
 *   kv_len[i]      >= 1: tokens in node i.
 *   query_node[r]  in [0, num_nodes): the deepest node on query r's path.
 *   node_masked    NULL or [num_nodes]: 1 = node i is masked (kv_len <= 64).
 *   query_mask     NULL or [num_queries]: for a query whose own node is
 *                  masked, bit j set = token j of that node visible.  Ignored
 *                  for queries on unmasked nodes.  Ancestors of a query's
 *                  node are always visible in full.
 *   page_size      0: each node is one contiguous run of the pools from
 *                  kv_offset[i].  > 0 (a power of two in [8, 65536]): paged
 *                  K/V, the layout of a paged KV cache (the FlashDecoding-
 *                  compatible input CoDec's implementation section takes):
 *                  token j of node i sits in pool row
 *                      page_idx[page_ptr[i] + j / page_size] * page_size
 *                        + j % page_size.
 *   page_ptr       [num_nodes + 1] when page_size > 0: page_ptr[0] = 0,
 *                  non-decreasing; node i owns the pages
 *                  page_idx[page_ptr[i] .. page_ptr[i+1]), at least
 *                  ceil(kv_len[i] / page_size) of them (growth through
 *                  pst_tree_set_lengths stays within them).
 *   page_idx       [page_ptr[num_nodes]] page numbers >= 0; every page lies
 *                  inside the pools (pool_tokens, or 0 = (largest page + 1)
 *                  * page_size).  Pages may be shared or in any order.
 * Every query must see at least one token. */
typedef struct {
  int32_t num_nodes;
  const int32_t* parent;
  const int64_t* kv_offset;
  const int32_t* kv_len;
  int32_t num_queries;
  const int32_t* query_node;
  const uint64_t* query_mask;
  const uint8_t* node_masked;
  int32_t page_size;
  const int32_t* page_ptr;
  const int32_t* page_idx;
} pst_tree_desc;

/* Head layout and dtypes.  head_dim in {64, 128}; num_q_heads a multiple of
 * num_kv_heads; in_dtype PST_F32 or PST_BF16; out_dtype PST_F32 or in_dtype.
 * scale <= 0 means 1/sqrt(head_dim).  Strides in elements; 0 selects the
 * head-major default; strides are multiples of 16 bytes and a token stride
 * is below 16 MiB.  pool_tokens = tokens per head in each pool (0 = the
 * largest kv_offset + kv_len); every node must lie inside it, and a paged
 * pool holds at most 2^31 - 1 tokens per head.  Otherwise
 * PST_E_INVALID_ARG. */
typedef struct {
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t head_dim;
  int32_t in_dtype;
  int32_t out_dtype;
  float scale;
  int64_t kv_stride_head;
  int64_t kv_stride_token;
  int64_t pool_tokens;
} pst_shape;

/* pst_tree_build flags */
#define PST_TREE_HOST_ONLY 1u /* build and validate the index on the host only (no GPU needed) */

/* Validate a tree and build its index: the node table (offset, length,
 * number of queries through the node, depth), the query->node CSR (each
 * query's path, root first) and the node->query CSR (each node's queries in
 * ascending id, with the 64-bit visibility mask of each entry: the query's
 * mask where the node is the query's own masked node, else all ones).  This
 * is CoDec's query<->KV index (section KV缓存管理) and DEFT's QMapKV / KVMapQ
 * (section A.8, Algorithm 1).  Unless PST_TREE_HOST_ONLY, the node table and
 * the node->query CSR are copied to the current device on `stream` (the call
 * returns after the copy).  On error *out is set to NULL. */
pst_status pst_tree_build(const pst_tree_desc* desc, const pst_shape* shape, uint32_t flags,
                          void* stream, pst_tree_t* out);

/* Decode-step growth: new lengths for every node, each >= the current one
 * (masked nodes stay <= 64).  Plans made from this tree stay valid: a node's
 * last piece simply grows (CoDec, implementation section: the partition is
 * reused across decoding steps).  The new lengths and the plans' patched
 * pieces are copied to the device on `stream` from pinned staging buffers
 * that the tree keeps (four, used in turn): the call queues the copies and
 * returns without waiting for them, except that it waits for the copies it
 * queued four calls earlier before writing their buffer again.  Launches
 * queued on `stream` after the call see the new lengths; work on another
 * stream must be ordered after `stream` by the caller, and a plan must not
 * be freed before the copies queued into it have run (synchronise `stream`).
 * Argument and tree checks come first: PST_E_INVALID_ARG / PST_E_INVALID_TREE
 * and PST_E_UNSUPPORTED (a flattened plan of the tree is live) change
 * nothing, nor does PST_E_OOM (the first call, or a call after plans were
 * added, allocates the staging memory). */
pst_status pst_tree_set_lengths(pst_tree_t tree, const int32_t* kv_len, void* stream);

/* One decode step of growth with its K/V (DEFT section A.1: each request's
 * tree grows by the token it just decoded; CoDec, implementation section:
 * the partition is reused across steps).  nodes: host int32 [n], distinct;
 * node nodes[i] gains one token whose K and V are row i of k_new / v_new
 * (device, [n][num_kv_heads][head_dim], in_dtype, contiguous).  The rows go
 * to each node's next position in k_pool / v_pool (contiguous: kv_offset +
 * kv_len; paged: through the page table), every kv head; the node grows by
 * one and the live plans' last pieces with it, so the plans stay valid, as
 * with pst_tree_set_lengths.  Everything is checked first and nothing
 * changes on an error (PST_E_INVALID_ARG: a node out of range or listed
 * twice; PST_E_INVALID_TREE: a node would outgrow its pages or the pools, or
 * a masked node pass 64 tokens; PST_E_UNSUPPORTED: a flattened plan of the
 * tree is live).  The pool tokens and the device words to update travel in
 * the arguments of kernel launches on `stream` (one launch per 128 rows):
 * no copy, no host wait; launches queued on `stream` afterwards see the new
 * rows and lengths. */
pst_status pst_tree_append(pst_tree_t tree, int32_t n, const int32_t* nodes, const void* k_new, const void* v_new,
                           void* k_pool, void* v_pool, void* stream);

/* Host views of the index, valid until the tree is freed. */
typedef struct {
  int32_t num_nodes;
  int32_t num_queries;
  int64_t num_entries;      /* sum over queries of path length */
  const int32_t* depth;     /* [num_nodes] nodes from the virtual root's child, >= 1 */
  const int32_t* n_q;       /* [num_nodes] queries whose path contains the node */
  const int32_t* qn_ptr;    /* [num_queries + 1] */
  const int32_t* qn_idx;    /* [num_entries] */
  const int32_t* nq_ptr;    /* [num_nodes + 1] */
  const int32_t* nq_idx;    /* [num_entries] */
  const uint64_t* nq_mask;  /* [num_entries] */
  const int64_t* visible;   /* [num_queries] tokens each query sees */
  int32_t page_size;        /* 0 = contiguous K/V */
  const int32_t* page_ptr;  /* [num_nodes + 1] when paged, else NULL */
  const int32_t* page_idx;  /* [page_ptr[num_nodes]] when paged, else NULL */
} pst_index_view;
pst_status pst_tree_get_index(pst_tree_t tree, pst_index_view* view);

/* Cost model C_est(rows, len) in integer nanoseconds: the time one
 * workgroup takes for one piece of `len` tokens and `rows` query rows (CoDec
 * section 工作负载平衡: profiled over a grid, interpolated elsewhere).  The
 * table is row-major [n_rows][n_len] over ascending grids, >= 1 everywhere and
 * non-decreasing along both axes.  Lookup: rows -> smallest grid point >=
 * rows (last point beyond the grid); len -> the first point's value below the
 * grid, integer linear interpolation inside it, linear extrapolation from the
 * last two points above it.  Arrays are copied. */
pst_status pst_cost_model_create(int32_t n_rows, const int32_t* rows_grid, int32_t n_len,
                                 const int32_t* len_grid, const int64_t* table, pst_cost_model_t* out);
pst_status pst_cost_model_lookup(pst_cost_model_t cost, int32_t rows, int64_t len, int64_t* ns);

/* The same model read from a JSON file (the format of the fitted gfx950
 * tables the library ships): an object whose "rows_grid" and "len_grid" are
 * arrays of integers and whose "table_ns" is an array holding one array of
 * integer nanoseconds per rows_grid point, each with one entry per len_grid
 * point; other keys are ignored.  The values must satisfy the rules of
 * pst_cost_model_create.  PST_E_INVALID_ARG (message names the file and the
 * problem) when the file cannot be read, is not such a JSON object, or holds
 * an invalid table; *out is then NULL. */
pst_status pst_cost_model_load(const char* json_path, pst_cost_model_t* out);

/* pst_plan options (zero-initialise for defaults) */
#define PST_PLAN_QUERY_GUIDED 1u /* FlashDecoding-style baseline: one query per row group (shared KV re-read per query) */
#define PST_PLAN_NO_SPLIT 2u     /* every node is one piece (b_k = 1) */
#define PST_PLAN_HOST_ONLY 4u    /* compute on the host only (no GPU needed) */
#define PST_PLAN_DOT_SMALL 8u    /* bf16 pieces of fewer than 16 rows take the wavefront dot-product path
                                    (the split CoDec and DEFT use); default: matrix cores for every bf16
                                    piece, which streams faster on gfx950 even at 1 row of 16 */
#define PST_PLAN_FLATTEN 16u     /* DEFT-Flatten partition instead of the cost-model one (see below);
                                    fixed_chunk = S_t, the chunk length (0 = 256) */
typedef struct {
  int32_t num_bins;    /* workgroups per kv head; 0 = resident capacity / num_kv_heads */
  int32_t max_rows;    /* rows one workgroup holds (R_max); 0 = 256 (bf16) or 16 (f32); <= 256 */
  int32_t tile;        /* piece granularity G in tokens; 0 = 64; a multiple of 64 */
  int32_t grid_steps;  /* K of the grid search; 0 = 8 */
  int32_t fixed_chunk; /* > 0: every node cut into pieces of this many tokens (ablation);
                          with PST_PLAN_FLATTEN: S_t, a multiple of 128 */
  uint32_t flags;
} pst_plan_opts;

/* Partition the tree's partial attention into pieces and assign them to
 * num_bins workgroups per kv head, minimising the largest workgroup cost
 * (CoDec section 工作负载平衡 and the min-max objective of section 速读):
 *  1. rows of node i: r_i = n_q[i] * g; cut into ceil(r_i / R_max) row
 *     groups of ceil(r_i / groups) rows when above R_max;
 *  2. b pieces of node i: Lp = roundup(ceil(n_i / b), G), pieces of Lp tokens;
 *  3. b_i(T): smallest b whose longest piece of the largest row group costs
 *     <= T; W(T) = total cost with b_i(T);
 *  4. cost_l: smallest T with num_bins * T >= W(T), by binary search;
 *  5. b_i <= ceil(C_est(rows_i, n_i) / cost_l);
 *  6. grid search over T_k = cost_l + cost_l * k / K, each candidate placed by
 *     longest-processing-time list scheduling (ties: lowest bin id); keep the
 *     smallest makespan (ties: fewer pieces, then smaller k).
 * `cost` NULL selects a built-in analytic model.  The plan keeps a pointer
 * to the tree.  Unless PST_PLAN_HOST_ONLY, the plan is copied to the device
 * on `stream` (returns after the copy).  Integer arithmetic throughout: the
 * same inputs give the same plan on every host. */
pst_status pst_plan(pst_tree_t tree, pst_cost_model_t cost, const pst_plan_opts* opts, void* stream,
                    pst_plan_t* out);

/* PST_PLAN_FLATTEN (DEFT: Decoding with Flash Tree-Attention, section 3.3,
 * remark 3.1, Fig. 3(c), and appendix A.9): the tree's K/V, in depth-first
 * order, is one logical sequence cut into chunks of S_t tokens; a chunk may
 * span nodes.  Each chunk is grouped with the queries that see any of its
 * tokens, and a 64-bit bit causal mask per (query, 64 tokens of the chunk)
 * says which ones.  K/V do not move: a per-token row table addresses them
 * (either layout).
 *  1. depth-first pre-order: roots, then children, by increasing node id;
 *     nodes no query sees are left out;
 *  2. chunk c = flattened tokens [c S_t, (c+1) S_t), the last one shorter;
 *  3. a chunk's entries: the queries that see one of its tokens, ascending;
 *  4. an entry's mask: S_t / 64 words, bit j of word w = token 64 w + j;
 *  5. row groups of whole entries, at most min(R_max / g, 1024 / (S_t / 64))
 *     entries: gq = ceil(entries / max) groups of ceil(entries / gq);
 *  6. row groups onto num_bins workgroups by longest-processing-time list
 *     scheduling on C_est(rows, chunk tokens), sorted by (cost desc, chunk,
 *     group), each to the bin with the smallest (load, id);
 *  7. a query's partial slots: one per chunk it is an entry of, in chunk order.
 * Tasks then name the chunk in `node`, its first flattened token in
 * `kv_begin`, and carry PST_TASK_FLAT.  Growth (pst_tree_set_lengths) is
 * refused while a flattened plan of the tree is live: the flattening moves.
 * PST_E_UNSUPPORTED when a kv head's K/V span more than 2^31 - 1 bytes. */

/* Bytes of device workspace pst_decode_attn needs: the partial outputs
 * [num_slots][num_q_heads][head_dim] plus their LSE [num_slots][num_q_heads],
 * each 256-byte aligned.  The partials are float32 with float32 LSE, except
 * when the tree's input and output are both bf16 and every piece of the plan
 * runs on the matrix cores (no PST_PLAN_DOT_SMALL): then each partial is
 * float16, scaled by a power of two 2^(15 - e) chosen from its piece's V,
 * and each LSE is an (LSE float32, e int32) pair.  The fp16 rounding
 * (2^-11 relative) is a quarter of the bf16 output's own. */
pst_status pst_plan_workspace_size(pst_plan_t plan, size_t* bytes);

/* Host views of a plan (bit-exact comparisons, introspection). */
#define PST_TASK_FIELDS 8 /* node, piece, kv_begin, kv_len, row_begin, row_count, flags, reserved */
#define PST_TASK_LAST_PIECE 1
#define PST_TASK_FLAT 2 /* a flattened chunk (PST_PLAN_FLATTEN) */
typedef struct {
  int32_t num_bins;
  int32_t num_tasks;
  int32_t num_queries;
  int32_t num_nodes;
  int64_t num_slots;
  int64_t num_entries;           /* node->query entries; flattened plans: (chunk, query) entries */
  const int32_t* tasks;          /* [num_tasks][PST_TASK_FIELDS], bin-major, assignment order */
  const int32_t* bin_ptr;        /* [num_bins + 1] */
  const int64_t* slot_ptr;       /* [num_queries + 1] */
  const int64_t* entry_slot;     /* [num_entries] first slot of each entry */
  const int32_t* piece_len;      /* [num_nodes] Lp (0 for nodes no query passes) */
  const int32_t* b_eff;          /* [num_nodes] pieces per node */
  const int32_t* rows_per_group; /* [num_nodes] */
  const int64_t* bin_load;       /* [num_bins] estimated ns */
  int64_t makespan;              /* estimated ns of the slowest bin */
  int64_t cost_l;                /* binary-search bound (0 for fixed geometries) */
  int32_t chosen_k;
  int32_t max_rows;
  int32_t mfma_min_rows;         /* bf16 pieces with at least this many rows use the matrix cores */
  int32_t flat_chunk;            /* S_t of a flattened plan, else 0 (the arrays below are then NULL) */
  int32_t num_chunks;
  const int32_t* flat_ptr;       /* [num_chunks + 1] entries of each chunk */
  const int32_t* flat_query;     /* [num_entries] query of each entry */
  const uint64_t* flat_mask;     /* [num_entries][flat_chunk / 64] bit causal masks */
  const int32_t* flat_rows;      /* [num_chunks * flat_chunk] pool row of each token, -1 past the end */
} pst_plan_view;
pst_status pst_plan_get(pst_plan_t plan, pst_plan_view* view);

/* The hot path: PAC then POR on `stream`.
 *   q        device, [B][H_q][d] in_dtype
 *   k_pool   device, in_dtype, layout from pst_shape
 *   v_pool   device, in_dtype, same layout as k_pool
 *   out      device, [B][H_q][d] out_dtype
 *   lse_out  device [B][H_q] float32, or NULL
 *   workspace device, >= pst_plan_workspace_size bytes, 256-byte aligned
 * Returns PST_E_PLAN_STALE if the tree was rebuilt under the plan,
 * PST_E_WORKSPACE if the workspace is missing or short, PST_E_NO_DEVICE for
 * host-only objects, PST_E_UNSUPPORTED if q spans more than 2^31 - 1 bytes. */
pst_status pst_decode_attn(pst_plan_t plan, const void* q, const void* k_pool, const void* v_pool,
                           void* out, float* lse_out, void* workspace, size_t workspace_bytes,
                           void* stream);

/* The two launches of pst_decode_attn, separately (for per-phase timing).
 * pst_pac writes the partials into the workspace; pst_por merges them into
 * out / lse_out.  pst_por must follow pst_pac on the same stream. */
pst_status pst_pac(pst_plan_t plan, const void* q, const void* k_pool, const void* v_pool,
                   void* workspace, size_t workspace_bytes, void* stream);
pst_status pst_por(pst_plan_t plan, void* out, float* lse_out, const void* workspace,
                   size_t workspace_bytes, void* stream);

/* The FlashDecoding-style comparator in the same library (KV-cache blog
 * section 4, FlashDecoding; DEFT section 3.3, Q-guided grouping): every
 * query's g rows form their own row groups, so a node shared by n_q queries
 * is read n_q times instead of once; the pieces, kernels and merge are those
 * of pst_decode_attn.  The tree keeps the query-guided plan it needs (made on
 * the first call with this cost model, NULL = the built-in model, default bins
 * for the current device; remade when the cost model changes) and frees it
 * with itself; growth through pst_tree_set_lengths keeps it valid.  The
 * tensors, their layouts and the workspace rules are those of
 * pst_decode_attn; the workspace size is pst_baseline_workspace_size's. */
pst_status pst_baseline_workspace_size(pst_tree_t tree, pst_cost_model_t cost, void* stream, size_t* bytes);
pst_status pst_decode_attn_baseline(pst_tree_t tree, pst_cost_model_t cost, const void* q, const void* k_pool,
                                    const void* v_pool, void* out, float* lse_out, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* A decode step's new K/V rows into the pools (DEFT section A.1: a request's
 * tree grows by the token it just decoded).  k_new, v_new: device,
 * [n][num_kv_heads][head_dim] in_dtype, contiguous; rows: device int64 [n],
 * the pool token each new row goes to (for a paged tree, page * page_size +
 * slot); k_pool, v_pool: the tree's pools, layout from pst_shape.  One launch
 * on `stream` writes every row of every kv head, K and V; rows outside
 * [0, pool_tokens) are not written.  Lengths are not changed: follow with
 * pst_tree_set_lengths. */
pst_status pst_write_kv_rows(pst_tree_t tree, const void* k_new, const void* v_new, const int64_t* rows, int32_t n,
                             void* k_pool, void* v_pool, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the hot
 * path of pst_decode_attn with the partial outputs in a scratch array the
 * library holds in device memory (PST_NOALLOC_SCRATCH_BYTES on every GPU it
 * runs on, from the library's load until the process ends) instead of a
 * caller workspace.  Allocates nothing: no hipMalloc, hipFree or allocating
 * library call.  q, k_pool, v_pool, out and lse_out are as for
 * pst_decode_attn, on the current device, which must be the plan's.
 * PST_E_WORKSPACE (nothing launched) when the plan's partial outputs
 * (pst_plan_workspace_size) exceed PST_NOALLOC_SCRATCH_BYTES.  Every call on
 * one GPU uses that GPU's one array: calls that overlap on a GPU (other
 * streams, other threads) race and must be serialised by the caller; the
 * array keeps the last call's partials, and nothing in it needs clearing
 * (every partial a call reads, the same call writes first). */
#define PST_NOALLOC_SCRATCH_BYTES ((size_t)128 << 20)
pst_status pst_decode_attn_noalloc(pst_plan_t plan, const void* q, const void* k_pool, const void* v_pool,
                                   void* out, float* lse_out, void* stream);

/* Release a tree, plan or cost model.  NULL is accepted.  A tree with live
 * plans (from pst_plan) is refused: free its plans first. */
pst_status pst_free(void* obj);

/* Thread-local message of the last failure in this thread ("" if none). */
const char* pst_last_error(void);

/* Device facts the planner uses: compute units and resident PAC workgroups
 * per compute unit on the current device. */
pst_status pst_device_info(int32_t* num_cu, int32_t* pac_blocks_per_cu);

/* Measurement helpers (not part of the attention).
 * pst_bench_flush: overwrite `bytes` of device memory at `buf` so that the
 * L2 and last-level caches hold nothing the next kernel reads.
 * pst_bench_read: read `bytes` (a multiple of 16) at `buf` with 128-bit loads
 * and write one float per workgroup into `sink` (>= 4096 floats): the
 * achievable HBM read bandwidth. */
pst_status pst_bench_flush(void* buf, size_t bytes, void* stream);
pst_status pst_bench_read(const void* buf, size_t bytes, float* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PST_H */
