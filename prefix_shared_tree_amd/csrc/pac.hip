// Partial attention computation (PAC) for prefix-shared tree decode attention, gfx950.
//
// CoDec: Prefix-Shared Decoding Kernel for LLMs, section 块内内核原语 (PAC
// kernel): a partial computation is ordinary attention between the queries
// aggregated from every request that shares one KV node and that node's K/V;
// K and V are brought on chip once and reused by all those queries, and the
// computation is cut into pieces that fit on chip and processed in turn.
// Section KV缓存管理: the queries are gathered into on-chip memory when the
// kernel starts (not materialised in global memory).  Section 块间启动与树归约:
// all pieces run in parallel, then a reduction merges each query's partials.
// DEFT: Decoding with Flash Tree-Attention, section A.4 (phase 1): each group
// returns its partial attention and LogSumExp for the reduction.
//
// Launch: one workgroup of 8 wavefronts per (plan bin, kv head); it runs the
// bin's pieces one after the other.  A piece is (node, KV range, row range);
// rows of a node are (node->query entry, head of the GQA group).
//
// Two paths, chosen per piece:
//  * matrix cores (bf16, >= 16 rows): K/V tiles of 64 tokens are staged in
//    LDS once for the whole workgroup (K row-major with an XOR swizzle, V
//    transposed so it can feed the MFMA's A operand), double-buffered with a
//    two-tile register prefetch; each wavefront owns 16 or 32 rows and half or
//    all of each tile's tokens and computes S^T = K Q^T and O^T += V^T P^T with
//    v_mfma_f32_16x16x32_bf16, so every row's softmax state stays in one lane;
//  * wavefront dot products (fewer rows, or float32): every group of
//    head_dim*elem/16 lanes streams one token at a time straight from HBM with
//    128-bit loads, reduces q.k across its lanes with DPP, and keeps a
//    running (max, sum, O) per row; states are merged across lane groups and
//    wavefronts at the end of the piece.
// Both use the streaming softmax of CoDec section KV缓存管理 (per-block
// maximum, rescale of the running sum and numerator at the common maximum)
// in base 2, and emit the normalised partial O and its natural-log LSE.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pst_internal.h"

namespace pst {
namespace {

typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2n __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int NW = kPacThreads / 64;  // wavefronts per workgroup
constexpr int TILE = kTile;           // tokens per tile
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_inff();
constexpr size_t kTileBytes = 64 * 1024;      // two stages of (K tile + transposed V tile) at d = 128
constexpr size_t kAuxBytes = 8 * 1024;        // softmax states exchanged between wavefronts
constexpr size_t kLdsBytes = kTileBytes + kAuxBytes;

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2n));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer over [base, base + bytes): loads past the end return zeros, so
// the ragged tail of a piece needs no branch.  Rebased per tile/block so the
// 32-bit offsets stay small whatever the pool size.
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit data format for gfx9-family buffer descriptors
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes < 0 ? 0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), static_cast<short>(0), n, kBufferWord3);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  typedef unsigned v4u __attribute__((ext_vector_type(4)));
  const v4u x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(x[0], x[1], x[2], x[3]);
}

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
// Sum over aligned groups of N lanes (N = 8, 16 or 32); every lane of the group gets the sum.
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp<0xB1>(x);   // quad_perm [1,0,3,2]: lane ^ 1
  x += dpp<0x4E>(x);   // quad_perm [2,3,0,1]: lane ^ 2
  x += dpp<0x141>(x);  // row_half_mirror: the other quad of each 8
  if (N >= 16) x += dpp<0x140>(x);  // row_mirror: the other half of each 16
  if (N >= 32) x += __shfl_xor(x, 16);
  return x;
}

// The workgroup's LDS (dynamic size kLdsBytes), visible to every path as LDS.
extern __shared__ __attribute__((aligned(16))) char pac_lds[];

struct TaskInfo {
  int node, piece, kv_begin, kv_len, row_begin, row_count;
  int e0;        // first node->query entry of the node
  int masked;    // node carries per-query masks
  const char* kbase;  // K of this kv head at the piece's first token
  const char* vbase;
};

// Row r of the task -> (query entry, q-head); returns false past the task's rows.
__device__ __forceinline__ bool row_target(const PacParams& p, const TaskInfo& t, int kvh, int r, int* entry, int* head) {
  if (r >= t.row_count) return false;
  const int rr = t.row_begin + r;
  *entry = t.e0 + rr / p.g;
  *head = kvh * p.g + rr % p.g;
  return true;
}

__device__ __forceinline__ void write_partial(const PacParams& p, const TaskInfo& t, int entry, int head, int D,
                                              int d0, const float* vals4, float lse, bool write_lse) {
  const int64_t slot = static_cast<int64_t>(p.entry_slot[entry]) + t.piece;
  float* dst = p.opart + (slot * p.hq + head) * D + d0;
  *reinterpret_cast<float4*>(dst) = make_float4(vals4[0], vals4[1], vals4[2], vals4[3]);
  if (write_lse) p.lsepart[slot * p.hq + head] = lse;
}

// ---------------------------------------------------------------------------
// Matrix-core path (bf16)
// ---------------------------------------------------------------------------
template <int D>
struct MfmaTile {
  static constexpr int CPT = D / 8;                  // 16-byte chunks per token row
  static constexpr int KCH = TILE * CPT / kPacThreads;  // K chunks each thread stages (D/64)
  static constexpr int VTHREADS = (TILE / 2) * CPT;     // threads staging V token pairs
  static constexpr int KBYTES = TILE * D * 2;
  static constexpr int VBYTES = D * TILE * 2;
  static constexpr int STAGE = KBYTES + VBYTES;
};

template <int D>
struct Staged {
  uint4 k[MfmaTile<D>::KCH];
  uint4 v0, v1;
};

template <int D>
__device__ __forceinline__ void stage_load(Staged<D>& s, const TaskInfo& t, int64_t stb, int tile0, int tid) {
  using M = MfmaTile<D>;
  const int64_t bytes = static_cast<int64_t>(min(TILE, t.kv_len - tile0)) * stb;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(t.kbase + tile0 * stb, bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(t.vbase + tile0 * stb, bytes);
#pragma unroll
  for (int c = 0; c < M::KCH; ++c) {
    const int chunk = tid + c * kPacThreads;
    const int tok = chunk / M::CPT, dc = chunk % M::CPT;
    s.k[c] = buf_load16(rk, static_cast<int>(tok * stb) + dc * 16, 0);
  }
  if (tid < M::VTHREADS) {
    const int pr = tid / M::CPT, dc = tid % M::CPT;
    const int off = static_cast<int>(2 * pr * stb) + dc * 16;
    s.v0 = buf_load16(rv, off, 0);
    s.v1 = buf_load16(rv, off + static_cast<int>(stb), 0);
  }
}

// Transposed V tile: row d holds 32 words, word w = tokens (2w, 2w+1) of the
// tile; the word position is XOR-swizzled by an even amount so that a word
// pair (4 tokens) stays together and both the transposing writes and the
// MFMA-operand reads of 16 consecutive rows spread over the banks.
__device__ __forceinline__ int vt_swz(int d) { return 2 * ((d & 15) ^ ((d >> 4) & 15)); }

template <int D>
__device__ __forceinline__ void stage_store(const Staged<D>& s, char* stage, int tid) {
  using M = MfmaTile<D>;
  uint16_t* Ks = reinterpret_cast<uint16_t*>(stage);
  uint32_t* Vt = reinterpret_cast<uint32_t*>(stage + M::KBYTES);
#pragma unroll
  for (int c = 0; c < M::KCH; ++c) {
    const int chunk = tid + c * kPacThreads;
    const int tok = chunk / M::CPT, dc = chunk % M::CPT;
    const int phys = dc ^ (tok & (M::CPT - 1));
    *reinterpret_cast<uint4*>(Ks + tok * D + phys * 8) = s.k[c];
  }
  if (tid < M::VTHREADS) {
    const int pr = tid / M::CPT, dc = tid % M::CPT;
    const uint32_t a[4] = {s.v0.x, s.v0.y, s.v0.z, s.v0.w};
    const uint32_t b[4] = {s.v1.x, s.v1.y, s.v1.z, s.v1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const uint32_t lo = (j & 1) ? (a[j >> 1] >> 16) : (a[j >> 1] & 0xffffu);
      const uint32_t hi = (j & 1) ? (b[j >> 1] & 0xffff0000u) : (b[j >> 1] << 16);
      const int d = dc * 8 + j;
      Vt[d * 32 + (pr ^ vt_swz(d))] = lo | hi;
    }
  }
}

// One piece on the matrix cores.  Each wavefront owns RBr blocks of 16 rows
// (RBr = 1 up to 64 rows, else 2) of a slab; TS wavefronts share a slab (TS =
// 2 while there are at most 4 slabs), each taking 64/TS tokens of every tile.
// Registers are sized for RB = 2; the second block is skipped when RBr = 1.
template <int D>
__device__ __forceinline__ void mfma_piece(const PacParams& p, const TaskInfo& t, int kvh) {
  char* const lds = pac_lds;
  using M = MfmaTile<D>;
  constexpr int RB = 2;
  constexpr int KS = D / 32;       // k-steps of S^T = K Q^T
  constexpr int DB = D / 16;       // d-blocks of O^T
  const int RBr = t.row_count <= 64 ? 1 : 2;
  const int ROWS_W = 16 * RBr;     // rows per wavefront
  const int slabs = (t.row_count + ROWS_W - 1) / ROWS_W;
  const int TS = slabs <= 4 ? 2 : 1;
  const int nsub = TS == 2 ? 1 : 2;  // 32-token sub-steps per wavefront per tile
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int slab = w / TS, half = w % TS;
  const bool active = slab < slabs;
  const int tok0 = half * (TILE / TS);
  const int64_t stb = p.stride_token * 2;

  // Gather the aggregated queries: B operand fragments of Q^T.
  bf16x8 qf[RB][KS];
  uint64_t rmask[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    int entry = 0, head = 0;
    const bool ok = active && rb < RBr && row_target(p, t, kvh, slab * ROWS_W + rb * 16 + l16, &entry, &head);
    const uint16_t* qrow =
        static_cast<const uint16_t*>(p.q) + (static_cast<int64_t>(ok ? p.nq_idx[entry] : 0) * p.hq + head) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      uint4 v = ok ? *reinterpret_cast<const uint4*>(qrow + ks * 32 + lg * 8) : make_uint4(0, 0, 0, 0);
      qf[rb][ks] = __builtin_bit_cast(bf16x8, v);
    }
    rmask[rb] = (ok && t.masked) ? p.nq_mask[entry] : ~0ull;
  }

  f32x4 o[DB][RB];
  float m[RB], l[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegInf;
    l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const int ntiles = (t.kv_len + TILE - 1) / TILE;
  Staged<D> sa;
  stage_load<D>(sa, t, stb, 0, tid);

  // One tile: the wavefront's 64/TS tokens in sub-steps of 32 (two 16-token
  // blocks); each sub-step updates the streaming softmax once.
  auto compute = [&](const char* stage, int tile) {
    const uint16_t* Ks = reinterpret_cast<const uint16_t*>(stage);
    const uint32_t* Vt = reinterpret_cast<const uint32_t*>(stage + M::KBYTES);
    for (int sub = 0; sub < nsub; ++sub) {
      const int tsub = tok0 + sub * 32;  // first token of the sub-step in the tile
      // S^T blocks: lane holds token rows (4 lg + i) of each 16-token block, query row l16.
      f32x4 s[2][RB];
#pragma unroll
      for (int hb = 0; hb < 2; ++hb) {
        const int tok = tsub + hb * 16 + l16;
#pragma unroll
        for (int rb = 0; rb < RB; ++rb) s[hb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          const int c = ks * 4 + lg;
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + tok * D + ((c ^ (tok & (M::CPT - 1))) * 8));
          s[hb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[0][ks], s[hb][0], 0, 0, 0);
          if (RBr == 2) s[hb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[1][ks], s[hb][1], 0, 0, 0);
        }
      }
      // Streaming softmax per row block (base 2), P packed to bf16 in the
      // MFMA k order: slots 0..3 = tokens 4 lg + i of block 0, slots 4..7 of block 1.
      bf16x8 bp[RB];
      bp[1] = bf16x8{};
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (rb >= RBr) continue;
        float mx = kNegInf;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const int tt = tile * TILE + tsub + hb * 16 + lg * 4 + i;
            const int bit = t.kv_begin + tt;
            const bool vis = tt < t.kv_len && (bit >= 64 || ((rmask[rb] >> bit) & 1ull));
            const float v = vis ? s[hb][rb][i] * p.scale_log2 : kNegInf;
            s[hb][rb][i] = v;
            mx = fmaxf(mx, v);
          }
        }
        mx = fmaxf(mx, __shfl_xor(mx, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(m[rb], mx);
        const float muse = mnew == kNegInf ? 0.f : mnew;
        const float alpha = fast_exp2(m[rb] - muse);
        m[rb] = mnew;
        float e[8];
        float ls = 0.f;
#pragma unroll
        for (int hb = 0; hb < 2; ++hb)
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            e[hb * 4 + i] = fast_exp2(s[hb][rb][i] - muse);
            ls += e[hb * 4 + i];
          }
        l[rb] = l[rb] * alpha + ls;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[db][rb] *= alpha;
        const uint4 u = make_uint4(pack_bf16(e[0], e[1]), pack_bf16(e[2], e[3]), pack_bf16(e[4], e[5]),
                                   pack_bf16(e[6], e[7]));
        bp[rb] = __builtin_bit_cast(bf16x8, u);
      }
      // O^T += V^T P^T over the 32 tokens: A = V^T rows d, tokens in the same slot order.
      const int pair0 = (tsub + lg * 4) >> 1;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int d = db * 16 + l16;
        const int swz = vt_swz(d);
        const uint2 x0 = *reinterpret_cast<const uint2*>(Vt + d * 32 + (pair0 ^ swz));
        const uint2 x1 = *reinterpret_cast<const uint2*>(Vt + d * 32 + ((pair0 + 8) ^ swz));
        const bf16x8 a = __builtin_bit_cast(bf16x8, make_uint4(x0.x, x0.y, x1.x, x1.y));
        o[db][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bp[0], o[db][0], 0, 0, 0);
        if (RBr == 2) o[db][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bp[1], o[db][1], 0, 0, 0);
      }
    }
  };

  // Two LDS stages, one register stage: tile i is written to LDS at the top
  // of its iteration, then the loads of tile i+1 are issued and tile i is computed.
  for (int tile = 0; tile < ntiles; ++tile) {
    char* st = lds + (tile & 1) * M::STAGE;
    stage_store<D>(sa, st, tid);
    __syncthreads();
    if (tile + 1 < ntiles) stage_load<D>(sa, t, stb, (tile + 1) * TILE, tid);
    if (active) compute(st, tile);
  }

  // Row sums: the four lane groups hold different tokens of the same rows.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l[rb] += __shfl_xor(l[rb], 16);
    l[rb] += __shfl_xor(l[rb], 32);
  }
  __syncthreads();  // all wavefronts are done with the tiles: reuse the LDS
  if (TS == 2) {  // uniform across the workgroup
    // Merge the two token halves of every slab: half 1 hands its state to half 0.
    float* so = reinterpret_cast<float*>(lds);          // [slab][rb][db][lane][4]
    float* sml = reinterpret_cast<float*>(lds + kTileBytes);  // [slab][rb][lane][2]
    if (active && half == 1) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (rb >= RBr) continue;
#pragma unroll
        for (int db = 0; db < DB; ++db)
          *reinterpret_cast<f32x4*>(so + (((slab * RB + rb) * DB + db) * 64 + lane) * 4) = o[db][rb];
        sml[((slab * RB + rb) * 64 + lane) * 2 + 0] = m[rb];
        sml[((slab * RB + rb) * 64 + lane) * 2 + 1] = l[rb];
      }
    }
    __syncthreads();
    if (active && half == 0) {
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (rb >= RBr) continue;
        const float m1 = sml[((slab * RB + rb) * 64 + lane) * 2 + 0];
        const float l1 = sml[((slab * RB + rb) * 64 + lane) * 2 + 1];
        const float mm = fmaxf(m[rb], m1);
        const float muse = mm == kNegInf ? 0.f : mm;
        const float a0 = fast_exp2(m[rb] - muse), a1 = fast_exp2(m1 - muse);
        l[rb] = l[rb] * a0 + l1 * a1;
        m[rb] = mm;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const f32x4 o1 = *reinterpret_cast<const f32x4*>(so + (((slab * RB + rb) * DB + db) * 64 + lane) * 4);
          o[db][rb] = o[db][rb] * a0 + o1 * a1;
        }
      }
    }
  }
  if (active && half == 0) {
#pragma unroll
    for (int rb = 0; rb < RB; ++rb) {
      int entry = 0, head = 0;
      if (rb >= RBr) continue;
      if (!row_target(p, t, kvh, slab * ROWS_W + rb * 16 + l16, &entry, &head)) continue;
      const float inv = l[rb] > 0.f ? 1.f / l[rb] : 0.f;
      const float lse = l[rb] > 0.f ? (m[rb] + __log2f(l[rb])) * kLn2 : kNegInf;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const float v4[4] = {o[db][rb][0] * inv, o[db][rb][1] * inv, o[db][rb][2] * inv, o[db][rb][3] * inv};
        write_partial(p, t, entry, head, D, db * 16 + lg * 4, v4, lse, db == 0 && lg == 0);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Wavefront dot-product path (any dtype, up to 16 rows)
// ---------------------------------------------------------------------------
template <typename T>
struct Elem;
template <>
struct Elem<float> {
  static constexpr int N = 4;  // elements per 16-byte chunk
  static constexpr int W = 4;  // 32-bit words per chunk
  // q.k over one chunk; q holds the row's 4 floats as words.
  __device__ __forceinline__ static float dot(const uint32_t* q, const uint4& k, float acc) {
    acc = fmaf(__uint_as_float(q[0]), __uint_as_float(k.x), acc);
    acc = fmaf(__uint_as_float(q[1]), __uint_as_float(k.y), acc);
    acc = fmaf(__uint_as_float(q[2]), __uint_as_float(k.z), acc);
    return fmaf(__uint_as_float(q[3]), __uint_as_float(k.w), acc);
  }
  __device__ __forceinline__ static void unpack(const uint4& u, float* f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
};
template <>
struct Elem<uint16_t> {  // bfloat16 bits
  static constexpr int N = 8;
  static constexpr int W = 4;
  // Products of two bf16 values are exact in float32; v_dot2_f32_bf16 sums pairs.
  __device__ __forceinline__ static float dot(const uint32_t* q, const uint4& k, float acc) {
    typedef __bf16 bf2 __attribute__((ext_vector_type(2)));
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, q[0]), __builtin_bit_cast(bf2, k.x), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, q[1]), __builtin_bit_cast(bf2, k.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, q[2]), __builtin_bit_cast(bf2, k.z), acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf2, q[3]), __builtin_bit_cast(bf2, k.w), acc, false);
  }
  __device__ __forceinline__ static void unpack(const uint4& u, float* f) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = bf16_lo(w[i]);
      f[2 * i + 1] = bf16_hi(w[i]);
    }
  }
};

// Up to RL = 8 rows per lane; RS row splits (2 when the piece has more than 8
// rows): lanes [k*64/RS, (k+1)*64/RS) own rows [k*RL, (k+1)*RL) and stream the
// same tokens (their loads coalesce).
template <typename T, int D>
__device__ __forceinline__ void dot_piece(const PacParams& p, const TaskInfo& t, int kvh) {
  char* const lds = pac_lds;
  constexpr int RL = 8;
  constexpr int E = Elem<T>::N;
  constexpr int LPT = D / E;             // lanes per token
  constexpr int U = 2;                   // tokens per stream in flight per stage
  const int RS = (t.row_count > RL && 64 / LPT >= 2) ? 2 : 1;
  const int LPS = 64 / RS;               // lanes per row split
  const int TPI = LPS / LPT;             // tokens per row split per instruction
  const int NS = NW * TPI;               // token streams in the workgroup
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int rs = lane / LPS;
  const int tg = (lane % LPS) / LPT, li = lane % LPT;
  const int stream = w * TPI + tg;
  const int64_t stb = p.stride_token * static_cast<int64_t>(sizeof(T));
  const int R = t.row_count;
  const int r0 = rs * RL;

  uint32_t q[RL][Elem<T>::W];
#pragma unroll
  for (int r = 0; r < RL; ++r) {
    int entry = 0, head = 0;
    const bool ok = row_target(p, t, kvh, r0 + r, &entry, &head);
    uint4 u = make_uint4(0, 0, 0, 0);
    if (ok) {
      const T* qrow = static_cast<const T*>(p.q) + (static_cast<int64_t>(p.nq_idx[entry]) * p.hq + head) * D;
      u = *reinterpret_cast<const uint4*>(qrow + li * E);
    }
    q[r][0] = u.x;
    q[r][1] = u.y;
    q[r][2] = u.z;
    q[r][3] = u.w;
  }
  const int nr = min(RL, max(0, R - r0));  // live rows of this lane (uniform per row split)
  float o[RL][E];
  float m[RL], l[RL];
#pragma unroll
  for (int r = 0; r < RL; ++r) {
    m[r] = kNegInf;
    l[r] = 0.f;
#pragma unroll
    for (int e = 0; e < E; ++e) o[r][e] = 0.f;
  }

  const int n = t.kv_len;
  const int BLK = NS * U;  // tokens per block
  const int voff = static_cast<int>(stream * stb) + li * 16;
  // Token of (block b, slot u) for this lane group: b * BLK + u * NS + stream.
  auto load_block = [&](uint4* kk, uint4* vv, int b) {
    const int64_t bytes = static_cast<int64_t>(min(BLK, n - b * BLK)) * stb;
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(t.kbase + b * BLK * stb, bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(t.vbase + b * BLK * stb, bytes);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      // The whole offset goes in the VGPR operand: the range check ignores soffset.
      kk[u] = buf_load16(rk, voff + static_cast<int>(u * NS * stb), 0);
      vv[u] = buf_load16(rv, voff + static_cast<int>(u * NS * stb), 0);
    }
  };
  // Visibility of token tt of the piece for row r of this lane.
  auto visible = [&](int r, int tt) {
    if (tt >= n) return false;
    if (!t.masked) return true;
    const int bit = t.kv_begin + tt;
    if (bit >= 64) return true;
    return ((p.nq_mask[t.e0 + (t.row_begin + r0 + r) / p.g] >> bit) & 1ull) != 0;
  };
  const int nblocks = (n + BLK - 1) / BLK;
  uint4 ka[U], va[U], kb[U], vb[U];
  load_block(ka, va, 0);
  auto process = [&](const uint4* kk, const uint4* vv, int b) {
    float s[U][RL];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int r = 0; r < RL; ++r) s[u][r] = r < nr ? group_sum<LPT>(Elem<T>::dot(q[r], kk[u], 0.f)) : 0.f;
    float alpha[RL];
#pragma unroll
    for (int r = 0; r < RL; ++r) {
      float mx = kNegInf;
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float v = (r < nr && visible(r, b * BLK + u * NS + stream)) ? s[u][r] * p.scale_log2 : kNegInf;
        s[u][r] = v;
        mx = fmaxf(mx, v);
      }
      const float mnew = fmaxf(m[r], mx);
      const float muse = mnew == kNegInf ? 0.f : mnew;
      alpha[r] = fast_exp2(m[r] - muse);
      m[r] = mnew;
      l[r] *= alpha[r];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        s[u][r] = fast_exp2(s[u][r] - muse);
        l[r] += s[u][r];
      }
#pragma unroll
      for (int e = 0; e < E; ++e) o[r][e] *= alpha[r];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[E];
      Elem<T>::unpack(vv[u], vf);
#pragma unroll
      for (int r = 0; r < RL; ++r)
#pragma unroll
        for (int e = 0; e < E; ++e) o[r][e] = fmaf(s[u][r], vf[e], o[r][e]);
    }
  };
  for (int b = 0; b < nblocks; b += 2) {
    if (b + 1 < nblocks) load_block(kb, vb, b + 1);
    process(ka, va, b);
    if (b + 1 < nblocks) {
      if (b + 2 < nblocks) load_block(ka, va, b + 2);
      process(kb, vb, b + 1);
    }
  }

  // Merge the TPI token streams of this row split (lanes li, li + LPT, ...).
#pragma unroll
  for (int off = LPT; off < LPS; off <<= 1) {
#pragma unroll
    for (int r = 0; r < RL; ++r) {
      if (r < nr) {
        const float m2 = __shfl_xor(m[r], off);
        const float l2 = __shfl_xor(l[r], off);
        const float mm = fmaxf(m[r], m2);
        const float muse = mm == kNegInf ? 0.f : mm;
        const float a1 = fast_exp2(m[r] - muse), a2 = fast_exp2(m2 - muse);
        l[r] = l[r] * a1 + l2 * a2;
        m[r] = mm;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const float o2 = __shfl_xor(o[r][e], off);
          o[r][e] = o[r][e] * a1 + o2 * a2;
        }
      }
    }
  }
  // Merge across wavefronts through LDS: [wave][row][D] numerators, [wave][row] (m, l).
  const int RT = RL * RS;  // rows per wavefront
  float* so = reinterpret_cast<float*>(lds);
  float* sml = reinterpret_cast<float*>(lds + kTileBytes);
  __syncthreads();  // previous users of the LDS are done
  if (tg == 0) {
#pragma unroll
    for (int r = 0; r < RL; ++r) {
      if (r < nr) {
        const int row = r0 + r;
#pragma unroll
        for (int e = 0; e < E; ++e) so[(w * RT + row) * D + li * E + e] = o[r][e];
        if (li == 0) {
          sml[(w * RT + row) * 2 + 0] = m[r];
          sml[(w * RT + row) * 2 + 1] = l[r];
        }
      }
    }
  }
  __syncthreads();
  // Thread -> (row, 4 channels).
  constexpr int C4 = D / 4;
  for (int idx = tid; idx < R * C4; idx += kPacThreads) {
    const int r = idx / C4, c4 = idx % C4;
    float mm = kNegInf;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) mm = fmaxf(mm, sml[(ww * RT + r) * 2]);
    const float muse = mm == kNegInf ? 0.f : mm;
    float lt = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float a = fast_exp2(sml[(ww * RT + r) * 2] - muse);
      lt += a * sml[(ww * RT + r) * 2 + 1];
      const float4 x = *reinterpret_cast<const float4*>(so + (ww * RT + r) * D + c4 * 4);
      acc[0] += a * x.x;
      acc[1] += a * x.y;
      acc[2] += a * x.z;
      acc[3] += a * x.w;
    }
    int entry = 0, head = 0;
    row_target(p, t, kvh, r, &entry, &head);
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse = lt > 0.f ? (mm + __log2f(lt)) * kLn2 : kNegInf;
    const float v4[4] = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    write_partial(p, t, entry, head, D, c4 * 4, v4, lse, c4 == 0);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kPacThreads) void pac_kernel(PacParams p) {
  const int bin = blockIdx.x % p.num_bins;
  const int kvh = blockIdx.x / p.num_bins;
  const int tb = p.bin_ptr[bin], te = p.bin_ptr[bin + 1];
  const int64_t esz = sizeof(T);
  for (int ti = tb; ti < te; ++ti) {
    const Task task = p.tasks[ti];
    TaskInfo t;
    t.node = task.node;
    t.piece = task.piece;
    t.kv_begin = task.kv_begin;
    t.kv_len = (task.flags & PST_TASK_LAST_PIECE) ? p.node_len[task.node] - task.kv_begin : task.kv_len;
    t.row_begin = task.row_begin;
    t.row_count = task.row_count;
    t.e0 = p.nq_ptr[task.node];
    t.masked = p.node_masked[task.node];
    const int64_t tok = p.node_off[task.node] + task.kv_begin;
    const int64_t off = (kvh * p.stride_head + tok * p.stride_token) * esz;
    t.kbase = static_cast<const char*>(p.k) + off;
    t.vbase = static_cast<const char*>(p.v) + off;
    const int R = t.row_count;
    if constexpr (sizeof(T) == 2) {
      if (R >= kMfmaMinRows) {
        mfma_piece<D>(p, t, kvh);
        __syncthreads();
        continue;
      }
    }
    dot_piece<T, D>(p, t, kvh);
    __syncthreads();
  }
}

template <typename T, int D>
int launch_one(const PacParams& p, void* stream) {
  const int grid = p.num_bins * p.hkv;
  static bool configured = false;
  if (!configured) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&pac_kernel<T, D>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(kLdsBytes));
    if (e != hipSuccess) return static_cast<int>(e);
    configured = true;
  }
  hipLaunchKernelGGL((pac_kernel<T, D>), dim3(grid), dim3(kPacThreads), kLdsBytes, static_cast<hipStream_t>(stream), p);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

size_t pac_lds_bytes() { return kLdsBytes; }

int launch_pac(const PacParams& p, int in_dtype, int head_dim, void* stream) {
  if (in_dtype == PST_BF16) return head_dim == 128 ? launch_one<uint16_t, 128>(p, stream) : launch_one<uint16_t, 64>(p, stream);
  return head_dim == 128 ? launch_one<float, 128>(p, stream) : launch_one<float, 64>(p, stream);
}

int pac_blocks_per_cu(int in_dtype, int head_dim, int* blocks) {
  hipError_t e;
  if (in_dtype == PST_BF16 && head_dim == 128)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, pac_kernel<uint16_t, 128>, kPacThreads, kLdsBytes);
  else if (in_dtype == PST_BF16)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, pac_kernel<uint16_t, 64>, kPacThreads, kLdsBytes);
  else if (head_dim == 128)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, pac_kernel<float, 128>, kPacThreads, kLdsBytes);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, pac_kernel<float, 64>, kPacThreads, kLdsBytes);
  return static_cast<int>(e);
}

}  // namespace pst
