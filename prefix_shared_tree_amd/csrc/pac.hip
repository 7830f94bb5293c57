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
// Memory pipeline (both paths): the piece's K and V stream through LDS in
// 16 KB tiles (64 tokens at d = 128 bf16) by direct HBM->LDS DMA
// (buffer_load_dwordx4 ... lds), four stages deep, so three tiles are in
// flight while one is computed and no registers hold staged data.  Rows are
// XOR-swizzled by 16-byte chunk so the reads below spread over the banks;
// loads past the piece end return zeros.
//
// Two compute paths, chosen per piece:
//  * matrix cores (bf16, >= 16 rows): each wavefront owns 16 or 32 rows and
//    half or all of each tile's tokens and computes S^T = K Q^T and
//    O^T += V^T P^T with v_mfma_f32_16x16x32_bf16, so every row's softmax
//    state stays in one lane.  V^T fragments come straight from the row-major
//    tile with the LDS transpose read ds_read_b64_tr_b16.  P enters the MFMA
//    as a bf16 hi/lo pair so its rounding stays near float32;
//  * wavefront dot products (fewer rows, or float32): groups of
//    head_dim*elem/16 lanes take one token each, reduce q.k across the group
//    with DPP, and keep a running (max, sum, O) per row; states are merged
//    across lane groups and wavefronts at the end of the piece.
// Both use the streaming softmax of CoDec section KV缓存管理 (per-block
// maximum, rescale of the running sum and numerator at the common maximum)
// in base 2, and emit the normalised partial O and its natural-log LSE.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "pst_internal.h"

namespace pst {
namespace {

typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef short bf16x4s __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2n __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int NW = kPacThreads / 64;  // wavefronts per workgroup
constexpr int NSTAGE = 4;             // LDS tile stages
constexpr int TILE_BYTES = 16384;     // bytes of one K (or V) tile
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLazy = 8.0f;  // log2 headroom before the reference maximum is raised
constexpr size_t kTileBytes = static_cast<size_t>(NSTAGE) * STAGE_BYTES;  // 128 KB of tile stages
constexpr size_t kAuxBytes = 8 * 1024;  // softmax states exchanged between wavefronts
constexpr size_t kLdsBytes = kTileBytes + kAuxBytes;
static_assert(kTileBytes >= 64 * 1024, "merge scratch reuses the tile stages");

// The workgroup's LDS (dynamic size kLdsBytes), visible to every path as LDS.
extern __shared__ __attribute__((aligned(16))) char pac_lds[];

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2n));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer over [base, base + bytes): loads past the end return zeros, so
// the ragged tail of a piece needs no branch.  Rebased per tile so the 32-bit
// offsets stay small whatever the pool size.
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit data format for gfx9-family buffer descriptors
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes < 0 ? 0 : bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(base), static_cast<short>(0), n, kBufferWord3);
}

// One 16-byte-per-lane HBM->LDS DMA: LDS destination = lds_addr + 16 * lane.
// Written as inline assembly so the compiler does not see an LDS store in
// flight: it would otherwise wait for every outstanding DMA before each LDS
// read.  The tile loop waits explicitly (wait_vmem) for the tile it reads.
// M0 carries the destination and is restored afterwards.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int voff, uint32_t lds_addr) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "buffer_load_dwordx4 %1, %2, 0 offen lds\n\t"
      "s_nop 0\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
      : "memory");
}
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}

// Wait until at most n of this wavefront's vector memory operations are
// outstanding (n in {0, 4, 8}); expcnt and lgkmcnt are left alone.
__device__ __forceinline__ void wait_vmem(int n) {
  if (n >= 8)
    __builtin_amdgcn_s_waitcnt(0x0F78);
  else if (n >= 4)
    __builtin_amdgcn_s_waitcnt(0x0F74);
  else
    __builtin_amdgcn_s_waitcnt(0x0F70);
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

template <int D, int EB>
struct Geo {
  static constexpr int ROWB = D * EB;           // bytes per token row
  static constexpr int CPT = ROWB / 16;         // 16-byte chunks per row
  static constexpr int TT = TILE_BYTES / ROWB;  // tokens per tile
};

struct TaskInfo {
  int piece, kv_begin, kv_len, row_begin, row_count, e0, masked;
  const char* kbase;  // K of this kv head at the piece's first token
  const char* vbase;
};

// Row r of the task -> (query entry, q-head); returns false past the task's rows.
__device__ __forceinline__ bool row_target(const PacParams& p, const TaskInfo& t, int kvh, int r, int* entry,
                                           int* head) {
  if (r >= t.row_count) return false;
  const int rr = t.row_begin + r;
  *entry = t.e0 + rr / p.g;
  *head = kvh * p.g + rr % p.g;
  return true;
}

// `slot` = first partial slot of the row's (query, node) entry (prefetched);
// the piece's slot is slot + piece.
__device__ __forceinline__ void write_partial(const PacParams& p, const TaskInfo& t, int slot0, int head, int D,
                                              int d0, const float* vals4, float lse, bool write_lse) {
  const int64_t slot = static_cast<int64_t>(slot0) + t.piece;
  float* dst = p.opart + (slot * p.hq + head) * D + d0;
  *reinterpret_cast<float4*>(dst) = make_float4(vals4[0], vals4[1], vals4[2], vals4[3]);
  if (write_lse) p.lsepart[slot * p.hq + head] = lse;
}

// DMA of tile `tile` of the piece into stage `stage`: every wavefront writes
// two 1 KB blocks of K and two of V; lane L of a block fills 16-byte chunk
// position P = block*64 + L, i.e. token P / CPT, chunk (P % CPT) ^ (token % CPT).
template <int D, int EB>
__device__ __forceinline__ void issue_tile(const TaskInfo& t, int64_t stb, int tile, int stage, int tid) {
  using G = Geo<D, EB>;
  const int tok_base = tile * G::TT;
  const int64_t bytes = static_cast<int64_t>(min(G::TT, t.kv_len - tok_base)) * stb;
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(t.kbase + tok_base * stb, bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(t.vbase + tok_base * stb, bytes);
  const int lane = tid & 63, w = tid >> 6;
  char* st = pac_lds + stage * STAGE_BYTES;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int b = c * NW + w;
    const int P = b * 64 + lane;
    const int tok = P / G::CPT, phys = P % G::CPT;
    const int voff = static_cast<int>(tok * stb) + ((phys ^ (tok & (G::CPT - 1))) << 4);
    dma16(rk, voff, lds_addr(st + b * 1024));
    dma16(rv, voff, lds_addr(st + TILE_BYTES + b * 1024));
  }
}

// Tiles 0 .. NSTAGE-2 (issued before the queries are gathered).
template <int D, int EB>
__device__ __forceinline__ void issue_prologue(const TaskInfo& t, int64_t stb, int tid) {
  using G = Geo<D, EB>;
  const int ntiles = (t.kv_len + G::TT - 1) / G::TT;
#pragma unroll
  for (int i = 0; i < NSTAGE - 1; ++i)
    if (i < ntiles) issue_tile<D, EB>(t, stb, i, i, tid);
}

// The tile loop: wait for tile i (4 DMA operations per thread and tile), a
// barrier without a memory fence (which would drain every DMA in flight),
// refill the stage of tile i-1 with tile i+3, compute tile i.
template <int D, int EB, typename F>
__device__ __forceinline__ void run_tiles(const TaskInfo& t, int64_t stb, int tid, F&& compute) {
  using G = Geo<D, EB>;
  const int ntiles = (t.kv_len + G::TT - 1) / G::TT;
  for (int tile = 0; tile < ntiles; ++tile) {
    wait_vmem(4 * min(NSTAGE - 2, ntiles - 1 - tile));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS access moves above the barrier
    if (tile + NSTAGE - 1 < ntiles) issue_tile<D, EB>(t, stb, tile + NSTAGE - 1, (tile + NSTAGE - 1) % NSTAGE, tid);
    compute(pac_lds + (tile % NSTAGE) * STAGE_BYTES, tile);
  }
}

// ---------------------------------------------------------------------------
// Matrix-core path (bf16)
// ---------------------------------------------------------------------------
// Each wavefront owns RBr blocks of 16 rows (RBr = 1 up to 64 rows, else 2)
// of a slab; TS wavefronts share a slab (TS = 2 while there are at most 4
// slabs), each taking TT/TS tokens of every tile in sub-steps of 32.
// Registers are sized for RB = 2; the second block is skipped when RBr = 1.
template <int D>
__device__ __forceinline__ void mfma_piece(const PacParams& p, const TaskInfo& t, int kvh) {
  using G = Geo<D, 2>;
  char* const lds = pac_lds;
  constexpr int RB = 2;
  constexpr int KS = D / 32;  // k-steps of S^T = K Q^T
  constexpr int DB = D / 16;  // d-blocks of O^T
  const int RBr = t.row_count <= 64 ? 1 : 2;
  const int ROWS_W = 16 * RBr;
  const int slabs = (t.row_count + ROWS_W - 1) / ROWS_W;
  const int TS = slabs <= 4 ? 2 : 1;
  const int nsub = G::TT / (32 * TS);  // 32-token sub-steps per wavefront per tile
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int l16 = lane & 15, lg = lane >> 4;
  const int slab = w / TS, half = w % TS;
  const bool active = slab < slabs;
  const int tok0 = half * (G::TT / TS);
  const int64_t stb = p.stride_token * 2;

  issue_prologue<D, 2>(t, stb, tid);

  // Gather the aggregated queries: B operand fragments of Q^T.  Branch-free
  // (dead rows read row 0 of the task and are zeroed) so that all index loads
  // and then all query loads are in flight together.
  bf16x8 qf[RB][KS];
  bool qok[RB];
  int qrow_off[RB], slot0[RB], qhead[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    int entry = t.e0 + t.row_begin / p.g, head = kvh * p.g + t.row_begin % p.g;
    qok[rb] = active && rb < RBr && row_target(p, t, kvh, slab * ROWS_W + rb * 16 + l16, &entry, &head);
    qrow_off[rb] = p.nq_idx[entry] * p.hq + head;
    slot0[rb] = p.entry_slot[entry];
    qhead[rb] = head;
  }
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    const uint16_t* qrow = static_cast<const uint16_t*>(p.q) + static_cast<int64_t>(qrow_off[rb]) * D;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint4 v = *reinterpret_cast<const uint4*>(qrow + ks * 32 + lg * 8);
      const uint4 z = make_uint4(qok[rb] ? v.x : 0u, qok[rb] ? v.y : 0u, qok[rb] ? v.z : 0u, qok[rb] ? v.w : 0u);
      qf[rb][ks] = __builtin_bit_cast(bf16x8, z);
    }
  }
  // The queries must be in registers before the tile loop: without this wait
  // the compiler would wait for them (and every DMA behind them) inside it.
  wait_vmem(0);
  // Mask of a row (masked nodes only; read when needed).
  auto row_mask = [&](int rb) -> uint64_t {
    int entry = 0, head = 0;
    if (!row_target(p, t, kvh, slab * ROWS_W + rb * 16 + l16, &entry, &head)) return ~0ull;
    return p.nq_mask[entry];
  };

  f32x4 o[DB][RB];
  float m[RB], l[RB];
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    m[rb] = kNegInf;
    l[rb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  auto compute = [&](const char* stage, int tile) {
    if (!active) return;
    const char* Ks = stage;
    const char* Vs = stage + TILE_BYTES;
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
          const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + tok * G::ROWB + ((c ^ (tok & (G::CPT - 1))) << 4));
          s[hb][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[0][ks], s[hb][0], 0, 0, 0);
          if (RBr == 2) s[hb][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[1][ks], s[hb][1], 0, 0, 0);
        }
      }
      // Streaming softmax per row block (base 2), P in the MFMA k order:
      // slots 0..3 = tokens 4 lg + i of block 0, slots 4..7 of block 1.
      // m is the reference maximum in scaled units.  It is raised only when a
      // score exceeds it by more than kLazy (then p <= 2^kLazy, harmless in
      // float32), so the cross-lane maximum and the rescale of O are skipped
      // in almost every step.  Full tiles of unmasked nodes skip the
      // visibility test.
      const bool full = !t.masked && (tile + 1) * G::TT <= t.kv_len;
      bf16x8 bp[RB], bq[RB];
      bp[1] = bf16x8{};
      bq[1] = bf16x8{};
#pragma unroll
      for (int rb = 0; rb < RB; ++rb) {
        if (rb >= RBr) continue;
        // Scaled scores (base 2); invisible tokens -inf.
        float v[8];
        if (full) {
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int i = 0; i < 4; ++i) v[hb * 4 + i] = s[hb][rb][i] * p.scale_log2;
        } else {
          const uint64_t rmask = t.masked ? row_mask(rb) : ~0ull;
#pragma unroll
          for (int hb = 0; hb < 2; ++hb)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
              const int tt = tile * G::TT + tsub + hb * 16 + lg * 4 + i;
              const int bit = t.kv_begin + tt;
              const bool vis = tt < t.kv_len && (bit >= 64 || ((rmask >> bit) & 1ull));
              v[hb * 4 + i] = vis ? s[hb][rb][i] * p.scale_log2 : kNegInf;
            }
        }
        float mx = kNegInf;
#pragma unroll
        for (int j = 0; j < 8; ++j) mx = fmaxf(mx, v[j]);
        if (__builtin_amdgcn_ballot_w64(mx > m[rb] + kLazy) != 0) {
          mx = fmaxf(mx, __shfl_xor(mx, 16));
          mx = fmaxf(mx, __shfl_xor(mx, 32));
          const float mnew = mx > m[rb] + kLazy ? mx : m[rb];
          const float alpha = mnew == m[rb] ? 1.f : fast_exp2(m[rb] - mnew);  // 0 when m was -inf
          m[rb] = mnew;
          l[rb] *= alpha;
#pragma unroll
          for (int db = 0; db < DB; ++db) o[db][rb] *= alpha;
        }
        const float muse = m[rb] == kNegInf ? 0.f : m[rb];
        float e[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          e[j] = fast_exp2(v[j] - muse);
          l[rb] += e[j];
        }
        // P = hi + lo with hi = bf16(P) and lo = bf16(P - hi).
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          hw[j] = pack_bf16(e[2 * j], e[2 * j + 1]);
          lw[j] = pack_bf16(e[2 * j] - bf16_lo(hw[j]), e[2 * j + 1] - bf16_hi(hw[j]));
        }
        bp[rb] = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
        bq[rb] = __builtin_bit_cast(bf16x8, make_uint4(lw[0], lw[1], lw[2], lw[3]));
      }
      // O^T += V^T P^T over the 32 tokens.  A = V^T rows d = 16 db + l16: two
      // transpose reads, tokens tsub + 4 lg + 0..3 and tsub + 16 + 4 lg + 0..3;
      // source lane s of each 16-lane group points at token (t0 + s/4),
      // channels 16 db + 4 (s%4) .. +3.
      const int ta = tsub + 4 * lg + (l16 >> 2), tb2 = ta + 16;
      const int dq = 4 * (l16 & 3);
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const int c = (db * 16 + dq) >> 3, hoff = ((db * 16 + dq) & 7) * 2;
        const char* pa = Vs + ta * G::ROWB + ((c ^ (ta & (G::CPT - 1))) << 4) + hoff;
        const char* pb = Vs + tb2 * G::ROWB + ((c ^ (tb2 & (G::CPT - 1))) << 4) + hoff;
        const bf16x4s x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) bf16x4s*)(pa));
        const bf16x4s x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) bf16x4s*)(pb));
        const bf16x8 a = __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7);
        o[db][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bp[0], o[db][0], 0, 0, 0);
        o[db][0] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq[0], o[db][0], 0, 0, 0);
        if (RBr == 2) {
          o[db][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bp[1], o[db][1], 0, 0, 0);
          o[db][1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bq[1], o[db][1], 0, 0, 0);
        }
      }
    }
  };

  run_tiles<D, 2>(t, stb, tid, compute);

  // Row sums: the four lane groups hold different tokens of the same rows.
#pragma unroll
  for (int rb = 0; rb < RB; ++rb) {
    l[rb] += __shfl_xor(l[rb], 16);
    l[rb] += __shfl_xor(l[rb], 32);
  }
  __syncthreads();  // all wavefronts are done with the tiles: reuse the LDS
  if (TS == 2) {    // uniform across the workgroup
    // Merge the two token halves of every slab: half 1 hands its state to half 0.
    float* so = reinterpret_cast<float*>(lds);                // [slab][rb][db][lane][4]
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
      if (!qok[rb]) continue;
      const float inv = l[rb] > 0.f ? 1.f / l[rb] : 0.f;
      const float lse = l[rb] > 0.f ? (m[rb] + __log2f(l[rb])) * kLn2 : kNegInf;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const float v4[4] = {o[db][rb][0] * inv, o[db][rb][1] * inv, o[db][rb][2] * inv, o[db][rb][3] * inv};
        write_partial(p, t, slot0[rb], qhead[rb], D, db * 16 + lg * 4, v4, lse, db == 0 && lg == 0);
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
// rows): lanes [k*64/RS, (k+1)*64/RS) own rows [k*RL, (k+1)*RL) and read the
// same tokens.  Each wavefront takes TT/8 tokens of every tile, TPI at a time.
template <typename T, int D>
__device__ __forceinline__ void dot_piece(const PacParams& p, const TaskInfo& t, int kvh) {
  constexpr int EB = sizeof(T);
  using G = Geo<D, EB>;
  char* const lds = pac_lds;
  constexpr int RL = 8;
  constexpr int E = Elem<T>::N;
  constexpr int LPT = G::CPT;                // lanes per token (one chunk each)
  constexpr int TPW = G::TT / NW;            // tokens per wavefront per tile
  constexpr int SPMAX = TPW * LPT * 2 / 64;  // steps per tile at RS = 2
  const int RS = (t.row_count > RL && 64 / LPT >= 2) ? 2 : 1;
  const int LPS = 64 / RS;    // lanes per row split
  const int TPI = LPS / LPT;  // tokens per row split per step
  const int nsteps = TPW / TPI;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int rs = lane / LPS;
  const int tg = (lane % LPS) / LPT, li = lane % LPT;
  const int64_t stb = p.stride_token * static_cast<int64_t>(EB);
  const int R = t.row_count;
  const int r0 = rs * RL;

  issue_prologue<D, EB>(t, stb, tid);

  // Branch-free gather (dead rows read row 0 of the task and are zeroed).
  uint32_t q[RL][4];
  int qrow_off[RL];
  bool qok[RL];
#pragma unroll
  for (int r = 0; r < RL; ++r) {
    int entry = t.e0 + t.row_begin / p.g, head = kvh * p.g + t.row_begin % p.g;
    qok[r] = row_target(p, t, kvh, r0 + r, &entry, &head);
    qrow_off[r] = p.nq_idx[entry] * p.hq + head;
  }
#pragma unroll
  for (int r = 0; r < RL; ++r) {
    const T* qrow = static_cast<const T*>(p.q) + static_cast<int64_t>(qrow_off[r]) * D;
    const uint4 u = *reinterpret_cast<const uint4*>(qrow + li * E);
    q[r][0] = qok[r] ? u.x : 0u;  // selects, not branches: the loads stay in flight together
    q[r][1] = qok[r] ? u.y : 0u;
    q[r][2] = qok[r] ? u.z : 0u;
    q[r][3] = qok[r] ? u.w : 0u;
  }
  // The row this thread writes at the end (one (row, 4 channels) per thread).
  constexpr int C4 = D / 4;
  static_assert(kMaxRowsDot * C4 <= kPacThreads, "one output chunk per thread");
  const int out_r = tid / C4, out_c4 = tid % C4;
  int out_slot = 0, out_head = 0;
  {
    int entry = t.e0 + t.row_begin / p.g, head = kvh * p.g + t.row_begin % p.g;
    row_target(p, t, kvh, out_r, &entry, &head);
    out_slot = p.entry_slot[entry];
    out_head = head;
  }
  wait_vmem(0);  // queries in registers before the tile loop (see the matrix-core path)
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
  // Visibility of token tt of the piece for row r of this lane.
  auto visible = [&](int r, int tt) {
    if (tt >= t.kv_len) return false;
    if (!t.masked) return true;
    const int bit = t.kv_begin + tt;
    if (bit >= 64) return true;
    return ((p.nq_mask[t.e0 + (t.row_begin + r0 + r) / p.g] >> bit) & 1ull) != 0;
  };

  auto compute = [&](const char* stage, int tile) {
    const char* Ks = stage;
    const char* Vs = stage + TILE_BYTES;
    float s[SPMAX][RL];
    uint4 vv[SPMAX];
#pragma unroll
    for (int sp = 0; sp < SPMAX; ++sp) {
      if (sp < nsteps) {
        const int tok = w * TPW + sp * TPI + tg;
        const int off = tok * G::ROWB + ((li ^ (tok & (G::CPT - 1))) << 4);
        const uint4 kk = *reinterpret_cast<const uint4*>(Ks + off);
        vv[sp] = *reinterpret_cast<const uint4*>(Vs + off);
#pragma unroll
        for (int r = 0; r < RL; ++r) s[sp][r] = r < nr ? group_sum<LPT>(Elem<T>::dot(q[r], kk, 0.f)) : 0.f;
      }
    }
#pragma unroll
    for (int r = 0; r < RL; ++r) {
      if (r >= nr) continue;
      float mx = kNegInf;
#pragma unroll
      for (int sp = 0; sp < SPMAX; ++sp) {
        if (sp < nsteps) {
          const float v = visible(r, tile * G::TT + w * TPW + sp * TPI + tg) ? s[sp][r] * p.scale_log2 : kNegInf;
          s[sp][r] = v;
          mx = fmaxf(mx, v);
        }
      }
      const float mnew = fmaxf(m[r], mx);
      const float muse = mnew == kNegInf ? 0.f : mnew;
      const float alpha = fast_exp2(m[r] - muse);
      m[r] = mnew;
      l[r] *= alpha;
#pragma unroll
      for (int e = 0; e < E; ++e) o[r][e] *= alpha;
#pragma unroll
      for (int sp = 0; sp < SPMAX; ++sp) {
        if (sp < nsteps) {
          s[sp][r] = fast_exp2(s[sp][r] - muse);
          l[r] += s[sp][r];
        }
      }
    }
#pragma unroll
    for (int sp = 0; sp < SPMAX; ++sp) {
      if (sp < nsteps) {
        float vf[E];
        Elem<T>::unpack(vv[sp], vf);
#pragma unroll
        for (int r = 0; r < RL; ++r)
          if (r < nr)
#pragma unroll
            for (int e = 0; e < E; ++e) o[r][e] = fmaf(s[sp][r], vf[e], o[r][e]);
      }
    }
  };

  run_tiles<D, EB>(t, stb, tid, compute);

  // Merge the TPI token streams of this row split (lanes li, li + LPT, ...).
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
  __syncthreads();  // every wavefront is done with the tiles
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
  if (out_r < R) {
    const int r = out_r, c4 = out_c4;
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
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const float lse = lt > 0.f ? (mm + __log2f(lt)) * kLn2 : kNegInf;
    const float v4[4] = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
    write_partial(p, t, out_slot, out_head, D, c4 * 4, v4, lse, c4 == 0);
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kPacThreads) void pac_kernel(PacParams p) {
  const int bin = blockIdx.x % p.num_bins;
  const int kvh = blockIdx.x / p.num_bins;
  const int tb = p.bin_ptr[bin], te = p.bin_ptr[bin + 1];
  const int64_t esz = sizeof(T);
  // The next piece's record travels one dword per lane (lanes 0..11 of every
  // wavefront) while the current piece runs, and is handed over through LDS.
  constexpr int TW = sizeof(DevTask) / 4;
  uint32_t* const task_lds = reinterpret_cast<uint32_t*>(pac_lds + kTileBytes + kAuxBytes - sizeof(DevTask));
  const int tid = threadIdx.x;
  if (tb < te && tid < TW) task_lds[tid] = reinterpret_cast<const uint32_t*>(p.tasks + tb)[tid];
  __syncthreads();
  for (int ti = tb; ti < te; ++ti) {
    DevTask task;
    __builtin_memcpy(&task, task_lds, sizeof(DevTask));
    uint32_t next_word = 0;
    if (ti + 1 < te && (tid & 63) < TW) next_word = reinterpret_cast<const uint32_t*>(p.tasks + ti + 1)[tid & 63];
    TaskInfo t;
    t.piece = task.piece;
    t.kv_begin = task.kv_begin;
    t.kv_len = task.kv_len;
    t.row_begin = task.row_begin;
    t.row_count = task.row_count;
    t.e0 = task.e0;
    t.masked = (task.flags & kDevMasked) != 0;
    const int64_t off = (kvh * p.stride_head + task.tok0 * p.stride_token) * esz;
    t.kbase = static_cast<const char*>(p.k) + off;
    t.vbase = static_cast<const char*>(p.v) + off;
    bool done = false;
    if constexpr (sizeof(T) == 2) {
      if (t.row_count >= p.mfma_min_rows) {
        mfma_piece<D>(p, t, kvh);
        done = true;
      }
    }
    if (!done) dot_piece<T, D>(p, t, kvh);
    __syncthreads();  // the piece is finished with the LDS (and with task_lds)
    if (tid < TW) task_lds[tid] = next_word;
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
  hipLaunchKernelGGL((pac_kernel<T, D>), dim3(grid), dim3(kPacThreads), kLdsBytes, static_cast<hipStream_t>(stream),
                     p);
  return static_cast<int>(hipGetLastError());
}

}  // namespace

size_t pac_lds_bytes() { return kLdsBytes; }

int launch_pac(const PacParams& p, int in_dtype, int head_dim, void* stream) {
  if (in_dtype == PST_BF16)
    return head_dim == 128 ? launch_one<uint16_t, 128>(p, stream) : launch_one<uint16_t, 64>(p, stream);
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
