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
// 16 KB half-tiles (64 tokens at d = 128 bf16) by direct HBM->LDS DMA
// (buffer_load_dwordx4 ... lds), four stages deep, so three tiles are in
// flight while one is computed and no registers hold staged data.  Rows are
// XOR-swizzled by 16-byte chunk so the reads below spread over the banks;
// loads past the piece end return zeros.  Paged K/V (a node as a list of
// pages of a paged pool) is a separate instantiation: each DMA block finds
// its page through the page table (one scalar read per page run).  So are
// flattened chunks (DEFT: Decoding with Flash Tree-Attention, section 3.3
// and appendix A.9: the depth-first tree KV cut into equal chunks that may
// span nodes): each token's pool row comes from the plan's row table, and
// every tile takes the test of the chunk's bit causal masks, which arrive
// in LDS with the queries.
//
// Two compute paths, chosen per piece:
//  * matrix cores (every bf16 piece by default): each wavefront owns 16 or 32
//    rows and half or all of each tile's tokens and computes S^T = K Q^T
//    (v_mfma_f32_16x16x32_bf16) and O^T += V^T P^T (v_mfma_f32_16x16x32_f16),
//    so every row's softmax state stays in one lane.  V^T fragments come
//    straight from the row-major tile with the LDS transpose read
//    ds_read_b64_tr_b16.  The product O += P V of a tile runs one tile late,
//    next to the next tile's softmax; for it each V tile is converted once in
//    LDS to fp16, scaled by a power of two chosen per piece from the data,
//    and P is rounded to fp16.  Layouts with two wavefronts per slab (up to
//    128 rows, bandwidth-bound) update the row maxima branch-free; one slab
//    per wavefront (more rows, compute-bound) tests the lazy maximum per lane;
//  * wavefront dot products (float32, or bf16 pieces below 16 rows on
//    request): groups of head_dim*elem/16 lanes take one token each, reduce
//    q.k across the group with DPP, and keep a running (max, sum, O) per row;
//    states are merged across lane groups and wavefronts at the end.
// Both use the streaming softmax of CoDec section KV缓存管理 (per-block
// maximum, rescale of the running sum and numerator at the common maximum)
// in base 2, and emit the normalised partial O and its natural-log LSE: in
// float32, or, for bf16 output, in fp16 scaled by the piece's power of two
// with the exponent beside the LSE.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "pst_internal.h"

namespace pst {
namespace {

typedef short bf16x8 __attribute__((ext_vector_type(8)));
typedef short bf16x4s __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2n __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

// Wavefronts per workgroup: two per SIMD, so that one wavefront's matrix-core
// work overlaps the other's vector work.
template <typename T>
constexpr int kWaves = 8;
constexpr int NSTAGE = 4;             // LDS tile stages
constexpr int TILE_BYTES = 16384;     // bytes of one K (or V) tile
constexpr int STAGE_BYTES = 2 * TILE_BYTES;
constexpr float kLn2 = 0.69314718055994531f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kLazy = 8.0f;  // log2 headroom before the reference maximum is raised
constexpr size_t kTileBytes = static_cast<size_t>(NSTAGE) * STAGE_BYTES;  // 128 KB of tile stages
// The aggregated queries of a matrix-core piece (up to 256 rows x 256 B)
// arrive in the V half of stage 2, stage 3 and 16 KB after the stages: the
// tile schedule refills none of them before the queries are in registers.
constexpr size_t kQOff = 2 * STAGE_BYTES + TILE_BYTES;
constexpr size_t kAuxOff = kQOff + 64 * 1024;
constexpr size_t kAuxBytes = 8 * 1024;  // softmax states exchanged between wavefronts; next task record
// After the first 4 KB of the aux area (the softmax-state exchange uses at
// most 4 KB): the largest |V| each wavefront converted in a piece.
constexpr size_t kVexpOff = kAuxOff + 4096;
constexpr size_t kLdsBytes = kAuxOff + kAuxBytes;
// Flattened chunks add their bit causal masks (up to kMaskWordsMax words per
// task) after the rest.
constexpr size_t kMaskOff = kLdsBytes;
constexpr size_t kMaskBytes = kMaskWordsMax * 8;
constexpr size_t kLdsBytesFlat = kMaskOff + kMaskBytes;
static_assert(kTileBytes >= 64 * 1024, "merge scratch reuses the tile stages");
static_assert(kLdsBytesFlat <= 160 * 1024, "one workgroup per compute unit");

// K/V layouts, one kernel instantiation each: contiguous node runs, paged
// nodes, flattened chunks (every token addressed through the plan's row table).
constexpr int kContig = 0, kPaged = 1, kFlat = 2;

// The workgroup's LDS (dynamic size kLdsBytes), visible to every path as LDS.
extern __shared__ __attribute__((aligned(16))) char pac_lds[];

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2n));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
// max(a, b, c).  Plain fmaxf: this file is compiled with IEEE mode off, so
// no quieting moves precede it and the compiler fuses pairs into v_max3.
// (Inline assembly must not be used here: the compiler inserts no wait
// states between a matrix-core result and an assembly statement reading it.)
__device__ __forceinline__ float max3(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Raw buffer over [base, base + bytes): loads past the end return zeros, so
// the ragged tail of a piece needs no branch.  Rebased per tile so the 32-bit
// offsets stay small whatever the pool size.
constexpr int kBufferWord3 = 0x00020000;  // raw 32-bit data format for gfx9-family buffer descriptors
// Callers pass wave-uniform values; they are re-read as such so that the
// descriptor lives in scalar registers (the DMA takes it as an SGPR operand).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const char* base, int64_t bytes) {
  const int n = __builtin_amdgcn_readfirstlane(bytes > 0x7fffffff ? 0x7fffffff : static_cast<int>(bytes < 0 ? 0 : bytes));
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t u = static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a)))) |
                     (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32)))) << 32);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<char*>(u), static_cast<short>(0), n, kBufferWord3);
}
// The same for a byte count already known to lie in [0, 2^31).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_n(const char* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t u = static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a)))) |
                     (static_cast<uint64_t>(static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(a >> 32)))) << 32);
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<char*>(u), static_cast<short>(0),
                                           __builtin_amdgcn_readfirstlane(static_cast<int>(bytes)), kBufferWord3);
}

// One 16-byte-per-lane HBM->LDS DMA: LDS destination = lds_addr + 16 * lane.
// Written as inline assembly so the compiler does not see an LDS store in
// flight: it would otherwise wait for every outstanding DMA before each LDS
// read.  The tile loop waits explicitly (wait_vmem) for the tile it reads.
// M0 carries the destination and is restored afterwards.  NT: the load
// carries the non-temporal hint (K/V read by one task only: streamed past
// the caches instead of displacing lines that are still to be read).
template <bool NT = false>
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int voff, uint32_t lds_addr) {
  uint32_t saved;
  if constexpr (NT)
    asm volatile(
        "s_mov_b32 %0, m0\n\t"
        "s_mov_b32 m0, %3\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, 0 offen nt lds\n\t"
        "s_nop 0\n\t"
        "s_mov_b32 m0, %0"
        : "=&s"(saved)
        : "v"(voff), "s"(r), "s"(__builtin_amdgcn_readfirstlane(lds_addr))
        : "memory");
  else
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
// threadIdx.x through an opaque move: values derived from it inside a piece
// are recomputed per piece instead of being hoisted out of the piece loop and
// held in registers across every piece.
__device__ __forceinline__ int piece_tid() {
  int t;
  asm volatile("v_mov_b32 %0, %1" : "=v"(t) : "v"(static_cast<int>(__builtin_amdgcn_workitem_id_x())));
  return t;
}
// LDS address of a generic pointer into the LDS: a flat address in the
// shared aperture holds the aperture base in its upper 32 bits and the LDS
// address in its lower 32, so truncation gives it.  (A cast to the LDS
// address space would test the pointer for null on every DMA.)
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(p));
}

// Wait until at most n (0..16) of this wavefront's vector memory operations
// are outstanding; expcnt and lgkmcnt are left alone (vmcnt: bits 3:0 and
// 15:14 of the s_waitcnt immediate).
#define PST_VMCNT(n) (0x0F70 | ((n) & 15) | (((n) >> 4) << 14))
__device__ __forceinline__ void wait_vmem_n(int n) {
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(PST_VMCNT(0)); break;
    case 1: __builtin_amdgcn_s_waitcnt(PST_VMCNT(1)); break;
    case 2: __builtin_amdgcn_s_waitcnt(PST_VMCNT(2)); break;
    case 3: __builtin_amdgcn_s_waitcnt(PST_VMCNT(3)); break;
    case 4: __builtin_amdgcn_s_waitcnt(PST_VMCNT(4)); break;
    case 5: __builtin_amdgcn_s_waitcnt(PST_VMCNT(5)); break;
    case 6: __builtin_amdgcn_s_waitcnt(PST_VMCNT(6)); break;
    case 7: __builtin_amdgcn_s_waitcnt(PST_VMCNT(7)); break;
    case 8: __builtin_amdgcn_s_waitcnt(PST_VMCNT(8)); break;
    case 9: __builtin_amdgcn_s_waitcnt(PST_VMCNT(9)); break;
    case 10: __builtin_amdgcn_s_waitcnt(PST_VMCNT(10)); break;
    case 11: __builtin_amdgcn_s_waitcnt(PST_VMCNT(11)); break;
    case 12: __builtin_amdgcn_s_waitcnt(PST_VMCNT(12)); break;
    case 13: __builtin_amdgcn_s_waitcnt(PST_VMCNT(13)); break;
    case 14: __builtin_amdgcn_s_waitcnt(PST_VMCNT(14)); break;
    case 15: __builtin_amdgcn_s_waitcnt(PST_VMCNT(15)); break;
    default: __builtin_amdgcn_s_waitcnt(PST_VMCNT(16)); break;
  }
}
#undef PST_VMCNT
__device__ __forceinline__ void wait_lds_all() { __builtin_amdgcn_s_waitcnt(0xC07F); }  // lgkmcnt(0)

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
  int piece, kv_begin, kv_len, row_begin, row_count, e0, masked, node;
  int flat0;          // flattened chunk: its first token in the row table
  int linear;         // flattened chunk over consecutive pool rows: addressed like a contiguous run
  int shared;         // other tasks (row groups, query-guided groups) read the same K/V tokens
  int pg0;            // paged: the node's first entry in the page table
  const char* kbase;  // K of this kv head at the piece's first token (paged: at the pool's first row)
  const char* vbase;
};

// Paged K/V.  Nodes start on a page, pieces at multiples of 64 tokens of
// their node and pages hold a power of two >= 8 tokens, so a 1 KB block
// (TPB <= 8 tokens) never crosses a page.  A half-tile is fetched one of
// three ways, the first that applies (wave-uniform, fixed per piece):
//   whole tiles  pages hold whole tiles and the piece starts on a tile: one
//                page per tile, blocks round-robin over the wavefronts;
//   runs         each wavefront takes KB consecutive blocks on one page;
//   blocks       (8-token pages under 8-token blocks) every block its own page.
// Each way builds as few buffer descriptors as it can, with scalar
// arithmetic, from the rows they start at; the lanes' offsets inside them
// are the same in every tile.
template <int TT>
__device__ __forceinline__ bool paged_whole_tiles(const PacParams& p, const TaskInfo& t) {
  return (1 << p.page_shift) >= TT && (t.kv_begin & (TT - 1)) == 0;
}
// Page of the token ft tokens into the piece (for a token past the piece's
// end, a page of the node: such blocks read nothing).
__device__ __forceinline__ int page_of(const PacParams& p, const TaskInfo& t, int ft) {
  const auto* idx = (const __attribute__((address_space(4))) int32_t*)(p.page_idx);
  return idx[t.pg0 + ((t.kv_begin + (ft < t.kv_len ? ft : 0)) >> p.page_shift)];
}
// Byte offset, from the kv head's first row, of the token ft tokens into the
// piece, which lies on page `page`.  32-bit row and stride: the library
// limits a paged pool to 2^31 - 1 rows and the token stride to 16 MB.
__device__ __forceinline__ uint64_t paged_off(const PacParams& p, const TaskInfo& t, int64_t stb, int ft, int page) {
  const uint32_t row = (static_cast<uint32_t>(page) << p.page_shift) |
                       (static_cast<uint32_t>(t.kv_begin + ft) & ((1u << p.page_shift) - 1u));
  return static_cast<uint64_t>(row) * static_cast<uint32_t>(stb);
}
// Offset of lane `lane`'s chunk of block b inside a descriptor that starts
// `lead` tokens before the block: token lane / CPT of the block, chunk
// (lane % CPT) ^ (token % CPT), the token counted from the tile's start (the
// swizzle of the LDS tile).
template <int CPT, int TPB>
__device__ __forceinline__ int block_voff(int b, int lead, int lane, int64_t stb) {
  const int lt = lane / CPT, phys = lane % CPT;
  return static_cast<int>((lead + lt) * stb) + ((phys ^ ((b * TPB + lt) & (CPT - 1))) << 4);
}
// The page numbers a wavefront's share of a paged half-tile needs: the
// tile's page (whole tiles), its run's page (runs), or its two blocks' pages.
// Scalar reads; K and V of a tile take the same.
struct PgPre {
  int a, b;
};
template <int D, int EB, int NW>
__device__ __forceinline__ PgPre pg_fetch(const PacParams& p, const TaskInfo& t, int tile, int w) {
  using G = Geo<D, EB>;
  constexpr int TPB = 64 / G::CPT, KB = TILE_BYTES / 1024 / NW;
  if (p.page_shift < 0) return PgPre{0, 0};
  const int tok_base = tile * G::TT;
  if (paged_whole_tiles<G::TT>(p, t)) {
    const int a = page_of(p, t, tok_base);
    return PgPre{a, a};
  }
  const int ft = tok_base + KB * w * TPB;
  const int a = page_of(p, t, ft);
  return PgPre{a, (1 << p.page_shift) >= KB * TPB ? a : page_of(p, t, ft + TPB)};
}
// The DMA operations of this wavefront for a paged half-tile: emit(off,
// bytes, voff, b) per operation, for block b, with a descriptor from byte
// `off` of the kv head over `bytes` bytes and the lane's offset voff in it.
template <int D, int EB, int NW, typename Emit>
__device__ __forceinline__ void paged_half(const PacParams& p, const TaskInfo& t, int64_t stb, int tile, int lane,
                                           int w, const PgPre& pg, Emit&& emit) {
  using G = Geo<D, EB>;
  constexpr int TPB = 64 / G::CPT, KB = TILE_BYTES / 1024 / NW;
  const int tok_base = tile * G::TT;
  if (paged_whole_tiles<G::TT>(p, t)) {
    const uint64_t off = paged_off(p, t, stb, tok_base, pg.a);
    const uint32_t bytes = static_cast<uint32_t>(min(G::TT, t.kv_len - tok_base)) * static_cast<uint32_t>(stb);
#pragma unroll
    for (int c = 0; c < KB; ++c) {
      const int b = c * NW + w;
      emit(off, bytes, block_voff<G::CPT, TPB>(b, b * TPB, lane, stb), b);
    }
    return;
  }
  const int ft = tok_base + KB * w * TPB;  // the wavefront's first token
  if ((1 << p.page_shift) >= KB * TPB) {
    const uint64_t off = paged_off(p, t, stb, ft, pg.a);
    const uint32_t bytes = static_cast<uint32_t>(min(max(t.kv_len - ft, 0), KB * TPB)) * static_cast<uint32_t>(stb);
#pragma unroll
    for (int c = 0; c < KB; ++c) emit(off, bytes, block_voff<G::CPT, TPB>(KB * w + c, c * TPB, lane, stb), KB * w + c);
    return;
  }
#pragma unroll
  for (int c = 0; c < KB; ++c) {
    const int fb = ft + c * TPB;
    const uint64_t off = paged_off(p, t, stb, fb, c == 0 ? pg.a : pg.b);
    const uint32_t bytes = static_cast<uint32_t>(min(max(t.kv_len - fb, 0), TPB)) * static_cast<uint32_t>(stb);
    emit(off, bytes, block_voff<G::CPT, TPB>(KB * w + c, 0, lane, stb), KB * w + c);
  }
}

// Row r of the task -> (query entry, q-head); returns false past the task's rows.
__device__ __forceinline__ bool row_target(const PacParams& p, const TaskInfo& t, int kvh, int r, int* entry,
                                           int* head) {
  if (r >= t.row_count) return false;
  const int rr = t.row_begin + r;
  *entry = t.e0 + rr / p.g;
  *head = kvh * p.g + rr % p.g;
  return true;
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b);
// `slot` = first partial slot of the row's (query, node) entry (prefetched);
// the piece's slot is slot + piece.  float32 partials: vals4 is the partial
// output.  fp16 partials (part_f16): vals4 is the partial output times
// 2^(15 - ev), below 2^16 in magnitude, rounded to nearest fp16; ev goes
// beside the LSE (one 8-byte pair).
__device__ __forceinline__ void write_partial(const PacParams& p, const TaskInfo& t, int slot0, int head, int D,
                                              int d0, const float* vals4, float lse, bool write_lse, int ev) {
  const int64_t slot = static_cast<int64_t>(slot0) + t.piece;
  const int64_t at = (slot * p.hq + head) * D + d0;
  if (p.part_f16) {
    *reinterpret_cast<uint2*>(reinterpret_cast<_Float16*>(p.opart) + at) =
        make_uint2(pack_f16(vals4[0], vals4[1]), pack_f16(vals4[2], vals4[3]));
    if (write_lse) reinterpret_cast<float2*>(p.lsepart)[slot * p.hq + head] = make_float2(lse, __int_as_float(ev));
  } else {
    *reinterpret_cast<float4*>(p.opart + at) = make_float4(vals4[0], vals4[1], vals4[2], vals4[3]);
    if (write_lse) p.lsepart[slot * p.hq + head] = lse;
  }
}

// Flattened chunk: pool rows of N consecutive tokens from token `tok` of the
// task (row table entries; wave-uniform, so scalar reads).
template <int N>
__device__ __forceinline__ void flat_rows_of(const PacParams& p, const TaskInfo& t, int tok, int* rw) {
  const auto* fr = (const __attribute__((address_space(4))) int32_t*)(p.flat_rows) + t.flat0 + tok;
#pragma unroll
  for (int k = 0; k < N; ++k) rw[k] = fr[k];
}
// Buffer offset of lane `lane`'s chunk of 1 KB block b: token b TPB +
// lane / CPT at pool row rw[lane / CPT] (an offset past the descriptor for
// the -1 rows past the chunk's end, which then read zeros).
template <int CPT, int TPB>
__device__ __forceinline__ int flat_voff(const int* rw, int b, int lane, int64_t stb) {
  const int P = b * 64 + lane;
  const int tok = P / CPT, phys = P % CPT, j = lane / CPT;
  int row = rw[0];
#pragma unroll
  for (int k = 1; k < TPB; ++k) row = j == k ? rw[k] : row;
  const uint32_t off = static_cast<uint32_t>(static_cast<int64_t>(row) * stb) + ((phys ^ (tok & (CPT - 1))) << 4);
  return static_cast<int>(row >= 0 ? off : 0x80000000u);
}

// Flattened chunk: the task's bit causal masks (mask_words words for each of
// its entries, in entry order) into the mask area of LDS, one 1 KB DMA block
// per wavefront at most.  Issued before the task's K/V, so the first tile's
// wait covers it.
template <int NW>
__device__ __forceinline__ void issue_masks(const PacParams& p, const TaskInfo& t, int tid) {
  static_assert(NW * 1024 >= kMaskBytes, "one block per wavefront holds the masks");
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int e_first = t.e0 + t.row_begin / p.g;
  const int bytes = (t.row_count / p.g) * p.mask_words * 8;
  const __amdgpu_buffer_rsrc_t r =
      make_rsrc(reinterpret_cast<const char*>(p.nq_mask + static_cast<int64_t>(e_first) * p.mask_words), bytes);
  if (w * 1024 < bytes) dma16(r, w * 1024 + lane * 16, lds_addr(pac_lds + kMaskOff + w * 1024));
}
__device__ __forceinline__ uint64_t flat_mask(const PacParams& p, int entry, int word) {
  return reinterpret_cast<const uint64_t*>(pac_lds + kMaskOff)[entry * p.mask_words + word];
}

// DMA of tile `tile` of the piece into stage `stage`: the 16 1 KB blocks of
// K and of V are spread over the NW wavefronts; lane L of a block fills
// 16-byte chunk position P = block*64 + L, i.e. token P / CPT, chunk
// (P % CPT) ^ (token % CPT).
template <int NW>
constexpr int kHalfOps = TILE_BYTES / 1024 / NW;  // DMA operations per thread for one K (or V) tile
template <int D, int EB, int NW>
__device__ __forceinline__ void issue_tile(const PacParams& p, const TaskInfo& t, int64_t stb, int tile, int stage,
                                           int tid) {
  using G = Geo<D, EB>;
  constexpr int TPB = 64 / G::CPT;  // tokens per 1 KB block
  const int tok_base = tile * G::TT;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  char* st = pac_lds + stage * STAGE_BYTES;
  constexpr int KB = kHalfOps<NW>;
  if (p.mask_words > 0 && !t.linear) {
    // Flattened chunk: the rows of this wavefront's consecutive blocks come
    // from the row table (scalar reads); K and V share them.
    int rw[KB * TPB];
    flat_rows_of<KB * TPB>(p, t, tok_base + KB * w * TPB, rw);
    const __amdgpu_buffer_rsrc_t rk = make_rsrc(t.kbase, p.pool_bytes);
    const __amdgpu_buffer_rsrc_t rv = make_rsrc(t.vbase, p.pool_bytes);
#pragma unroll
    for (int c = 0; c < KB; ++c) {
      const int b = KB * w + c;
      const int voff = flat_voff<G::CPT, TPB>(rw + c * TPB, b, lane, stb);
      dma16(rk, voff, lds_addr(st + b * 1024));
      dma16(rv, voff, lds_addr(st + TILE_BYTES + b * 1024));
    }
    return;
  }
  if (p.page_shift >= 0) {
    // Paged: K and V of a block sit at the same rows.
    const PgPre pg = pg_fetch<D, EB, NW>(p, t, tile, w);
    paged_half<D, EB, NW>(p, t, stb, tile, lane, w, pg, [&](uint64_t off, uint32_t bytes, int voff, int b) {
      dma16(make_rsrc_n(t.kbase + off, bytes), voff, lds_addr(st + b * 1024));
      dma16(make_rsrc_n(t.vbase + off, bytes), voff, lds_addr(st + TILE_BYTES + b * 1024));
    });
    return;
  }
  const uint64_t toff = static_cast<uint64_t>(static_cast<uint32_t>(tok_base)) * static_cast<uint32_t>(stb);
  const uint32_t bytes = static_cast<uint32_t>(min(G::TT, t.kv_len - tok_base)) * static_cast<uint32_t>(stb);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc_n(t.kbase + toff, bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc_n(t.vbase + toff, bytes);
#pragma unroll
  for (int c = 0; c < kHalfOps<NW>; ++c) {
    const int b = c * NW + w;
    const int P = b * 64 + lane;
    const int tok = P / G::CPT, phys = P % G::CPT;
    const int voff = static_cast<int>(tok * stb) + ((phys ^ (tok & (G::CPT - 1))) << 4);
    dma16(rk, voff, lds_addr(st + b * 1024));
    dma16(rv, voff, lds_addr(st + TILE_BYTES + b * 1024));
  }
}

// Tiles 0 .. NSTAGE-2 (issued before the queries are gathered).
template <int D, int EB, int NW>
__device__ __forceinline__ void issue_prologue(const PacParams& p, const TaskInfo& t, int64_t stb, int tid) {
  using G = Geo<D, EB>;
  const int ntiles = (t.kv_len + G::TT - 1) / G::TT;
#pragma unroll
  for (int i = 0; i < NSTAGE - 1; ++i)
    if (i < ntiles) issue_tile<D, EB, NW>(p, t, stb, i, i, tid);
}

// The tile loop: wait for tile i (2 kHalfOps DMA operations per thread and tile), a
// barrier without a memory fence (which would drain every DMA in flight),
// refill the stage of tile i-1 with tile i+3, compute tile i.
template <int D, int EB, int NW, typename F>
__device__ __forceinline__ void run_tiles(const PacParams& p, const TaskInfo& t, int64_t stb, int tid, F&& compute) {
  using G = Geo<D, EB>;
  const int ntiles = (t.kv_len + G::TT - 1) / G::TT;
  for (int tile = 0; tile < ntiles; ++tile) {
    wait_vmem_n(2 * kHalfOps<NW> * min(NSTAGE - 2, ntiles - 1 - tile));
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS access moves above the barrier
    if (tile + NSTAGE - 1 < ntiles) issue_tile<D, EB, NW>(p, t, stb, tile + NSTAGE - 1, (tile + NSTAGE - 1) % NSTAGE, tid);
    compute(pac_lds + (tile % NSTAGE) * STAGE_BYTES, tile);
  }
}

// ---------------------------------------------------------------------------
// Matrix-core path (bf16)
// ---------------------------------------------------------------------------
// O^T += V^T P^T runs in fp16: P <= 2^kLazy is rounded to nearest fp16
// (2^-11 relative per weight, four times finer than bf16) and the row sums
// add the same rounded P.  Each V tile is converted once in LDS, by all
// threads together, from bf16 to fp16 times 2^(15 - ev), with one exponent ev
// per piece.  The piece is right for ev when its largest |v| has exponent E
// in [ev - kEvWindow, ev]: then every |v| < 2^(ev + 1) lands below 2^16 (no
// saturation), the largest lands at or above 2^(15 - kEvWindow), and bf16
// values (8 significant bits) convert exactly down to 2^(ev - 29), keep 8
// bits down to 2^(ev - 32) and below that carry an absolute error under
// 2^(ev - 39) (round toward zero into fp16 subnormals): at least 2^26 below
// the piece's largest |v| keeps bf16 precision.  Each lane keeps the largest
// |v| it converts; at the piece's end the workgroup takes their maximum, and
// if E fell outside the window the piece is computed once more with ev = E,
// which fits by construction.  The next piece of the workgroup starts from
// the last ev (plus headroom after a repeat), so a repeat happens only when
// the V scale moves by more than the window between pieces.  The output takes
// 2^(ev - 15) back when it is normalised.
constexpr int kEvStart = 3;     // the first piece of a workgroup: |v| below 16
constexpr int kEvWindow = 6;    // accepted E in [ev - kEvWindow, ev]
constexpr int kEvMin = -100;    // ev never goes lower (nor is a piece of smaller |v| repeated for it)
constexpr int kEvMax = 127;

__device__ __forceinline__ float exp2i(int e) {  // 2^e for integer e in [-126, 127]
  return __uint_as_float(static_cast<uint32_t>(e + 127) << 23);
}

__device__ __forceinline__ uint32_t pack_f16(float a, float b) {
  const f32x2 x = {a, b};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
}

__device__ __forceinline__ char* kslot(int j) { return pac_lds + (j % NSTAGE) * STAGE_BYTES; }
__device__ __forceinline__ char* vslot(int j) { return pac_lds + (j % NSTAGE) * STAGE_BYTES + TILE_BYTES; }

// Which 1 KB blocks of a K or V half a wavefront's DMA fills: runs of
// kHalfOps consecutive blocks per wavefront when blocks find their own rows
// (flattened chunks; paged tiles that may cross a page), else round-robin
// over the wavefronts.  Wave-uniform.
template <int D>
__device__ __forceinline__ bool half_in_runs(const PacParams& p, const TaskInfo& t) {
  using G = Geo<D, 2>;
  return (p.mask_words > 0 && !t.linear) || (p.page_shift >= 0 && !paged_whole_tiles<G::TT>(p, t));
}

// DMA of the K (or V) half of tile `tile` (16 KB) into `dst`: every wavefront
// writes kHalfOps 1 KB blocks; lane L of block b fills chunk position
// P = 64 b + L, i.e. token P / CPT, chunk (P % CPT) ^ (token % CPT).  `pg`:
// the tile's page numbers (paged pieces; see pg_fetch).
template <int D, int NW, bool NT>
__device__ __forceinline__ void issue_half(const PacParams& p, const TaskInfo& t, const char* base, int64_t stb,
                                           int tile, char* dst, int tid, const PgPre& pg) {
  using G = Geo<D, 2>;
  constexpr int TPB = 64 / G::CPT;  // tokens per 1 KB block
  const int tok_base = tile * G::TT;
  const int lane = tid & 63, w = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (p.mask_words > 0 && !t.linear) {
    // Flattened chunk: this wavefront takes the consecutive blocks kHalfOps w
    // .. kHalfOps w + kHalfOps - 1; their tokens' rows come from the row table.
    constexpr int KB = kHalfOps<NW>;
    int rw[KB * TPB];
    flat_rows_of<KB * TPB>(p, t, tok_base + KB * w * TPB, rw);
    const __amdgpu_buffer_rsrc_t r = make_rsrc(base, p.pool_bytes);
#pragma unroll
    for (int c = 0; c < KB; ++c) {
      const int b = KB * w + c;
      dma16<NT>(r, flat_voff<G::CPT, TPB>(rw + c * TPB, b, lane, stb), lds_addr(dst + b * 1024));
    }
    return;
  }
  if (p.page_shift >= 0) {
    paged_half<D, 2, NW>(p, t, stb, tile, lane, w, pg, [&](uint64_t off, uint32_t bytes, int voff, int b) {
      dma16<NT>(make_rsrc_n(base + off, bytes), voff, lds_addr(dst + b * 1024));
    });
    return;
  }
  // (tile < nt: at least one token; the library limits the token stride to
  // 16 MB, so a tile's bytes fit 31 bits.)
  const char* tbase = base + static_cast<uint64_t>(static_cast<uint32_t>(tok_base)) * static_cast<uint32_t>(stb);
  const uint32_t bytes = static_cast<uint32_t>(min(G::TT, t.kv_len - tok_base)) * static_cast<uint32_t>(stb);
  const __amdgpu_buffer_rsrc_t r = make_rsrc_n(tbase, bytes);
#pragma unroll
  for (int c = 0; c < kHalfOps<NW>; ++c) {
    const int b = c * NW + w;
    const int P = b * 64 + lane;
    const int tok = P / G::CPT, phys = P % G::CPT;
    dma16<NT>(r, static_cast<int>(tok * stb) + ((phys ^ (tok & (G::CPT - 1))) << 4), lds_addr(dst + b * 1024));
  }
}

// DMA schedule of a piece of nt tiles: group j holds K of tile j (j < nt)
// and V of tile j - 1 (1 <= j <= nt), kHalfOps operations per thread each.
// Iteration i of the tile loop consumes group i (QK of tile i, PV of tile
// i - 1) and issues group i + 3, so three groups stay in flight; K of tile
// i + 3 refills the K half of tile i - 1 and V of tile i + 2 the V half of
// tile i - 2, both finished before iteration i's barrier.
template <int NW>
__device__ __forceinline__ int group_ops(int j, int nt) {
  return (j < nt ? kHalfOps<NW> : 0) + (j >= 1 && j <= nt ? kHalfOps<NW> : 0);
}


// Each wavefront owns RBR blocks of 16 rows of a slab; TS wavefronts share a
// slab, each taking TT/TS tokens of every tile in NSUB = TT/(32 TS) sub-steps
// of 32 tokens (a tile is 64 tokens at d = 128, 128 at d = 64).  The
// sub-steps are software-pipelined: step k computes S = K Q^T and the
// softmax of step k while the matrix cores run O += P V of step k - 1, so
// matrix-core and vector work overlap inside a wavefront.
// Returns false when the piece's V did not fit the scale it started from
// (ev_carry then holds the scale to run it again with, `retry` true).
template <int D, int RBR, int TS, int NW, bool NT>
__device__ __forceinline__ bool mfma_piece(const PacParams& p, const TaskInfo& t, int kvh, int& ev_carry, bool retry) {
  using G = Geo<D, 2>;
  constexpr int KS = D / 32;  // k-steps of S^T = K Q^T
  constexpr int DB = D / 16;  // d-blocks of O^T
  constexpr int NSUB = G::TT / (32 * TS);  // 32-token sub-steps per wavefront and tile
  constexpr int ROWS_W = 16 * RBR;
  constexpr bool kSpread = TS == 1;  // refills issued inside the steps (see `step`)
  constexpr int QOPS = kMaxRows * G::CPT / 64 / NW;  // Q DMA operations per thread at most
  char* const lds = pac_lds;
  const int tid = piece_tid();
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int l16 = lane & 15, lg = lane >> 4;
  const int R = t.row_count;
  const int slabs = (R + ROWS_W - 1) / ROWS_W;
  const int slab = w / TS, half = w % TS;
  const bool active = slab < slabs;
  const int tok0 = half * (G::TT / TS);
  const int64_t stb = p.stride_token * 2;
  const int nt = (t.kv_len + G::TT - 1) / G::TT;
  const float c2 = p.scale_log2;
  char* const qarea = lds + kQOff;

  // Gather offsets of the Q chunks this thread moves (rows past R read out
  // of range: zeros), and the slot, head and mask of the rows this lane owns.
  const int qops_total = (R * G::CPT + 63) / 64;
  uint32_t qoff[QOPS];
#pragma unroll
  for (int o = 0; o < QOPS; ++o) {
    const int P = (o * NW + w) * 64 + lane;
    const int row = P / G::CPT, phys = P % G::CPT;
    int entry = t.e0 + t.row_begin / p.g, head = kvh * p.g + t.row_begin % p.g;
    const bool ok = row_target(p, t, kvh, row, &entry, &head);
    const uint32_t qrow = static_cast<uint32_t>(p.nq_idx[entry] * p.hq + head);
    qoff[o] = ok ? qrow * G::ROWB + ((phys ^ (row & (G::CPT - 1))) << 4) : 0x80000000u;
  }
  bool qok[RBR];
  int slot0[RBR], qhead[RBR];
  uint64_t rmask[RBR];
#pragma unroll
  for (int rb = 0; rb < RBR; ++rb) {
    int entry = t.e0 + t.row_begin / p.g, head = kvh * p.g + t.row_begin % p.g;
    qok[rb] = active && row_target(p, t, kvh, slab * ROWS_W + rb * 16 + l16, &entry, &head);
    slot0[rb] = p.entry_slot[entry];
    qhead[rb] = head;
    rmask[rb] = ~0ull;
    if (p.mask_words == 0 && t.masked && qok[rb]) rmask[rb] = p.nq_mask[entry];
  }
  // Flattened chunk: each row's entry among the task's (row groups hold
  // whole entries), which indexes its masks in LDS.
  int mrow[RBR] = {};
  if (p.mask_words > 0) {
#pragma unroll
    for (int rb = 0; rb < RBR; ++rb) mrow[rb] = qok[rb] ? (slab * ROWS_W + rb * 16 + l16) / p.g : 0;
  }

  // Queries first (needed first), then groups 0..2.
  {
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(static_cast<const char*>(p.q), p.q_bytes);
#pragma unroll
    for (int o = 0; o < QOPS; ++o)
      if (o * NW + w < qops_total) dma16(rq, static_cast<int>(qoff[o]), lds_addr(qarea + (o * NW + w) * 1024));
  }
  if (p.mask_words > 0) issue_masks<NW>(p, t, tid);
  // Paged pieces: the page numbers of the next K refill (pg_cur) and of the
  // next V refill (pg_prev, the K refill's of one iteration earlier), read
  // one refill ahead of their use.
  PgPre pg_prev, pg_cur;
  {
    const PgPre pg0 = pg_fetch<D, 2, NW>(p, t, 0, w), pg1 = pg_fetch<D, 2, NW>(p, t, 1, w);
    pg_prev = pg_fetch<D, 2, NW>(p, t, 2, w);
    if (0 < nt) issue_half<D, NW, NT>(p, t, t.kbase, stb, 0, kslot(0), tid, pg0);
    if (1 < nt) issue_half<D, NW, NT>(p, t, t.kbase, stb, 1, kslot(1), tid, pg1);
    if (0 < nt) issue_half<D, NW, NT>(p, t, t.vbase, stb, 0, vslot(0), tid, pg0);
    if (2 < nt) issue_half<D, NW, NT>(p, t, t.kbase, stb, 2, kslot(2), tid, pg_prev);
    if (1 < nt) issue_half<D, NW, NT>(p, t, t.vbase, stb, 1, vslot(1), tid, pg1);
    pg_cur = pg_fetch<D, 2, NW>(p, t, 3, w);
  }
  // The refills of one iteration: K of tile j and V of tile j - 1 (those
  // within the piece); then the pages move one tile on.
  auto refill_kv = [&](int j) {
    if (j < nt) issue_half<D, NW, NT>(p, t, t.kbase, stb, j, kslot(j), tid, pg_cur);
    if (j - 1 < nt) issue_half<D, NW, NT>(p, t, t.vbase, stb, j - 1, vslot(j - 1), tid, pg_prev);
    pg_prev = pg_cur;
    pg_cur = pg_fetch<D, 2, NW>(p, t, j + 1, w);
  };

  bf16x8 qf[RBR][KS];
  f32x4 o[DB][RBR];
  float m[RBR], l[RBR];
  float nm[RBR];   // -m, or 0 while m is -inf (the exponent offset of P)
  float thr[RBR];  // (m + kLazy) / c: raw scores above it raise the reference maximum
  bf16x8 pp[NSUB][RBR];  // fp16 P (bits) of each sub-step of the previous tile
  const float ic2 = 1.f / c2;
#pragma unroll
  for (int rb = 0; rb < RBR; ++rb) {
    m[rb] = kNegInf;
    l[rb] = 0.f;
    nm[rb] = 0.f;
    thr[rb] = kNegInf;
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) pp[sb][rb] = bf16x8{};
#pragma unroll
    for (int db = 0; db < DB; ++db) o[db][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // O^T += V^T P^T over the 32 tokens from `tp` of the (converted) V half `Vs`
  // with the fp16 P of sub-step `sb`.  A = V^T
  // rows d = 16 db + l16: two transpose reads, tokens tp + 4 lg + 0..3 and
  // tp + 16 + 4 lg + 0..3 (the k order of P); source lane s of each 16-lane
  // group points at token (t0 + s/4), channels 16 db + 4 (s%4) .. +3.
  auto pv = [&](const char* Vs, int tp, int sb) {
    const int ta = tp + 4 * lg + (l16 >> 2), tb2 = ta + 16;
    const int dq = 4 * (l16 & 3);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      const int c = (db * 16 + dq) >> 3, hoff = ((db * 16 + dq) & 7) * 2;
      const char* pa = Vs + ta * G::ROWB + ((c ^ (ta & (G::CPT - 1))) << 4) + hoff;
      const char* pb = Vs + tb2 * G::ROWB + ((c ^ (tb2 & (G::CPT - 1))) << 4) + hoff;
      const bf16x4s x0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) bf16x4s*)(pa));
      const bf16x4s x1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) bf16x4s*)(pb));
      const f16x8 a = __builtin_bit_cast(f16x8, __builtin_shufflevector(x0, x1, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
      for (int rb = 0; rb < RBR; ++rb)
        o[db][rb] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, __builtin_bit_cast(f16x8, pp[sb][rb]), o[db][rb], 0, 0, 0);
    }
  };

  // Raise row rb's reference maximum to this lane group's maximum mx (raw
  // score units) when it exceeds m + kLazy; *al = the factor that takes
  // values relative to the old reference to the new one.
  auto update_ref = [&](int rb, float mx, float* al) {
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));  // lanes i, i ^ 32
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(mx), __float_as_uint(mx), false, false);
    mx = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));  // and i ^ 16: the row
    const float mr = mx * c2;
    const float mnew = mr > m[rb] + kLazy ? mr : m[rb];
    *al = mnew == m[rb] ? 1.f : fast_exp2(m[rb] - mnew);  // 0 when m was -inf
    m[rb] = mnew;
    l[rb] *= *al;
    nm[rb] = mnew == kNegInf ? 0.f : -mnew;
    thr[rb] = mnew == kNegInf ? kNegInf : (mnew + kLazy) * ic2;
  };

  // One pipelined step, sub-step `sb` of tile `tile`: S for its 32 tokens
  // (K half `Ks`), O += P V of the same sub-step of the previous tile (whose
  // V was waited for and converted at this tile's start) with the P kept
  // from it, then the softmax of S into pp[sb].  The products of the
  // previous tile are independent of this step's softmax, so the matrix
  // cores run them while the vector ALU computes the new P.  With two
  // wavefronts per slab the reference-maximum update is branch-free
  // (cross-lane maximum by lane swaps), so all of it is one basic block; with
  // one slab per wavefront (compute-bound) a per-lane test skips the
  // cross-lane maximum in almost every step and the products follow it.
  // Only the rare rescale of O is a branch.  Tile 0 has no previous tile
  // (pv_tag false).  The order of the reads, products and vector work
  // inside a step is left to the compiler's scheduler: scheduling-group
  // hints (products first, or products interleaved with the vector work)
  // measured 5-8% slower on the 64- and 256-row layouts.
  auto step = [&](auto vis_tag, auto pv_tag, const char* Ks, int tile, int sb) {
    const int ts = tok0 + sb * 32;
    constexpr bool kVis = decltype(vis_tag)::value;  // tile needs the visibility test (partial or masked)
    constexpr bool kPrev = decltype(pv_tag)::value;  // a previous step exists
    f32x4 s[2][RBR];
#pragma unroll
    for (int hb = 0; hb < 2; ++hb) {
      const int tok = ts + hb * 16 + l16;
#pragma unroll
      for (int rb = 0; rb < RBR; ++rb) s[hb][rb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = ks * 4 + lg;
        const bf16x8 a = *reinterpret_cast<const bf16x8*>(Ks + tok * G::ROWB + ((c ^ (tok & (G::CPT - 1))) << 4));
#pragma unroll
        for (int rb = 0; rb < RBR; ++rb) s[hb][rb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qf[rb][ks], s[hb][rb], 0, 0, 0);
      }
    }
    if constexpr (kPrev) {
      // Compute-bound layout (TS = 1): this wavefront's share of the refills
      // of iteration `tile` (K of tile + 3 in the first sub-step, V of tile +
      // 2 in the last), issued here rather than all at once after the
      // barrier: a DMA instruction holds its wavefront for tens of cycles,
      // and eight wavefronts issuing together right after a barrier queue up
      // behind each other.  (Bandwidth-bound layouts refill at the barrier,
      // as early as possible.)
      if (kSpread && sb == 0 && tile + 3 < nt)
        issue_half<D, NW, NT>(p, t, t.kbase, stb, tile + 3, kslot(tile + 3), tid, pg_cur);
      if (kSpread && sb == NSUB - 1) {
        if (tile + 2 < nt) issue_half<D, NW, NT>(p, t, t.vbase, stb, tile + 2, vslot(tile + 2), tid, pg_prev);
        pg_prev = pg_cur;
        pg_cur = pg_fetch<D, 2, NW>(p, t, tile + 4, w);
      }
      if constexpr (!kSpread) pv(vslot(tile - 1), ts, sb);
    }
    // Raw scores; lane holds tokens 4 lg + i of each 16-token block, row l16.
    float x[RBR][8];
#pragma unroll
    for (int rb = 0; rb < RBR; ++rb)
#pragma unroll
      for (int j = 0; j < 8; ++j) x[rb][j] = s[j >> 2][rb][j & 3];
    if constexpr (kVis) {
      if (p.mask_words > 0) {
        // Flattened chunk: the 32 tokens of this step lie in one 64-token
        // mask word (tiles are multiples of 64 tokens); clear bits past the
        // chunk's end.
        const int word = (tile * G::TT + ts) >> 6;
#pragma unroll
        for (int rb = 0; rb < RBR; ++rb) {
          const uint64_t mk = flat_mask(p, mrow[rb], word);
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int bit = (ts + (j >> 2) * 16 + lg * 4 + (j & 3)) & 63;
            x[rb][j] = ((mk >> bit) & 1ull) ? x[rb][j] : kNegInf;
          }
        }
      } else {
#pragma unroll
        for (int rb = 0; rb < RBR; ++rb)
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            const int tt = tile * G::TT + ts + (j >> 2) * 16 + lg * 4 + (j & 3);
            const int bit = t.kv_begin + tt;
            const bool vis = tt < t.kv_len && (bit >= 64 || ((rmask[rb] >> bit) & 1ull));
            x[rb][j] = vis ? x[rb][j] : kNegInf;
          }
      }
    }
    // Reference maximum m (scaled units) per row, raised only when the row's
    // maximum exceeds it by more than kLazy (then p <= 2^kLazy, harmless in
    // fp16 and float32): alpha is 1 and O needs no rescale in almost every
    // step.
    float al[RBR];
    float lmx[RBR];  // one-slab layout: this lane's maximum of each row
    bool resc = false;
    if constexpr (kSpread) {
      // One slab per wavefront (compute-bound): each lane tests its own
      // scores against the raw threshold and P is formed with the current
      // references at once; only when a lane exceeds the threshold does the
      // wavefront (below, after the products) form the row maxima across the
      // four lanes of a row, move the references and form this P again.
#pragma unroll
      for (int rb = 0; rb < RBR; ++rb) {
        lmx[rb] = max3(max3(x[rb][0], x[rb][1], x[rb][2]), max3(x[rb][3], x[rb][4], x[rb][5]),
                       fmaxf(x[rb][6], x[rb][7]));
        resc = resc || lmx[rb] > thr[rb];
        al[rb] = 1.f;
      }
      // O += P V of the same sub-step of the previous tile, issued between
      // the vector work of the new P.
      if constexpr (kPrev) pv(vslot(tile - 1), ts, sb);
    } else {
      // Branch-free (the products of O += P V above overlap it): every step
      // forms the row maxima.
#pragma unroll
      for (int rb = 0; rb < RBR; ++rb) {
        const float mx = max3(max3(x[rb][0], x[rb][1], x[rb][2]), max3(x[rb][3], x[rb][4], x[rb][5]),
                              fmaxf(x[rb][6], x[rb][7]));
        update_ref(rb, mx, &al[rb]);
        resc = resc || al[rb] != 1.f;
      }
    }
    // P = exp2(x * c - m) of row block rb in the MFMA k order (slots 0..3:
    // block 0, 4..7: block 1) into pp[sb][rb]; returns the sum of the
    // rounded P added to `acc`.
    auto make_p = [&](int rb, float acc) {
      float e[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) e[j] = fast_exp2(fmaf(x[rb][j], c2, nm[rb]));
      uint32_t hw[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        hw[j] = pack_f16(e[2 * j], e[2 * j + 1]);
        acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, hw[j]), __builtin_bit_cast(f16x2, 0x3C003C00u), acc, false);
      }
      pp[sb][rb] = __builtin_bit_cast(bf16x8, make_uint4(hw[0], hw[1], hw[2], hw[3]));
      return acc;
    };
    float lst[RBR];  // one-slab layout: the sum of this step's P
#pragma unroll
    for (int rb = 0; rb < RBR; ++rb) {
      if constexpr (kSpread)
        lst[rb] = make_p(rb, 0.f);
      else
        l[rb] = make_p(rb, l[rb]);
    }
    // Keep the new P in this block (the compiler would otherwise sink its
    // computation next to its use in the following step).
#pragma unroll
    for (int rb = 0; rb < RBR; ++rb) asm volatile("" ::"v"(pp[sb][rb]), "v"(kSpread ? lst[rb] : l[rb]));
    if (__builtin_amdgcn_ballot_w64(resc) != 0) {
      if constexpr (kSpread) {
        // A lane exceeded its threshold: move the references (l *= alpha),
        // then form this step's P again relative to them.
#pragma unroll
        for (int rb = 0; rb < RBR; ++rb) update_ref(rb, lmx[rb], &al[rb]);
#pragma unroll
        for (int rb = 0; rb < RBR; ++rb) lst[rb] = make_p(rb, 0.f);
      }
      // Everything relative to the old maximum: O (which includes the
      // products issued above), and the P of the other sub-steps still
      // waiting for their products.
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int rb = 0; rb < RBR; ++rb) o[db][rb] *= al[rb];
#pragma unroll
      for (int s2 = 0; s2 < NSUB; ++s2)
        if (s2 != sb)
#pragma unroll
          for (int rb = 0; rb < RBR; ++rb)
            pp[s2][rb] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(f16x8, pp[s2][rb]) * static_cast<_Float16>(al[rb]));
    }
    if constexpr (kSpread) {
#pragma unroll
      for (int rb = 0; rb < RBR; ++rb) l[rb] += lst[rb];
    }
  };

  // The piece's V scale (see above).
  const int ev = ev_carry;
  const float vs = exp2i(15 - ev);  // bf16 -> fp16 factor
  float vmax = 0.f;           // largest |v| this lane has converted in the piece
  // V of tile j to fp16 in place: each lane converts the 16-byte chunks that
  // its own DMA wrote, which its own wait has made visible to it, so no
  // barrier is needed between the wait and the conversion.
  auto convert_own_v = [&](int j) {
    constexpr int KB = kHalfOps<NW>;
    const bool runs = half_in_runs<D>(p, t);
    uint4* vp[KB];
    uint4 x[KB];
#pragma unroll
    for (int c = 0; c < KB; ++c) {
      const int b = runs ? KB * w + c : c * NW + w;
      vp[c] = reinterpret_cast<uint4*>(vslot(j) + b * 1024 + lane * 16);
      x[c] = *vp[c];
    }
    float f[KB][8];
#pragma unroll
    for (int c = 0; c < KB; ++c) {
      const uint32_t wv[4] = {x[c].x, x[c].y, x[c].z, x[c].w};
      uint32_t h[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        f[c][2 * k] = bf16_lo(wv[k]);
        f[c][2 * k + 1] = bf16_hi(wv[k]);
        h[k] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(f[c][2 * k] * vs, f[c][2 * k + 1] * vs));
      }
      *vp[c] = make_uint4(h[0], h[1], h[2], h[3]);
    }
    // The chunks' largest |v|, as a shallow tree after the stores (it runs
    // while they complete), kept before the barrier: left to the scheduler it
    // sinks into the next steps and holds the 16 values in registers there.
    float t[KB];
#pragma unroll
    for (int c = 0; c < KB; ++c) {
      const float u0 = max3(fabsf(f[c][0]), fabsf(f[c][1]), fabsf(f[c][2]));
      const float u1 = max3(fabsf(f[c][3]), fabsf(f[c][4]), fabsf(f[c][5]));
      t[c] = max3(u0, u1, fmaxf(fabsf(f[c][6]), fabsf(f[c][7])));
    }
    float tm = t[0];
#pragma unroll
    for (int c = 1; c < KB; ++c) tm = fmaxf(tm, t[c]);
    vmax = fmaxf(vmax, tm);
    asm volatile("" : "+v"(vmax));
  };
  // Start of iteration i (0 <= i <= nt): wait for group i (K of tile i, V of
  // tile i - 1); for i > 0 convert this lane's chunks of V of tile i - 1 to
  // fp16; one barrier publishes both; issue group i + 3 into the halves
  // finished in iteration i - 1.  At i = 0 the queries go into registers
  // instead, and a second barrier frees their stages, which group 3 then
  // refills.
  auto sync = [&](int i, bool refill) {
    wait_vmem_n(group_ops<NW>(i + 1, nt) + group_ops<NW>(i + 2, nt));
    if (i > 0) {
      convert_own_v(i - 1);
      wait_lds_all();
    }
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");  // no LDS access moves above the barrier
    // K of tile i - 1 and V of tile i - 2 are finished: refill them (here, or
    // in the steps of tile i when `refill` is false; at i = 0 the refill
    // targets hold the queries: after the reads below).
    if (i > 0 && refill) refill_kv(i + 3);
    if (i == 0) {
      if (active) {
#pragma unroll
        for (int rb = 0; rb < RBR; ++rb) {
          const int row = slab * ROWS_W + rb * 16 + l16;
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            const int c = ks * 4 + lg;
            const uint4 v = *reinterpret_cast<const uint4*>(qarea + row * G::ROWB + ((c ^ (row & (G::CPT - 1))) << 4));
            const uint4 z = make_uint4(qok[rb] ? v.x : 0u, qok[rb] ? v.y : 0u, qok[rb] ? v.z : 0u, qok[rb] ? v.w : 0u);
            qf[rb][ks] = __builtin_bit_cast(bf16x8, z);
          }
        }
      }
      wait_lds_all();
      __builtin_amdgcn_s_barrier();
      asm volatile("" ::: "memory");
      refill_kv(3);
    }
  };
  // The NSUB steps of tile i (tile 0: no products of a previous tile).
  auto tile_steps = [&](auto vis_tag, int i) {
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) step(vis_tag, std::true_type{}, kslot(i), i, sb);
  };
  auto tile0_steps = [&](auto vis_tag) {
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) step(vis_tag, std::false_type{}, kslot(0), 0, sb);
  };
  if (active && nt > 0) {
    // Full tiles of unmasked nodes take the branch-free steps; the ragged
    // last tile, or the one tile of a masked node, the visibility test.  One
    // straight path per loop keeps the accumulators in place.
    const int nfull = t.masked ? 0 : t.kv_len / G::TT;
    sync(0, !kSpread);
    if (nfull > 0)
      tile0_steps(std::false_type{});
    else
      tile0_steps(std::true_type{});
    for (int i = 1; i < nfull; ++i) {
      sync(i, !kSpread);
      tile_steps(std::false_type{}, i);
    }
    for (int i = nfull > 1 ? nfull : 1; i < nt; ++i) {
      sync(i, !kSpread);
      tile_steps(std::true_type{}, i);
    }
    sync(nt, true);
#pragma unroll
    for (int sb = 0; sb < NSUB; ++sb) pv(vslot(nt - 1), tok0 + sb * 32, sb);  // O += P V of the last tile
  } else {
    for (int i = 0; i <= nt; ++i) sync(i, true);
  }
  // The piece's largest |v|: per wavefront by lane swaps, across the
  // wavefronts through LDS, published by the barrier that ends the tiles.
  float* const wave_vmax = reinterpret_cast<float*>(lds + kVexpOff);  // [NW]
  {
    float x = vmax;
    x = fmaxf(x, dpp<0xB1>(x));   // lane ^ 1
    x = fmaxf(x, dpp<0x4E>(x));   // lane ^ 2
    x = fmaxf(x, dpp<0x141>(x));  // the other quad of each 8
    x = fmaxf(x, dpp<0x140>(x));  // the other half of each 16
    const auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(s16[0]), __uint_as_float(s16[1]));
    const auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    x = fmaxf(__uint_as_float(s32[0]), __uint_as_float(s32[1]));
    if (lane == 0) wave_vmax[w] = x;
  }
  // Two wavefronts per slab hand half 1's state to half 0 through LDS.  With
  // one row block per wavefront (at most 32 rows) that state fits the 16 KB
  // above the tile stages, which no tile uses, so it is written before the
  // barrier that ends the tiles and that one barrier publishes both; larger
  // states reuse the tile stages after it.
  constexpr bool kEarlyHandOff = TS == 2 && RBR == 1;
  float* const so = reinterpret_cast<float*>(lds + (kEarlyHandOff ? kTileBytes : 0));  // [slab][rb][db][lane][4]
  float* const sml = reinterpret_cast<float*>(lds + kAuxOff);                             // [slab][rb][lane][2]
  auto hand_off = [&]() {
    // Row sums first: the four lane groups hold different tokens of the same rows.
#pragma unroll
    for (int rb = 0; rb < RBR; ++rb) {
      l[rb] += __shfl_xor(l[rb], 16);
      l[rb] += __shfl_xor(l[rb], 32);
    }
    if (TS == 2 && active && half == 1) {
#pragma unroll
      for (int rb = 0; rb < RBR; ++rb) {
#pragma unroll
        for (int db = 0; db < DB; ++db)
          *reinterpret_cast<f32x4*>(so + (((slab * RBR + rb) * DB + db) * 64 + lane) * 4) = o[db][rb];
        sml[((slab * RBR + rb) * 64 + lane) * 2 + 0] = m[rb];
        sml[((slab * RBR + rb) * 64 + lane) * 2 + 1] = l[rb];
      }
    }
  };
  if constexpr (kEarlyHandOff) hand_off();
  __syncthreads();  // all wavefronts are done with the tiles: reuse the LDS
  {
    float pm = 0.f;
#pragma unroll
    for (int k = 0; k < NW; ++k) pm = fmaxf(pm, wave_vmax[k]);
    const uint32_t pbits = __builtin_amdgcn_readfirstlane(__float_as_uint(pm));  // the same in every lane
    // E = the exponent of the piece's largest |v| (an all-zero piece fits any ev).
    const int e_u = pbits == 0u ? ev : min(kEvMax, max(kEvMin, static_cast<int>((pbits >> 23) & 0xffu) - 127));
    if (!retry && (e_u > ev || (e_u < ev - kEvWindow && ev > kEvMin))) {
      // Outside the window: the caller runs the piece again with ev = E
      // (which fits by construction); nothing of this pass is written.
      ev_carry = e_u;
      return false;
    }
    if (retry) ev_carry = min(kEvMax, ev + 2);  // headroom for the next piece's larger values
  }

  if constexpr (!kEarlyHandOff) hand_off();
  if constexpr (TS == 2) {
    // Merge the two token halves of every slab: half 1 handed its state to half 0.
    if constexpr (!kEarlyHandOff) __syncthreads();
    if (active && half == 0) {
#pragma unroll
      for (int rb = 0; rb < RBR; ++rb) {
        const float m1 = sml[((slab * RBR + rb) * 64 + lane) * 2 + 0];
        const float l1 = sml[((slab * RBR + rb) * 64 + lane) * 2 + 1];
        const float mm = fmaxf(m[rb], m1);
        const float muse = mm == kNegInf ? 0.f : mm;
        const float a0 = fast_exp2(m[rb] - muse), a1 = fast_exp2(m1 - muse);
        l[rb] = l[rb] * a0 + l1 * a1;
        m[rb] = mm;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const f32x4 o1 = *reinterpret_cast<const f32x4*>(so + (((slab * RBR + rb) * DB + db) * 64 + lane) * 4);
          o[db][rb] = o[db][rb] * a0 + o1 * a1;
        }
      }
    }
  }
  if (active && half == 0) {
#pragma unroll
    for (int rb = 0; rb < RBR; ++rb) {
      if (!qok[rb]) continue;
      // O carries the 2^(15 - ev) of V; fp16 partials keep it (ev goes with them).
      const float inv = l[rb] > 0.f ? (p.part_f16 ? 1.f : exp2i(ev - 15)) / l[rb] : 0.f;
      const float lse = l[rb] > 0.f ? (m[rb] + __log2f(l[rb])) * kLn2 : kNegInf;
#pragma unroll
      for (int db = 0; db < DB; ++db) {
        const float v4[4] = {o[db][rb][0] * inv, o[db][rb][1] * inv, o[db][rb][2] * inv, o[db][rb][3] * inv};
        write_partial(p, t, slot0[rb], qhead[rb], D, db * 16 + lg * 4, v4, lse, db == 0 && lg == 0, ev);
      }
    }
  }
  return true;
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
template <typename T, int D, int NW>
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
  const int tid = piece_tid();
  const int lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform
  const int rs = lane / LPS;
  const int tg = (lane % LPS) / LPT, li = lane % LPT;
  const int64_t stb = p.stride_token * static_cast<int64_t>(EB);
  const int R = t.row_count;
  const int r0 = rs * RL;

  if (p.mask_words > 0) issue_masks<NW>(p, t, tid);
  issue_prologue<D, EB, NW>(p, t, stb, tid);

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
  // The (row, 4 channels) chunks this thread writes at the end: chunk
  // tid + k * threads.
  constexpr int C4 = D / 4;
  constexpr int OUTS = (kMaxRowsDot * C4 + NW * 64 - 1) / (NW * 64);
  int out_slot[OUTS], out_head[OUTS];
#pragma unroll
  for (int k = 0; k < OUTS; ++k) {
    int entry = t.e0 + t.row_begin / p.g, head = kvh * p.g + t.row_begin % p.g;
    row_target(p, t, kvh, (tid + k * NW * 64) / C4, &entry, &head);
    out_slot[k] = p.entry_slot[entry];
    out_head[k] = head;
  }
  wait_vmem_n(0);  // queries in registers before the tile loop (see the matrix-core path)
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
    if (p.mask_words > 0)  // flattened chunk (row groups hold whole entries)
      return ((flat_mask(p, (r0 + r) / p.g, tt >> 6) >> (tt & 63)) & 1ull) != 0;
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

  run_tiles<D, EB, NW>(p, t, stb, tid, compute);

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
  float* sml = reinterpret_cast<float*>(lds + kAuxOff);
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
#pragma unroll
  for (int k = 0; k < OUTS; ++k) {
    const int r = (tid + k * NW * 64) / C4, c4 = (tid + k * NW * 64) % C4;
    if (r >= R) break;
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
    write_partial(p, t, out_slot[k], out_head[k], D, c4 * 4, v4, lse, c4 == 0, 15);
  }
}

// LAYOUT selects the instantiation (kContig, kPaged, kFlat); each is
// compiled without the other layouts' addressing code (its registers and
// scalar registers stay with the tile loop).  DOT: the kernel holds the
// dot-product path (float inputs; bf16 plans that send small pieces there).
// The bf16 kernels of the other plans leave it out: its code, inlined
// beside the matrix-core loops, costs them registers and schedule.  F16: the
// partials are written in fp16 (PacParams::part_f16), fixed per kernel so
// the other format's stores compile away (as a run-time flag it cost the
// contiguous kernel scalar-register spills).
template <typename T, int D, int LAYOUT, bool DOT, bool F16>
__global__ __launch_bounds__(kWaves<T> * 64) __attribute__((amdgpu_waves_per_eu(kWaves<T> / 4, kWaves<T> / 4)))
void pac_kernel(PacParams p) {
  constexpr int NW = kWaves<T>;
  p.part_f16 = F16 ? 1 : 0;
  if constexpr (LAYOUT != kPaged)
    p.page_shift = -1;  // every page-table branch folds away
  else
    __builtin_assume(p.page_shift >= 3 && p.page_shift <= 16);  // and every contiguous one
  if constexpr (LAYOUT != kFlat)
    p.mask_words = 0;  // and every row-table branch
  else
    __builtin_assume(p.mask_words > 0);
  // The work-group and work-item ids are read with the intrinsics: in a
  // kernel this large the library accessors stay out-of-line calls, whose
  // calling convention pushes the kernel arguments out of scalar registers.
  const int wg = static_cast<int>(__builtin_amdgcn_workgroup_id_x());
  const int bin = wg % p.num_bins;
  const int kvh = wg / p.num_bins;
  const int tb = p.bin_ptr[bin], te = p.bin_ptr[bin + 1];
  const int64_t esz = sizeof(T);
  // The next piece's record travels one dword per lane (lanes 0..11 of every
  // wavefront) while the current piece runs, and is handed over through LDS.
  // Two record slots: piece ti reads slot (ti - tb) & 1 and, before the
  // barrier that ends it, wavefront 0 writes the next record into the other
  // slot, which nobody reads any more, so that one barrier per piece orders
  // both.
  constexpr int TW = sizeof(DevTask) / 4;
  uint32_t* const rec_lds = reinterpret_cast<uint32_t*>(pac_lds + kAuxOff + kAuxBytes - 2 * sizeof(DevTask));
  const int tid = static_cast<int>(__builtin_amdgcn_workitem_id_x());
  if (tb < te && tid < TW) rec_lds[tid] = reinterpret_cast<const uint32_t*>(p.tasks + tb)[tid];
  __syncthreads();
  int ev_carry = kEvStart;  // the V scale exponent the next matrix-core piece starts from
  bool retry = false;  // the current task runs again with the V scale its first pass found
  for (int ti = tb; ti < te;) {
    const int slot = (ti - tb) & 1;
    DevTask task;
    __builtin_memcpy(&task, rec_lds + slot * TW, sizeof(DevTask));
    uint32_t next_word = 0;
    if (ti + 1 < te && tid < TW) next_word = reinterpret_cast<const uint32_t*>(p.tasks + ti + 1)[tid];
    // The record is the same in every lane: read it as wave-uniform values so
    // that everything derived from it (trip counts, active wavefronts) is
    // scalar control flow and the barriers stay in uniform code.
    TaskInfo t;
    t.piece = __builtin_amdgcn_readfirstlane(task.piece);
    t.kv_begin = __builtin_amdgcn_readfirstlane(task.kv_begin);
    t.kv_len = __builtin_amdgcn_readfirstlane(task.kv_len);
    t.row_begin = __builtin_amdgcn_readfirstlane(task.row_begin);
    t.row_count = __builtin_amdgcn_readfirstlane(task.row_count);
    t.e0 = __builtin_amdgcn_readfirstlane(task.e0);
    t.masked = (__builtin_amdgcn_readfirstlane(task.flags) & kDevMasked) != 0;
    const int64_t tok0 = (static_cast<int64_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(task.tok0 >> 32))) << 32) |
                         static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(task.tok0)));
    t.node = __builtin_amdgcn_readfirstlane(task.node);
    t.flat0 = static_cast<int>(tok0);
    t.linear = (__builtin_amdgcn_readfirstlane(task.flags) & kDevLinear) != 0;
    t.shared = (__builtin_amdgcn_readfirstlane(task.flags) & kDevShared) != 0;
    t.pg0 = p.page_shift >= 0 ? ((const __attribute__((address_space(4))) int32_t*)(p.page_ptr))[t.node] : 0;
    // Contiguous: K/V at the piece's first token; paged and flattened: the
    // head's pool start (blocks add their rows), or for a flattened chunk
    // over consecutive rows its first row.
    int64_t first = p.page_shift >= 0 ? 0 : tok0;
    if (p.mask_words > 0)
      first = t.linear ? (static_cast<int64_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(task.row0 >> 32))) << 32) |
                             static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(task.row0)))
                       : 0;
    const int64_t off = (kvh * p.stride_head + first * p.stride_token) * esz;
    t.kbase = static_cast<const char*>(p.k) + off;
    t.vbase = static_cast<const char*>(p.v) + off;
    bool done = false, finished = true;
    if constexpr (sizeof(T) == 2) {
      if (!DOT || t.row_count >= p.mfma_min_rows) {
        // Slabs of 16 RBR rows, TS wavefronts per slab.
        static_assert(NW == 8, "row dispatch for 8 wavefronts");
        // Bandwidth-bound layouts stream K/V with the non-temporal hint
        // unless other tasks read the same tokens (row groups, the
        // query-guided baseline): those reads may still hit in L2.  The
        // compute-bound layout (more than 128 rows, where the row groups
        // are) keeps the default policy.
        if (t.row_count <= 32) {
          if (t.shared)
            finished = mfma_piece<D, 1, 2, NW, false>(p, t, kvh, ev_carry, retry);
          else
            finished = mfma_piece<D, 1, 2, NW, true>(p, t, kvh, ev_carry, retry);
        } else if (t.row_count <= 128) {
          if (t.shared)
            finished = mfma_piece<D, 2, 2, NW, false>(p, t, kvh, ev_carry, retry);
          else
            finished = mfma_piece<D, 2, 2, NW, true>(p, t, kvh, ev_carry, retry);
        } else {
          finished = mfma_piece<D, 2, 1, NW, false>(p, t, kvh, ev_carry, retry);
        }
        done = true;
      }
    }
    if constexpr (DOT) {
      if (!done) dot_piece<T, D, NW>(p, t, kvh);
    }
    if (tid < TW) rec_lds[(slot ^ 1) * TW + tid] = next_word;
    __syncthreads();  // the piece is finished with the LDS; the next record is in place
    retry = !finished;
    if (finished) ++ti;
  }
}

template <typename T, int D, int LAYOUT, bool DOT, bool F16>
int launch_layout(const PacParams& p, void* stream) {
  const int grid = p.num_bins * p.hkv;
  constexpr size_t lds = LAYOUT == kFlat ? kLdsBytesFlat : kLdsBytes;
  // The dynamic-LDS limit is raised once per device (the attribute is per
  // device); a race between two threads only sets it twice.
  constexpr int kMaxDevices = 64;
  static bool configured[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return static_cast<int>(e);
  if (dev < 0 || dev >= kMaxDevices || !configured[dev]) {
    e = hipFuncSetAttribute(reinterpret_cast<const void*>(&pac_kernel<T, D, LAYOUT, DOT, F16>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return static_cast<int>(e);
    if (dev >= 0 && dev < kMaxDevices) configured[dev] = true;
  }
  hipLaunchKernelGGL((pac_kernel<T, D, LAYOUT, DOT, F16>), dim3(grid), dim3(kWaves<T> * 64), lds,
                     static_cast<hipStream_t>(stream), p);
  return static_cast<int>(hipGetLastError());
}
template <typename T, int D, bool DOT, bool F16>
int launch_dot(const PacParams& p, void* stream) {
  if (p.mask_words > 0) return launch_layout<T, D, kFlat, DOT, F16>(p, stream);
  return p.page_shift >= 0 ? launch_layout<T, D, kPaged, DOT, F16>(p, stream)
                           : launch_layout<T, D, kContig, DOT, F16>(p, stream);
}
// fp16 partials only come with bf16 plans that run every piece on the
// matrix cores (the kernels without the dot path).
template <typename T, int D>
int launch_one(const PacParams& p, void* stream) {
  if constexpr (sizeof(T) == 2) {
    if (p.mfma_min_rows <= 1)
      return p.part_f16 ? launch_dot<T, D, false, true>(p, stream) : launch_dot<T, D, false, false>(p, stream);
  }
  if (p.part_f16) return static_cast<int>(hipErrorInvalidValue);
  return launch_dot<T, D, true, false>(p, stream);
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
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, pac_kernel<uint16_t, 128, kContig, false, true>, kWaves<uint16_t> * 64, kLdsBytes);
  else if (in_dtype == PST_BF16)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, pac_kernel<uint16_t, 64, kContig, false, true>, kWaves<uint16_t> * 64, kLdsBytes);
  else if (head_dim == 128)
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, pac_kernel<float, 128, kContig, true, false>, kWaves<float> * 64, kLdsBytes);
  else
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(blocks, pac_kernel<float, 64, kContig, true, false>, kWaves<float> * 64, kLdsBytes);
  return static_cast<int>(e);
}

}  // namespace pst
