// Partial output reduction (POR) and measurement helpers, gfx950.
//
// CoDec: Prefix-Shared Decoding Kernel for LLMs, section 块内内核原语 (POR
// kernel): two partial results of the same query are merged at the common
// maximum m = max(m1, m2) with weights s_i e^{m_i - m}; section 块间启动与树归约:
// the merge is associative and commutative, so the tree reduction becomes one
// independent chain per query, and the chains run in parallel.  With
// normalised partials and their natural-log LSE (DEFT: Decoding with Flash
// Tree-Attention, section 速读 and A.4 phase 2; FlashDecoding's second level
// in the KV-cache engineering blog, section 4) the n-way merge of a chain is
//     L* = max_i LSE_i,  w_i = exp(LSE_i - L*),
//     O = sum_i w_i O_i / sum_i w_i,  LSE = L* + ln sum_i w_i,
// which is the binary POR folded over the chain; empty partials (LSE = -inf)
// get weight 0.  Each thread owns one chain: (query, q-head, 4 channels).
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "pst_internal.h"

namespace pst {
namespace {

typedef __bf16 bf16x2n __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

constexpr int kPorThreads = 256;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kNegInf = -__builtin_inff();

// Grid: (query, chunk of kPorThreads (head, 4-channel) pairs).  One pass over
// the chain in batches: all loads of a batch are in flight together, then the
// batch is folded into the running (max, sum, O) at the batch maximum (the
// binary merge applied to the whole batch at once).  Full batches take 8
// slots; the tail (fewer than 8) is one batch of 8, 4, 2 or 1 slots whose
// unused entries are not loaded and get weight 0.  The slot range is
// uniform over the workgroup, so these choices are scalar branches.
constexpr int kBatch = 8;
// F16: the partials are fp16 values times 2^(15 - e), with e per (slot, head)
// in the (LSE, e) pair that replaces the LSE.
template <int D, bool BF16_OUT, bool F16>
__global__ __launch_bounds__(kPorThreads) void por_kernel(PorParams p, int chunks) {
  const int r = blockIdx.x / chunks;
  const int chunk = blockIdx.x % chunks;
  const int64_t s0 = p.slot_ptr[r], s1 = p.slot_ptr[r + 1];
  constexpr int C4 = D / 4;
  const int idx = chunk * kPorThreads + threadIdx.x;
  if (idx >= p.hq * C4) return;
  const int h = idx / C4, c4 = idx % C4;
  float m = kNegInf, z = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // Fold slots [s, s + n) (n <= NB) into the running state.
  auto fold = [&](auto nb_tag, int64_t s, int n) {
    constexpr int NB = decltype(nb_tag)::value;
    float lse[NB];
    float4 x[NB];
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      lse[j] = kNegInf;
      x[j] = make_float4(0.f, 0.f, 0.f, 0.f);
      if (j < n) {
        const int64_t at = ((s + j) * p.hq + h) * D + c4 * 4;
        if constexpr (F16) {
          typedef _Float16 h2 __attribute__((ext_vector_type(2)));
          const float2 le = reinterpret_cast<const float2*>(p.lsepart)[(s + j) * p.hq + h];
          const uint2 u = *reinterpret_cast<const uint2*>(reinterpret_cast<const _Float16*>(p.opart) + at);
          lse[j] = le.x;
          const float sc = __uint_as_float(static_cast<uint32_t>(__float_as_int(le.y) - 15 + 127) << 23);
          const h2 a = __builtin_bit_cast(h2, u.x), b = __builtin_bit_cast(h2, u.y);
          x[j] = make_float4(static_cast<float>(a[0]) * sc, static_cast<float>(a[1]) * sc,
                             static_cast<float>(b[0]) * sc, static_cast<float>(b[1]) * sc);
        } else {
          lse[j] = p.lsepart[(s + j) * p.hq + h];
          x[j] = *reinterpret_cast<const float4*>(p.opart + at);
        }
      }
    }
    float bm = lse[0];
#pragma unroll
    for (int j = 1; j < NB; ++j) bm = fmaxf(bm, lse[j]);
    const float mn = fmaxf(m, bm);
    const float mref = mn == kNegInf ? 0.f : mn;
    const float a = __builtin_amdgcn_exp2f((m - mref) * kLog2e);  // 0 while m is -inf
    z *= a;
    acc.x *= a;
    acc.y *= a;
    acc.z *= a;
    acc.w *= a;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const float wgt = __builtin_amdgcn_exp2f((lse[j] - mref) * kLog2e);
      const bool live = wgt > 0.f;  // an empty partial's O may be anything
      z += wgt;
      acc.x += live ? wgt * x[j].x : 0.f;
      acc.y += live ? wgt * x[j].y : 0.f;
      acc.z += live ? wgt * x[j].z : 0.f;
      acc.w += live ? wgt * x[j].w : 0.f;
    }
    m = mn;
  };
  int64_t s = s0;
  for (; s + kBatch <= s1; s += kBatch) fold(std::integral_constant<int, kBatch>{}, s, kBatch);
  const int rem = static_cast<int>(s1 - s);
  if (rem > 4)
    fold(std::integral_constant<int, 8>{}, s, rem);
  else if (rem > 2)
    fold(std::integral_constant<int, 4>{}, s, rem);
  else if (rem == 2)
    fold(std::integral_constant<int, 2>{}, s, 2);
  else if (rem == 1)
    fold(std::integral_constant<int, 1>{}, s, 1);
  const float inv = z > 0.f ? 1.f / z : 0.f;
  const int64_t o = (static_cast<int64_t>(r) * p.hq + h) * D + c4 * 4;
  if (BF16_OUT) {
    f32x2 a = {acc.x * inv, acc.y * inv}, b = {acc.z * inv, acc.w * inv};
    uint2 u;
    u.x = __builtin_bit_cast(uint32_t, __builtin_convertvector(a, bf16x2n));
    u.y = __builtin_bit_cast(uint32_t, __builtin_convertvector(b, bf16x2n));
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.out) + o) = u;
  } else {
    *reinterpret_cast<float4*>(static_cast<float*>(p.out) + o) =
        make_float4(acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv);
  }
  if (p.lse_out && c4 == 0) p.lse_out[static_cast<int64_t>(r) * p.hq + h] = z > 0.f ? m + __logf(z) : kNegInf;
}

// Overwrite a buffer with 128-bit stores (evicts L2 and the last-level cache).
__global__ __launch_bounds__(256) void flush_kernel(uint4* buf, size_t n16) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n16; i += stride)
    buf[i] = make_uint4(static_cast<uint32_t>(i), 0u, 0u, 0u);
}

// Stream a buffer with 128-bit loads; one float per workgroup keeps the loads alive.
__global__ __launch_bounds__(256) void read_kernel(const uint4* buf, size_t n16, float* sink) {
  const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
  uint32_t acc = 0;
  size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4 a = buf[i], b = buf[i + stride], c = buf[i + 2 * stride], d = buf[i + 3 * stride];
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4 a = buf[i];
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  __shared__ uint32_t red[256];
  red[threadIdx.x] = acc;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t x = 0;
    for (int j = 0; j < 256; ++j) x ^= red[j];
    sink[blockIdx.x] = static_cast<float>(x & 1u);
  }
}

}  // namespace

int launch_por(const PorParams& p, int head_dim, int out_dtype, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int chunks = (p.hq * (head_dim / 4) + kPorThreads - 1) / kPorThreads;
  const dim3 grid(static_cast<unsigned>(p.num_queries) * chunks), block(kPorThreads);
  const bool bf = out_dtype == PST_BF16;
  auto go = [&](auto kern) { hipLaunchKernelGGL(kern, grid, block, 0, s, p, chunks); };
  if (p.part_f16) {  // bf16 output only
    if (head_dim == 128)
      go(por_kernel<128, true, true>);
    else
      go(por_kernel<64, true, true>);
  } else if (head_dim == 128) {
    if (bf)
      go(por_kernel<128, true, false>);
    else
      go(por_kernel<128, false, false>);
  } else {
    if (bf)
      go(por_kernel<64, true, false>);
    else
      go(por_kernel<64, false, false>);
  }
  return static_cast<int>(hipGetLastError());
}

int launch_flush(void* buf, size_t bytes, void* stream) {
  hipLaunchKernelGGL(flush_kernel, dim3(4096), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<uint4*>(buf), bytes / 16);
  return static_cast<int>(hipGetLastError());
}

int launch_read(const void* buf, size_t bytes, float* sink, void* stream) {
  hipLaunchKernelGGL(read_kernel, dim3(4096), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const uint4*>(buf), bytes / 16, sink);
  return static_cast<int>(hipGetLastError());
}

}  // namespace pst
