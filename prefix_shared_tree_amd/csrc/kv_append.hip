// Writing a decode step's new K/V rows into the pools (gfx950).
//
// DEFT: Decoding with Flash Tree-Attention, section A.1: each request's tree
// grows by the token it just decoded, whose K and V join the cache before
// the next step's attention.  One launch copies the new rows of every
// request, K and V together: thread = one 16-byte chunk of one (row, kv head);
// for pst_tree_append the same launch also sets the grown lengths.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>

#include "pst_internal.h"

namespace pst {
namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void write_rows_kernel(KvRowsParams p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  const int64_t per_row = static_cast<int64_t>(p.hkv) * p.chunks;  // chunks of one new row, all heads
  if (i >= p.n * per_row) return;
  const int64_t r = i / per_row;
  const int h = static_cast<int>((i % per_row) / p.chunks);
  const int c = static_cast<int>(i % p.chunks);
  const int64_t row = p.rows[r];
  if (row < 0 || row >= p.pool_tokens) return;  // outside the pools: not written
  const int64_t src = (r * p.hkv + h) * p.chunks + c;  // [n][hkv][chunks] of 16 bytes
  const int64_t dst = h * p.stride_head_bytes + row * p.stride_token_bytes + c * 16;
  *reinterpret_cast<uint4*>(static_cast<char*>(p.k_pool) + dst) = reinterpret_cast<const uint4*>(p.k_new)[src];
  *reinterpret_cast<uint4*>(static_cast<char*>(p.v_pool) + dst) = reinterpret_cast<const uint4*>(p.v_new)[src];
}

// pst_tree_append: threads below n * hkv * chunks copy one 16-byte chunk of K
// and of V each (pool tokens from the arguments); threads below n_sets store
// one word each.
__global__ __launch_bounds__(kThreads) void append_kernel(AppendParams p) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (i < p.n_sets) *p.set_addr[i] = p.set_val[i];
  const int64_t per_row = static_cast<int64_t>(p.kv.hkv) * p.kv.chunks;
  if (i >= p.kv.n * per_row) return;
  const int64_t r = i / per_row;
  const int h = static_cast<int>((i % per_row) / p.kv.chunks);
  const int c = static_cast<int>(i % p.kv.chunks);
  const int64_t row = p.rows[r];
  if (row < 0 || row >= p.kv.pool_tokens) return;
  const int64_t src = (r * p.kv.hkv + h) * p.kv.chunks + c;
  const int64_t dst = h * p.kv.stride_head_bytes + row * p.kv.stride_token_bytes + c * 16;
  *reinterpret_cast<uint4*>(static_cast<char*>(p.kv.k_pool) + dst) = reinterpret_cast<const uint4*>(p.kv.k_new)[src];
  *reinterpret_cast<uint4*>(static_cast<char*>(p.kv.v_pool) + dst) = reinterpret_cast<const uint4*>(p.kv.v_new)[src];
}

}  // namespace

int launch_append(const AppendParams& p, void* stream) {
  const int64_t total = std::max<int64_t>(p.kv.n * p.kv.hkv * p.kv.chunks, p.n_sets);
  if (total == 0) return 0;
  const int blocks = static_cast<int>((total + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(append_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
  return static_cast<int>(hipGetLastError());
}

int launch_write_rows(const KvRowsParams& p, void* stream) {
  const int64_t total = p.n * p.hkv * p.chunks;
  if (total == 0) return 0;
  const int blocks = static_cast<int>((total + kThreads - 1) / kThreads);
  hipLaunchKernelGGL(write_rows_kernel, dim3(blocks), dim3(kThreads), 0, static_cast<hipStream_t>(stream), p);
  return static_cast<int>(hipGetLastError());
}

}  // namespace pst
