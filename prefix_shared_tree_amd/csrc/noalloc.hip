// pst_decode_attn_noalloc: the hot path for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops,
// harnesses that forbid hipMalloc).  The partial outputs that
// pst_decode_attn keeps in a caller-owned workspace live here in one
// file-scope device array instead, which every GPU the library runs on holds
// from the library's load until the process ends.
#include <hip/hip_runtime.h>

#include <mutex>
#include <string>

#include "pst_internal.h"

namespace pst {
namespace {

constexpr size_t kScratchBytes = PST_NOALLOC_SCRATCH_BYTES;  // per device
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};  // the array's device address, per device

// The device address of `scratch` on the current device (looked up once per
// device, with that device current).  In host code `scratch` names a host-side
// stand-in, never the device memory, so only this address is passed on.
pst_status scratch_on_current_device(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    set_error(std::string("no HIP device: ") + hipGetErrorString(e));
    return PST_E_NO_DEVICE;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    set_error("device ordinal beyond the library's table");
    return PST_E_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !ptr) {
      set_error(std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
      return PST_E_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return PST_OK;
}

}  // namespace
}  // namespace pst

using namespace pst;

extern "C" {

pst_status pst_decode_attn_noalloc(pst_plan_t plan, const void* q, const void* k_pool, const void* v_pool,
                                   void* out, float* lse_out, void* stream) {
  pst_status st = plan_ready_for_launch(plan);  // before any device call
  if (st != PST_OK) return st;
  size_t need = 0;
  st = pst_plan_workspace_size(plan, &need);
  if (st != PST_OK) return st;
  if (need > kScratchBytes) {
    set_error("the plan's partial outputs need " + std::to_string(need) + " bytes; pst_decode_attn_noalloc holds " +
              std::to_string(kScratchBytes) + " (use pst_decode_attn with a workspace)");
    return PST_E_WORKSPACE;
  }
  void* ws = nullptr;
  st = scratch_on_current_device(&ws);
  if (st != PST_OK) return st;
  return pst_decode_attn(plan, q, k_pool, v_pool, out, lse_out, ws, kScratchBytes, stream);
}

}  // extern "C"
