// situ_moe_run_static: the layer with the library's own per-device scratch
// array in place of a caller workspace, for callers that cannot allocate
// device memory (code under HIP graph capture, tight serving loops, harnesses
// that forbid allocation).
//
// The array is a file-scope __device__ object: each GPU the library runs on
// holds its own copy, from the first call on that GPU until the process
// ends.  In host code its name is only a stand-in for the symbol, not a
// device address; the address comes from hipGetSymbolAddress, once per
// device with that device current, and only that address is handed to the
// kernels.  Every call on one GPU uses the same array: calls that overlap in
// time on one GPU race, and nothing in it is assumed to start at zero (each
// call writes every region it reads).
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/situ_moe.h"
#include "internal.hpp"

namespace {

static __device__ __align__(256) uint8_t scratch[SITU_MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

extern "C" situ_status situ_moe_run_static(const situ_moe_plan_t* plan, const situ_moe_tensors* tensors,
                                           void* hip_stream) {
  if (!plan) return situ::fail_status(SITU_E_NULL_ARG, "plan is NULL");
  if (plan->workspace_bytes > SITU_MOE_STATIC_SCRATCH_BYTES)
    return situ::fail_status(SITU_E_WORKSPACE,
                             "the plan needs %llu bytes of workspace; the static scratch holds %llu (use situ_moe_run "
                             "with a caller workspace)",
                             (unsigned long long)plan->workspace_bytes,
                             (unsigned long long)SITU_MOE_STATIC_SCRATCH_BYTES);
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return situ::fail_status(SITU_E_DEVICE, "no current HIP device");
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lk(g_mu);
    if (!g_ptr[dev]) {
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || !p)
        return situ::fail_status(SITU_E_DEVICE, "hipGetSymbolAddress of the static scratch failed on device %d: %s",
                                 dev, hipGetErrorString(e));
      g_ptr[dev] = p;
    }
    ptr = g_ptr[dev];
  }
  return situ_moe_run(plan, tensors, ptr, SITU_MOE_STATIC_SCRATCH_BYTES, hip_stream);
}
