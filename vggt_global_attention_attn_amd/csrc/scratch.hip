// Workspace of vggt_attn_forward_noalloc: a file-scope device array instead of caller memory,
// for callers that cannot allocate (code under HIP graph capture, tight serving loops).  The
// array is part of the code object, so every GPU the library runs on holds one copy of it from
// module load until the process ends; its size is the stated limit of that entry point.
//
// In host code `scratch` names a host-side stand-in, not the device array: its device address
// is looked up once per device with hipGetSymbolAddress (that device current) and only that
// address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "plan.h"

namespace vggt {
namespace {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxScratchDevices = 64;

}  // namespace

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  static std::mutex mu;
  static void* addr[kMaxScratchDevices] = {};
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *out = addr[dev];
  return hipSuccess;
}

}  // namespace vggt
