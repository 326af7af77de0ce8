// Fixed device scratch of the no-allocation forward (sparse_mla_fwd_noalloc):
// the split partials of a call whose caller cannot allocate device memory
// (code under HIP graph capture, tight serving loops) live in a file-scope
// device array instead of a hipMalloc'ed workspace.
//
// Each GPU the library runs on holds its own copy of the array, at its own
// address, until the process ends. The array's name in host code is only a
// host-side stand-in, so kernels get the device address resolved here with
// hipGetSymbolAddress, once per device, with that device current.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <string>

#include "launch.h"

namespace smla {
namespace {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

int scratch_buffer(int dev, void** out, std::string* err) {
  if (dev < 0 || dev >= kMaxDevices) {
    *err = "device id beyond " + std::to_string(kMaxDevices - 1);
    return SMLA_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    // The caller made `dev` current (hipGetDevice), so the address resolved
    // is that device's copy of the array.
    void* ptr = nullptr;
    const hipError_t e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr) {
      *err = std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e);
      return SMLA_ERR_HIP;
    }
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return SMLA_OK;
}

}  // namespace smla
