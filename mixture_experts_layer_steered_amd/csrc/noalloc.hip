// Fixed device scratch for moe_forward_noalloc: the workspace of the layer
// for callers that cannot allocate device memory (code under HIP graph
// capture, tight serving loops, harnesses that forbid hipMalloc).
//
// The array lives in this library's code object, so each device the library
// runs on holds one copy of it until the process ends.  Host code never
// passes the array's name to a kernel (on the host that name is only a
// stand-in, not a device address): the device address of each device's copy
// is looked up once, with that device current, and kept per device.
#include <mutex>

#include "kernels.h"

namespace {

constexpr int kScratchDevices = 64;

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES_DEV];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kScratchDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  *bytes = sizeof(scratch);
  return hipSuccess;
}
