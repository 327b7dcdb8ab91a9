// static_scratch.hip -- the workspace of pkvd_decode_static: a file-scope
// device array, so that calls through that entry point never allocate.
//
// Each device the library runs on holds its own copy of `scratch` (kStaticScratchBytes)
// from the time the code object is loaded until the process ends.  Device
// globals start zero-filled, which is the state the decode's int32 area (the
// arrival counters) must start in; every call leaves it at zero again.  In
// host code the array's name is only a stand-in for the symbol: its device
// address comes from hipGetSymbolAddress, once per device (with that device
// current), and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "decode_args.h"

namespace pkvd {

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

namespace {

std::mutex g_mutex;
void* g_addr[64] = {nullptr};

}  // namespace

hipError_t static_scratch(void** ptr, size_t* bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  *bytes = kStaticScratchBytes;
  return hipSuccess;
}

}  // namespace pkvd
