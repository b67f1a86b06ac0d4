// The library's one static device buffer: the workspace of dr_chunk_fwd_noalloc, for callers that
// cannot allocate device memory. Each GPU the library runs on holds its own copy for the life of
// the process. Host code never passes the array's name to a kernel (on the host it is only a
// stand-in for the symbol): it asks the runtime for the array's device address once per device and
// uses that address everywhere.
#include <mutex>

#include "../../include/deltarule.h"
#include "launch.hpp"

namespace dr {

static __device__ __align__(256) unsigned char scratch[DR_NOALLOC_SCRATCH_BYTES];

hipError_t scratch_buffer(void** ptr) {
  static std::mutex mu;
  static void* addr[256] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 256) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with device `dev` current
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace dr
