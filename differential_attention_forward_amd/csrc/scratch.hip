// Library-held device scratch for diffattn_decode_noalloc, the decode entry
// point for callers that cannot allocate device memory.  The array below is
// the split-K partial-state buffer of that call: one copy per GPU, resident
// from the library's load until the process ends.
//
// On the host, `scratch` names a host-side stand-in, not the device array:
// its device address is looked up once per device (hipGetSymbolAddress, with
// that device current) and only that address is ever handed to kernels.
#include <mutex>

#include "../../include/diffattn.h"
#include "kernels.h"

static __device__ __align__(256) float scratch[DIFFATTN_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace {

constexpr int kMaxDevices = 64;
void* g_scratch_addr[kMaxDevices];  // device address of `scratch`, per device
std::mutex g_scratch_mutex;

}  // namespace

namespace diffattn {

hipError_t decode_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_addr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev] = p;
  }
  *ptr = g_scratch_addr[dev];
  return hipSuccess;
}

}  // namespace diffattn
