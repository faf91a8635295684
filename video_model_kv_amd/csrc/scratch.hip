// Library-held scratch memory for the entry point that allocates nothing
// (qkv_quantize_chunk_noalloc): one file-scope device array, which every GPU
// the library runs on holds until the process ends, at its own address on
// each device.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in symbol): the device address comes from
// hipGetSymbolAddress, looked up once per device with that device current.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace qkv {

namespace {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

}  // namespace

hipError_t scratch_of_current_device(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace qkv
