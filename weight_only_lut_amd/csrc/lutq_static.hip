// Fixed device scratch for lutq_matmul_noalloc: the split-K arrival counters
// and fp32 partial sums of callers that cannot allocate device memory.
//
// The array below lives in the library's device image: each GPU the library
// runs on holds its own copy, at its own address, until the process ends.
// In host code its name is only a host-side stand-in, so the device address
// is looked up once per device (hipGetSymbolAddress, with that device
// current) and only that pointer is handed to kernels.
#include <mutex>

#include "lutq_internal.h"

namespace lutq {

static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_static_mu;
void* g_static_ptr[kMaxDevices];  // per device ordinal; null until looked up
}  // namespace

hipError_t static_scratch(void** out, hipStream_t s) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_static_mu);
  if (!g_static_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    // The image zero-fills the array when it is loaded; the counters are
    // cleared once more on the first call's stream, before its launches.
    e = launch_fill_u16(reinterpret_cast<uint16_t*>(ptr), (long long)(kSplitCounterBytes / 2), 0, s);
    if (e != hipSuccess) return e;
    g_static_ptr[dev] = ptr;
  }
  *out = g_static_ptr[dev];
  return hipSuccess;
}

}  // namespace lutq
