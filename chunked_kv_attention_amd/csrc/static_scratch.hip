// The library's own split scratch, for callers that cannot allocate.
//
// ckv_chunk_attention_static runs the same kernels as ckv_chunk_attention but
// keeps the fp16 partial outputs and float32 log-sum-exps of a split call in this
// file-scope device array instead of the cache arena, so a caller can issue
// it with nothing allocated for it.  Each GPU the library runs on holds its
// own copy of the array until the process ends; every call on a GPU shares
// it, so calls that overlap in time on one GPU (two streams, two caches)
// race on it.  The kernels overwrite every partial a call reads before the
// merge reads it, so nothing needs clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace ckv {
namespace {

static __device__ __align__(256) char scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // device address of `scratch`, per device

}  // namespace

hipError_t static_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    // the array's host-side name is not a device address: look the device
    // address up once per device, with that device current
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace ckv
