// Fixed device scratch for the entry point that allocates nothing
// (mssm_selective_scan_fwd_noalloc), for callers that cannot allocate device memory
// at the call (code under stream capture, tight serving loops, harnesses that forbid
// it).
//
// The array below is a file-scope device variable: every GPU the library runs on
// holds its own copy, at its own address, from the first call on that GPU until the
// process ends.  In host code its name is only a stand-in for the symbol, never a
// device address, so the address is looked up once per device with
// hipGetSymbolAddress (with that device current) and kept; kernels get that pointer.
//
// Calls on one GPU share its copy.  A later call may start before an earlier one has
// finished only if the two are ordered on one stream; calls that overlap on one GPU
// (different streams, no ordering) race on it.
#include <atomic>
#include <mutex>

#include "internal.h"

namespace mssm {
namespace {

__device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
std::atomic<void*> g_ptr[kMaxDevices];

}  // namespace

hipError_t scratch_address(hipStream_t stream, void** out) {
  int dev = 0;
  hipError_t e = stream != nullptr ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_mu);
    p = g_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      int cur = 0;
      e = hipGetDevice(&cur);
      if (e != hipSuccess) return e;
      if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (cur != dev) {
        const hipError_t back = hipSetDevice(cur);
        if (e == hipSuccess) e = back;
      }
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}

}  // namespace mssm
