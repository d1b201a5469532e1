// Scratch memory of the entry point that allocates nothing
// (fa_fwd_splitkv_noalloc): one file-scope device array of kScratchBytes.
// Each GPU the library runs on holds its own copy, at its own address, from
// the first use on that device until the process ends.  Host code never
// uses the array's name as an address (on the host it only names the
// symbol): the device address of each GPU's copy is looked up once, with
// that device current, and kept.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "fa_launch.h"

namespace iofa {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_ptr[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t scratch_address(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch_ptr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr) return hipErrorInvalidSymbol;
      g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace iofa
