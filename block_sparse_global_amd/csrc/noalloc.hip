// The refinement scratch of ress_refine_dropset_noalloc: a fixed device
// array inside the library's code object, for callers that cannot allocate
// device memory (code under graph capture, tight serving loops, harnesses
// that forbid allocation). Each GPU that loads the library holds its own
// copy until the process ends.
//
// Host code never passes the array's name to a kernel or a copy: in host
// code that name is only a stand-in for the symbol. The device address of
// each GPU's copy is looked up once per device, with that device current,
// on the first call there (hipGetSymbolAddress), and kept.
#include <atomic>
#include <mutex>

#include "ress_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[RESS_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::atomic<void*> g_addr[kMaxDevices];
std::mutex g_lock;

}  // namespace

namespace ress {

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    std::lock_guard<std::mutex> guard(g_lock);
    p = g_addr[dev].load(std::memory_order_relaxed);
    if (p == nullptr) {
      e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (p == nullptr || ((uintptr_t)p & 255u) != 0) return hipErrorInvalidSymbol;
      g_addr[dev].store(p, std::memory_order_release);
    }
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace ress
