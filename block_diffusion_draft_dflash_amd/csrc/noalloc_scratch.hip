// Library-owned scratch memory of dflash_block_attention_noalloc, the entry
// point for callers that cannot allocate device memory (code under HIP-graph
// capture, tight serving loops, harnesses that forbid allocation).
//
// The array is a file-scope device variable: every GPU that loads the library
// holds its own copy, at its own address, until the process ends. In host
// code the array's name only stands in for it; the device address of the
// current device's copy is looked up here once per device (with that device
// current) and kept, and that address is what the kernels receive.
#include <mutex>

#include "dflash_internal.h"

namespace dflash {
namespace {

static __device__ __align__(256) unsigned char scratch[DFLASH_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_addr[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(void** addr) {
  *addr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> hold(g_lock);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *addr = g_addr[dev];
  return hipSuccess;
}

}  // namespace dflash
