// Library-owned device scratch for the one entry point that allocates nothing
// (linattn_noncausal_fwd_noalloc, for callers that cannot call hipMalloc: code
// under HIP graph capture, tight serving loops, harnesses that forbid it).
//
// `scratch` is a file-scope device array: every GPU the library runs on holds
// its own copy, at its own address, until the process ends.  In host code the
// array's name is only a stand-in for the symbol, never a device address: its
// address on a device comes from hipGetSymbolAddress, taken once per device
// with that device current and cached here, and only that address is ever
// handed to a kernel.
#include <atomic>
#include <mutex>

#include "kernels.hpp"
#include "linattn.h"

namespace la {

static __device__ __align__(256) unsigned char scratch[LINATTN_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::atomic<void*> g_addr[MAX_DEVICES];
std::mutex g_mu;
}  // namespace

void* noalloc_scratch() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return nullptr;
  void* p = g_addr[dev].load(std::memory_order_acquire);
  if (p) return p;
  std::lock_guard<std::mutex> lock(g_mu);
  p = g_addr[dev].load(std::memory_order_relaxed);
  if (!p) {
    // `dev` is the current device: the address is that device's copy.
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    g_addr[dev].store(p, std::memory_order_release);
  }
  return p;
}

}  // namespace la
