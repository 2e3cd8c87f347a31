// Static device scratch for the entry point that allocates nothing
// (attn_bwd_noalloc): the backward's workspace, held by the library on every
// device it runs on until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory, so it
// is never passed to a kernel or a copy: its device address is looked up once
// per device with hipGetSymbolAddress (the device current, as each device
// holds its own copy at its own address) and cached here.
#include <hip/hip_runtime.h>

#include <atomic>

#include "attn_launch.h"

namespace attn {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch_addr[kMaxDevices];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch_addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // Two threads may race here; both store the same address.
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_addr[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace attn
