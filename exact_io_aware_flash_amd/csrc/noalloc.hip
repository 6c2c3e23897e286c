// Fixed device scratch for the allocation-free backward entry point (flash_attn_bwd_noalloc).
//
// The backward pass needs one buffer beyond its inputs and outputs: D = rowsum(dO * O), float32,
// one value per query row.  flash_attn_bwd takes it from the caller's workspace; callers that may
// not allocate device memory at all (code under stream capture, tight serving loops, harnesses
// that forbid it) use this file-scope array instead.  Each GPU the library runs on holds its own
// copy of the array, at its own address, until the process ends.
//
// In host code the name `scratch` is only a host-side stand-in: passing it to a kernel would
// compile and then fault.  Its device address is therefore looked up once per device with
// hipGetSymbolAddress (with that device current) and only that address is ever handed to kernels.
#include <mutex>

#include "fa_kernels.h"

namespace fa {

namespace {

static __device__ __align__(256) char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_lock);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace fa
