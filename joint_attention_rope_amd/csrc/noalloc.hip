// Scratch memory of klein_rope4d_attn_fwd_noalloc, the entry point for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// The scratch is one file-scope device array per GPU, `scratch`, of
// kNoallocScratchBytes.  It sits in a code object of its own: the runtime
// loads a code object (and allocates its globals) on the first use of
// something in it, so only a process that calls the no-allocation entry
// point holds this memory, once per GPU it calls it on, until it exits.
//
// In host code the name `scratch` is only a host-side stand-in for the
// array: its device address, which differs from GPU to GPU, comes from
// hipGetSymbolAddress with that GPU current, taken once per device and kept;
// only that address is ever handed to kernels.
#include <mutex>

#include "klein_launch.hpp"

namespace klein {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace klein
