// kda_noalloc.hip -- the per-GPU scratch buffer behind kda_chunk_fwd_no_alloc.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// serving loops, harnesses that forbid hipMalloc) get the prefill's workspace
// from a file-scope device array instead of an argument.  Each GPU the library
// runs on holds its own copy of the array, at its own address, until the
// process ends.  In host code the array's name is only a stand-in for the
// symbol: its device address is looked up once per device with
// hipGetSymbolAddress and kept, and only that address is ever handed to
// kernels.
#include <mutex>

#include "kda_internal.h"

namespace kda {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_addr[kMaxDevices];  // device address of `scratch` on each device, once looked up

}  // namespace

hipError_t no_alloc_scratch(void **addr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[dev] = p;
  }
  *addr = g_addr[dev];
  return hipSuccess;
}

}  // namespace kda
