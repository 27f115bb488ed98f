// kda_status.hip -- the per-GPU status word of failures that kernels detect on
// the device and cannot return through the host call that enqueued them.
//
// Kernels OR KDA_DEVICE_* bits into `status_word` with device-scope atomics.
// kda_device_status reads it in stream order: a one-thread kernel exchanges the
// word (with zero when clearing) into `status_snapshot`, and the host copies the
// snapshot back after the stream has drained.  Each GPU holds its own pair of
// words at its own address, looked up once per device with
// hipGetSymbolAddress; only those addresses are handed to kernels.
#include <atomic>
#include <mutex>

#include "kda_internal.h"

namespace kda {
namespace {

static __device__ __align__(16) uint32_t status_word[4];  // [0]: the word, [1]: the snapshot

constexpr int kMaxDevices = 64;
std::mutex g_mu;
uint32_t *g_addr[kMaxDevices];
std::atomic<int32_t> g_poll_limit{kDefaultHandoffPolls};

__global__ void status_exchange_kernel(uint32_t *words, uint32_t replace) {
  if (threadIdx.x == 0)
    words[1] = __hip_atomic_exchange(&words[0], replace, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace

hipError_t device_status_word(uint32_t **addr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(status_word));
    if (e != hipSuccess) return e;
    g_addr[dev] = static_cast<uint32_t *>(p);
  }
  *addr = g_addr[dev];
  return hipSuccess;
}

int32_t handoff_poll_limit() { return g_poll_limit.load(std::memory_order_relaxed); }
void set_handoff_poll_limit(int32_t polls) { g_poll_limit.store(polls, std::memory_order_relaxed); }

hipError_t read_device_status(hipStream_t stream, bool clear, uint32_t *bits) {
  uint32_t *words = nullptr;
  hipError_t e = device_status_word(&words);
  if (e != hipSuccess) return e;
  uint32_t cur = 0;
  if (clear) {
    hipLaunchKernelGGL(status_exchange_kernel, dim3(1), dim3(64), 0, stream, words, 0u);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = hipMemcpyAsync(&cur, words + 1, sizeof(cur), hipMemcpyDeviceToHost, stream);
  } else {
    e = hipMemcpyAsync(&cur, words, sizeof(cur), hipMemcpyDeviceToHost, stream);
  }
  if (e != hipSuccess) return e;
  e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return e;
  *bits = cur;
  return hipSuccess;
}

}  // namespace kda
