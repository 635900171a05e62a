// scratch.hip -- the fixed device array that gemm_tuned_noalloc uses as its
// workspace (GEMV slice counters, split-K partial sums, transposed operand
// copies), for callers that cannot allocate device memory.
//
// Each GPU the library runs on holds its own copy of the array (kScratchBytes)
// from the first allocation-free call on that GPU until the process ends.
// In host code the name `scratch` is only a host-side stand-in for the
// symbol: the device address of a GPU's copy comes from hipGetSymbolAddress,
// called once per device with that device current, and only that address is
// ever handed to kernels.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>

#include "launchers.h"

static __device__ __align__(256) unsigned char scratch[gt::kScratchBytes];

namespace gt {

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
std::atomic<void*> g_addr[kMaxDevices];
}  // namespace

int scratch_address(int device, hipStream_t stream, void** out) {
  *out = nullptr;
  if (device < 0 || device >= kMaxDevices) return LS_UNSUPPORTED;
  void* p = g_addr[device].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> g(g_mu);
    p = g_addr[device].load(std::memory_order_relaxed);
    if (!p) {
      void* q = nullptr;
      if (hipGetSymbolAddress(&q, HIP_SYMBOL(scratch)) != hipSuccess || !q) return LS_HIP_ERROR;
      // the counter region must start at zero (every launch that uses a
      // counter leaves it zero again); cleared by a kernel, not a memset, so
      // that a first call under stream capture records a kernel node
      if (launch_zero(q, 1, (int64_t)(kCounterRegion / 4), (int64_t)(kCounterRegion / 4), DT_F32, stream) != LS_OK)
        return LS_HIP_ERROR;
      g_addr[device].store(q, std::memory_order_release);
      p = q;
    }
  }
  *out = p;
  return LS_OK;
}

}  // namespace gt
