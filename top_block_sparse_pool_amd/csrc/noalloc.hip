// Allocation-free variant of the sparse attention call: the persistent
// queue's control block (two dequeue counters) lives in a file-scope device
// array instead of a caller-provided workspace.
//
// Each GPU the library runs on holds its own copy of `scratch` until the
// process ends.  Host code never passes the array's name to a kernel (on the
// host it is only a stand-in for the symbol): the device address is looked up
// once per device with hipGetSymbolAddress, with that device current, and
// kept in g_scratch_ptr.  Every call on one GPU shares that GPU's array, so
// calls that overlap in time on one GPU (two streams without ordering) race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

namespace tbs {
namespace {

constexpr size_t kNoAllocScratchBytes = kCtrlBytes;   // the control block
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {nullptr};

__global__ __launch_bounds__(64) void clear_scratch_kernel(uint32_t* __restrict__ p, int n) {
  const int i = blockIdx.x * 64 + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

size_t noalloc_scratch_bytes() { return kNoAllocScratchBytes; }

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!ptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t noalloc_clear(void* ptr, size_t bytes, hipStream_t stream) {
  const int n = static_cast<int>(bytes / sizeof(uint32_t));
  hipLaunchKernelGGL(clear_scratch_kernel, dim3((n + 63) / 64), dim3(64), 0, stream, static_cast<uint32_t*>(ptr), n);
  return hipGetLastError();
}

}  // namespace tbs
